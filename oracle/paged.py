"""CPU oracle for attention over a paged KV cache with per-sequence key lengths (fp64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module. The GPU library never calls
it and shares no code with it; this module imports numpy and the plain
oracle only.

The pages name FlashAttention's paged KV cache as the way to serve
sequences of dynamic length, and to keep caches of sequences longer than
8192 tokens within memory (Stable-Diffusion GQA guide, application scenario
one and the troubleshooting checklist), without fixing a layout. Reading
taken here (the plainest one, listed in the design notes):

* The cache is a pool of fixed-size pages, ``[num_pages, page_size, Hk, d]``
  for keys and the same for values.
* ``block_table[b, p]`` is the pool page holding keys ``p*page_size`` to
  ``(p+1)*page_size - 1`` of sequence b, so key j of sequence b is row
  ``j % page_size`` of page ``block_table[b, j // page_size]``.
* Sequence b has ``seqlens_k[b]`` keys; table entries past its last page
  and page rows past its last key are never read. A sequence may have no
  key at all: every query row then has output 0 and log-sum-exp -inf.
* Queries are ``[B, Sq, Hq, d]`` as in the contiguous call, and the causal
  alignment is bottom-right per sequence: key j is visible to query i iff
  ``j <= i + seqlens_k[b] - Sq``.

The result for sequence b is exactly the contiguous attention of its
queries against its gathered keys and values.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from .attention import NEG_INF, attention_fp64


def gather_pages(cache, table_row, seqlen: int) -> np.ndarray:
    """Keys (or values) 0 .. seqlen-1 of one sequence: [seqlen, Hk, d] in key order."""
    cache = np.asarray(cache)
    page_size = cache.shape[1]
    rows = []
    for j in range(int(seqlen)):
        page = int(table_row[j // page_size])
        rows.append(cache[page, j % page_size])
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows)


def attention_paged_fp64(q, k_cache, v_cache, block_table, seqlens_k, causal: bool, scale: float,
                         batches: Optional[Iterable[int]] = None,
                         heads: Optional[Iterable[int]] = None,
                         rows: Optional[Sequence[int]] = None):
    """Exact GQA forward over a paged cache.

    q: [B, Sq, Hq, d]; k_cache, v_cache: [num_pages, page_size, Hk, d];
    block_table: [B, max_pages] ints; seqlens_k: [B] ints.
    Returns O [nb, nr, nh, d] and LSE [nb, nh, nr] for the selected batches,
    heads and query rows (all by default), as attention_fp64 does.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Sq, Hq, d = q.shape
    Hk = np.asarray(k_cache).shape[2]
    bs = list(range(B)) if batches is None else list(batches)
    hs = list(range(Hq)) if heads is None else list(heads)
    rs = list(range(Sq)) if rows is None else list(rows)
    O = np.zeros((len(bs), len(rs), len(hs), d))
    LSE = np.full((len(bs), len(hs), len(rs)), NEG_INF)
    for ib, b in enumerate(bs):
        n = int(seqlens_k[b])
        kb = gather_pages(k_cache, block_table[b], n).astype(np.float64)
        vb = gather_pages(v_cache, block_table[b], n).astype(np.float64)
        if n == 0:
            kb = np.zeros((0, Hk, d))
            vb = np.zeros((0, Hk, d))
        Ob, Lb = attention_fp64(q[b:b + 1], kb[None], vb[None], causal, scale, heads=hs, rows=rs)
        O[ib] = Ob[0]
        LSE[ib] = Lb[0]
    return O, LSE
