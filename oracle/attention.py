"""CPU oracle for the exact grouped-query attention forward pass (fp64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module. The GPU library never
calls it and shares no code with it; this module imports numpy only.

What it computes (plain definition, no tiling, no online softmax):

* Scaled dot-product attention ``softmax(Q K^T * scale) V`` per query row
  (PyTorch profiling guide part 3, "the computational challenge of
  attention" formula; Llama-2 GQA article, section 1.2).
* Grouped heads: Hq query heads share Hk key/value heads, Hq must be a
  multiple of Hk, and query head h reads key/value head h // (Hq/Hk), so
  with Hq=6, Hk=2 heads 0-2 read head 0 and heads 3-5 read head 1
  (batch-sensitivity article, "core design of grouped-query attention";
  rise-and-fall tuning article, "root cause"). The heads of one group are
  consecutive, as in the article's ``view(batch, seq, num_groups,
  group_size, head_dim)`` reshape (Llama-2 GQA article, section 1.2).
* Optional causal mask (``causal=True`` in every tuning snippet of the
  Stable-Diffusion GQA guide, "dynamic batch scheduling").

Readings where the pages are silent (each listed in the design notes):

* Causal alignment when Sq != Sk is bottom-right: key j is visible to query i
  iff j <= i + Sk - Sq. At Sq == Sk this is the usual j <= i.
* A row with no visible key (only possible when causal and Sq > Sk) has
  output 0 and log-sum-exp -inf.
* The log-sum-exp is natural-log of the sum of exp of the *scaled* scores,
  laid out [B, Hq, Sq].
* ``scale`` is whatever value the caller passes (the default 1/sqrt(d) of the
  Stable-Diffusion GQA guide's code is the caller's choice); the oracle uses
  it exactly as given.

Split-KV ("split + combine", rise-and-fall tuning article, "fix" table):
``split_combine_fp64`` computes, for each key range, the partial result
normalised within that range together with its log-sum-exp, and merges the
partials with weights exp(LSE_s - LSE). The merge is an identity of real
arithmetic, so its result equals ``attention_fp64``; the tests pin that.
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def kv_head_of(h: int, Hq: int, Hk: int) -> int:
    """Key/value head read by query head h: h // (Hq/Hk)."""
    if Hq % Hk != 0:
        raise ValueError("the number of query heads must be a multiple of the number of KV heads")
    return h // (Hq // Hk)


def visible_keys(i: np.ndarray, Sq: int, Sk: int, causal: bool) -> np.ndarray:
    """Boolean [len(i), Sk] matrix: key j visible to query row i."""
    j = np.arange(Sk)[None, :]
    if not causal:
        return np.ones((len(i), Sk), dtype=bool)
    return j <= (np.asarray(i)[:, None] + (Sk - Sq))


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _row_softmax(S: np.ndarray, vis: np.ndarray):
    """Masked rows of scores -> (P, LSE, m). Rows with no visible key give P=0, LSE=-inf."""
    S = np.where(vis, S, NEG_INF)
    m = S.max(axis=1) if S.shape[1] > 0 else np.full(S.shape[0], NEG_INF)
    live = np.isfinite(m)
    lse = np.full(S.shape[0], NEG_INF)
    P = np.zeros_like(S)
    if live.any():
        Sl = S[live]
        ml = m[live]
        ssum = np.exp(Sl - ml[:, None]).sum(axis=1)
        lse[live] = ml + np.log(ssum)
        P[live] = np.exp(Sl - lse[live][:, None])
    return P, lse, m


def attention_fp64(q, k, v, causal: bool, scale: float,
                   batches: Optional[Iterable[int]] = None,
                   heads: Optional[Iterable[int]] = None,
                   rows: Optional[Sequence[int]] = None,
                   return_p: bool = False):
    """Exact GQA forward in fp64.

    q: [B, Sq, Hq, d]; k, v: [B, Sk, Hk, d] (any real dtype, upcast exactly).
    Returns O [nb, nr, nh, d] and LSE [nb, nh, nr] for the selected batches,
    heads and query rows (all by default), plus P [nb, nh, nr, Sk] if asked.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Sq, Hq, d = q.shape
    Bk, Sk, Hk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    kv_head_of(0, Hq, Hk)  # divisibility check
    bs = list(range(B)) if batches is None else list(batches)
    hs = list(range(Hq)) if heads is None else list(heads)
    rs = np.arange(Sq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    scale = float(scale)

    O = np.zeros((len(bs), len(rs), len(hs), d))
    LSE = np.full((len(bs), len(hs), len(rs)), NEG_INF)
    P_all = np.zeros((len(bs), len(hs), len(rs), Sk)) if return_p else None
    vis = visible_keys(rs, Sq, Sk, causal)
    for ib, b in enumerate(bs):
        for ih, h in enumerate(hs):
            g = kv_head_of(h, Hq, Hk)
            Qr = q[b, rs, h, :]           # [R, d]
            Kg = k[b, :, g, :]            # [Sk, d]
            Vg = v[b, :, g, :]            # [Sk, d]
            S = scale * (Qr @ Kg.T)       # [R, Sk]
            P, lse, _ = _row_softmax(S, vis)
            O[ib, :, ih, :] = P @ Vg
            LSE[ib, ih, :] = lse
            if return_p:
                P_all[ib, ih] = P
    if return_p:
        return O, LSE, P_all
    return O, LSE


def split_tiles(Sk: int, block_n: int, num_splits: int) -> List[Tuple[int, int]]:
    """Key ranges of a balanced split of ceil(Sk/block_n) key tiles into num_splits parts.

    Split s owns tiles [floor(s*T/ns), floor((s+1)*T/ns)); a split may be empty.
    """
    T = -(-Sk // block_n)
    out = []
    for s in range(num_splits):
        t0 = (s * T) // num_splits
        t1 = ((s + 1) * T) // num_splits
        out.append((min(t0 * block_n, Sk), min(t1 * block_n, Sk)))
    return out


def split_partials_fp64(q, k, v, causal: bool, scale: float,
                        key_ranges: Sequence[Tuple[int, int]],
                        batches=None, heads=None, rows=None):
    """Per-split partials: O_s [ns, nb, nr, nh, d] normalised within the split, LSE_s [ns, nb, nh, nr].

    A split with no visible key gets O_s = 0 and LSE_s = -inf.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Sq, Hq, d = q.shape
    Sk = k.shape[1]
    Hk = k.shape[2]
    kv_head_of(0, Hq, Hk)
    bs = list(range(B)) if batches is None else list(batches)
    hs = list(range(Hq)) if heads is None else list(heads)
    rs = np.arange(Sq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    scale = float(scale)
    ns = len(key_ranges)
    Os = np.zeros((ns, len(bs), len(rs), len(hs), d))
    Ls = np.full((ns, len(bs), len(hs), len(rs)), NEG_INF)
    vis_all = visible_keys(rs, Sq, Sk, causal)
    for s, (j0, j1) in enumerate(key_ranges):
        in_split = np.zeros(Sk, dtype=bool)
        in_split[j0:j1] = True
        vis = vis_all & in_split[None, :]
        for ib, b in enumerate(bs):
            for ih, h in enumerate(hs):
                g = kv_head_of(h, Hq, Hk)
                S = scale * (q[b, rs, h, :] @ k[b, :, g, :].T)
                P, lse, _ = _row_softmax(S, vis)
                Os[s, ib, :, ih, :] = P @ v[b, :, g, :]
                Ls[s, ib, ih, :] = lse
    return Os, Ls


def combine_fp64(Os: np.ndarray, Ls: np.ndarray):
    """LSE-weighted merge of split partials.

    Os [ns, nb, nr, nh, d], Ls [ns, nb, nh, nr] ->
    LSE = M + ln sum_s exp(LSE_s - M) with M = max_s LSE_s, O = sum_s exp(LSE_s - LSE) O_s.
    If every split is empty the row gets O = 0 and LSE = -inf.
    """
    M = Ls.max(axis=0)                                   # [nb, nh, nr]
    live = np.isfinite(M)
    Msafe = np.where(live, M, 0.0)
    w_un = np.where(np.isfinite(Ls), np.exp(Ls - Msafe[None]), 0.0)   # [ns, nb, nh, nr]
    tot = w_un.sum(axis=0)
    LSE = np.where(live, Msafe + np.log(np.where(live, tot, 1.0)), NEG_INF)
    w = np.where(live[None], w_un / np.where(live, tot, 1.0)[None], 0.0)   # [ns, nb, nh, nr]
    # weights to [ns, nb, nr, nh, 1] to match O's layout
    wO = np.transpose(w, (0, 1, 3, 2))[..., None]
    O = (wO * Os).sum(axis=0)
    return O, LSE


def split_combine_fp64(q, k, v, causal: bool, scale: float,
                       key_ranges: Sequence[Tuple[int, int]], **sel):
    """Attention computed split by split over key_ranges, then merged (see combine_fp64)."""
    Os, Ls = split_partials_fp64(q, k, v, causal, scale, key_ranges, **sel)
    return combine_fp64(Os, Ls)
