"""Pins of the paged-cache oracle to facts other than itself (CPU only).

* gather: the keys drawn for a sequence (batch_slice's tensors 1 and 2) come
  back from the pool in key order, for several page sizes, empty and
  one-key sequences;
* brute force: scalar loops that look every key up in the pool directly
  (page = table[j // page_size], row = j % page_size) with math.fsum and
  math.exp, per-sequence bottom-right causal alignment;
* per-sequence lengths: sequence b gives the contiguous oracle's result on
  its own first seqlens_k[b] keys (the contiguous oracle is pinned in
  test_oracle_pins.py);
* closed forms: an empty sequence gives O = 0 and LSE = -inf; with causal
  and Sq > n the first Sq - n tokens see no key;
* invariants: different garbage in unused pages, unused page rows and unused
  table entries changes nothing.
Planted mistakes (row and page index swapped, one length for every sequence,
top-left causal alignment) must each fail a pin.
"""

import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import oracle
from oracle import paged as opg


def f64(t):
    return t.to(torch.float64).numpy()


def brute_force_paged(q, kc, vc, table, lens, causal, scale):
    B, Sq, Hq, d = q.shape
    ps, Hk = kc.shape[1], kc.shape[2]
    G = Hq // Hk
    O = np.zeros((B, Sq, Hq, d))
    L = np.full((B, Hq, Sq), -math.inf)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            g = h // G
            for i in range(Sq):
                scores = []
                for j in range(n):
                    if causal and j > i + n - Sq:
                        continue
                    page, row = int(table[b][j // ps]), j % ps
                    dot = math.fsum(float(q[b, i, h, c]) * float(kc[page, row, g, c]) for c in range(d))
                    scores.append((page, row, scale * dot))
                if not scores:
                    continue
                mx = max(s for _, _, s in scores)
                w = [(pg, r, math.exp(s - mx)) for pg, r, s in scores]
                tot = math.fsum(x for _, _, x in w)
                L[b, h, i] = mx + math.log(tot)
                for c in range(d):
                    O[b, i, h, c] = math.fsum(x * float(vc[pg, r, g, c]) for pg, r, x in w) / tot
    return O, L


CASES = [
    # seed, seqlens, page_size, Sq, Hq, Hk, d
    (1, [5, 0, 40, 17], 16, 1, 4, 2, 4),
    (2, [33, 1, 32], 16, 3, 6, 2, 3),
    (3, [64, 63, 65], 32, 2, 2, 1, 5),
    (4, [7, 100], 48, 4, 8, 2, 2),
]


def pin_gather(gather):
    for seed, lens, ps, Sq, Hq, Hk, d in CASES:
        kv = gi.paged_kv(seed, lens, ps, Hk, d)
        for b, n in enumerate(lens):
            _, kb, vb = gi.batch_slice(seed, b, 1, n, Hq, Hk, d)
            got_k = np.asarray(gather(f64(kv.k_cache), kv.block_table[b].tolist(), n))
            got_v = np.asarray(gather(f64(kv.v_cache), kv.block_table[b].tolist(), n))
            assert got_k.shape == (n, Hk, d) and got_v.shape == (n, Hk, d)
            assert np.array_equal(got_k, f64(kb)) and np.array_equal(got_v, f64(vb))


def pin_brute_force(attn):
    for seed, lens, ps, Sq, Hq, Hk, d in CASES:
        kv = gi.paged_kv(seed, lens, ps, Hk, d)
        q = f64(gi.random_bf16(seed + 100, (len(lens), Sq, Hq, d)))
        table = kv.block_table.tolist()
        for causal in (False, True):
            Ob, Lb = brute_force_paged(q, f64(kv.k_cache), f64(kv.v_cache), table, lens, causal, 0.41)
            O, L = attn(q, f64(kv.k_cache), f64(kv.v_cache), kv.block_table.numpy(), kv.seqlens_k.numpy(), causal, 0.41)
            assert np.allclose(O, Ob, rtol=0, atol=1e-12), (seed, causal)
            fin = np.isfinite(Lb)
            assert np.array_equal(fin, np.isfinite(L)), (seed, causal)
            assert np.allclose(L[fin], Lb[fin], rtol=0, atol=1e-12), (seed, causal)


def pin_per_sequence_lengths(attn):
    seed, lens, ps, Sq, Hq, Hk, d = 5, [9, 30, 1], 16, 2, 4, 2, 8
    kv = gi.paged_kv(seed, lens, ps, Hk, d)
    q = f64(gi.random_bf16(seed + 100, (len(lens), Sq, Hq, d)))
    for causal in (False, True):
        O, L = attn(q, f64(kv.k_cache), f64(kv.v_cache), kv.block_table.numpy(), kv.seqlens_k.numpy(), causal, 0.3)
        for b, n in enumerate(lens):
            _, kb, vb = gi.batch_slice(seed, b, 1, n, Hq, Hk, d)
            Oc, Lc = oracle.attention_fp64(q[b:b + 1], f64(kb)[None], f64(vb)[None], causal, 0.3)
            assert np.allclose(O[b], Oc[0], rtol=0, atol=1e-13), (b, causal)
            assert np.allclose(L[b], Lc[0], rtol=0, atol=1e-13), (b, causal)


def pin_closed_forms(attn):
    seed, lens, ps, Hq, Hk, d = 6, [0, 3], 16, 4, 2, 4
    kv = gi.paged_kv(seed, lens, ps, Hk, d)
    Sq = 5
    q = f64(gi.random_bf16(seed + 100, (2, Sq, Hq, d)))
    for causal in (False, True):
        O, L = attn(q, f64(kv.k_cache), f64(kv.v_cache), kv.block_table.numpy(), kv.seqlens_k.numpy(), causal, 0.5)
        assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
        if causal:   # 3 keys, 5 queries: tokens 0 and 1 see nothing, token 2 sees key 0 only
            assert np.all(O[1, :2] == 0) and np.all(np.isneginf(L[1, :, :2]))
            _, kb, vb = gi.batch_slice(seed, 1, 1, 3, Hq, Hk, d)
            for h in range(Hq):
                assert np.allclose(O[1, 2, h], f64(vb)[0, h // 2], atol=1e-12)
        else:
            assert np.all(np.isfinite(L[1]))


def pin_garbage_is_never_read(attn):
    seed, lens, ps, Sq, Hq, Hk, d = 7, [20, 5, 33], 16, 2, 6, 3, 4
    a = gi.paged_kv(seed, lens, ps, Hk, d, spare_pages=3, max_pages=6, fill=float("nan"))
    b = gi.paged_kv(seed, lens, ps, Hk, d, spare_pages=3, max_pages=6, fill=1e4)
    tb = b.block_table.clone()
    tb[tb < 0] = 10 ** 6                      # another kind of unused entry
    q = f64(gi.random_bf16(seed + 100, (len(lens), Sq, Hq, d)))
    for causal in (False, True):
        Oa, La = attn(q, f64(a.k_cache), f64(a.v_cache), a.block_table.numpy(), a.seqlens_k.numpy(), causal, 0.5)
        Ob, Lb = attn(q, f64(b.k_cache), f64(b.v_cache), tb.numpy(), b.seqlens_k.numpy(), causal, 0.5)
        assert np.all(np.isfinite(Oa)) and np.array_equal(Oa, Ob) and np.array_equal(La, Lb)


PINS = [pin_brute_force, pin_per_sequence_lengths, pin_closed_forms, pin_garbage_is_never_read]


def test_gather_pin():
    pin_gather(opg.gather_pages)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_paged_oracle_pins(pin):
    pin(oracle.attention_paged_fp64)


def _fails(attn=None, gather=None):
    try:
        if gather is not None:
            pin_gather(gather)
        for pin in PINS:
            pin(attn or oracle.attention_paged_fp64)
    except AssertionError:
        return True
    return False


def test_planted_row_and_page_swapped():
    def bad_gather(cache, table_row, n):
        cache = np.asarray(cache)
        ps = cache.shape[1]
        rows = [cache[int(table_row[j % ps]) if j % ps < len(table_row) else 0, j // ps] for j in range(n)]
        return np.stack(rows) if rows else np.zeros((0,) + cache.shape[2:])
    assert _fails(gather=bad_gather)


def test_planted_one_length_for_all(monkeypatch):
    real = opg.attention_paged_fp64

    def bad(q, kc, vc, table, lens, causal, scale, **kw):
        lens = np.full_like(np.asarray(lens), int(np.max(lens)))
        return real(q, kc, vc, table, lens, causal, scale, **kw)
    assert _fails(attn=bad)


def test_planted_top_left_causal(monkeypatch):
    from oracle import attention as oatt

    def vis(i, Sq, Sk, causal):
        j = np.arange(Sk)[None, :]
        if not causal:
            return np.ones((len(i), Sk), dtype=bool)
        return j <= np.asarray(i)[:, None]
    monkeypatch.setattr(oatt, "visible_keys", vis)
    assert _fails()
