"""Pins of the CPU oracle to facts other than itself (CPU only).

Each pin is a function taking the attention function under test, so the same
pins also run against deliberately broken copies of the oracle (planted
mistakes below) and must catch every one of them.

Pins used (none of them retypes the oracle's vectorised formula):
* brute force: scalar Python loops with math.fsum / math.exp on tiny inputs,
  heads enumerated group by group, softmax normalised by its own sum;
* the MHA identity: GQA equals multi-head attention with each KV head
  repeated Hq/Hk times in place (repeat_interleave), and a library routine,
  torch's fp64 CPU scaled_dot_product_attention with enable_gqa;
* the printed head-map example Hq=6, Hk=2 (tests/golden/head_map_hq6_hk2.txt);
* closed forms: Q = 0 gives the mean of the visible values and LSE = ln(count);
  causal row 0 gives V[0] and LSE = scale * q0.k0; one key gives V[0];
* invariants: softmax rows sum to one, max <= LSE <= max + ln(count),
  key shift and key permutation behaviour, independent (b, head) slices;
* split + combine: equal to the one-pass result for any partition.
"""

import math
import os
import random

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as oatt

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(shape, seed, std=1.0):
    rs = np.random.RandomState(seed)
    return rs.standard_normal(shape) * std


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, causal, scale):
    """Scalar loops. Query head h of group g is h = g*G + t (t < G)."""
    B, Sq, Hq, d = q.shape
    Sk, Hk = k.shape[1], k.shape[2]
    G = Hq // Hk
    O = np.zeros((B, Sq, Hq, d))
    L = np.full((B, Hq, Sq), -math.inf)
    for b in range(B):
        for g in range(Hk):
            for t in range(G):
                h = g * G + t
                for i in range(Sq):
                    scores = []
                    for j in range(Sk):
                        if causal and j - i > Sk - Sq:
                            continue
                        dot = math.fsum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(d))
                        scores.append((j, scale * dot))
                    if not scores:
                        continue
                    mx = max(s for _, s in scores)
                    w = [(j, math.exp(s - mx)) for j, s in scores]
                    tot = math.fsum(x for _, x in w)
                    L[b, h, i] = mx + math.log(tot)
                    for c in range(d):
                        O[b, i, h, c] = math.fsum(x * float(v[b, j, g, c]) for j, x in w) / tot
    return O, L


TINY_SHAPES = [
    # B, Sq, Sk, Hq, Hk, d
    (1, 5, 5, 1, 1, 4),
    (2, 4, 7, 2, 1, 3),
    (1, 6, 6, 3, 1, 8),
    (1, 7, 5, 4, 2, 5),
    (2, 3, 9, 6, 2, 4),
    (1, 9, 4, 6, 3, 2),
    (1, 8, 8, 4, 4, 6),
    (1, 1, 9, 6, 2, 8),
]


def pin_brute_force(attn):
    for n, (B, Sq, Sk, Hq, Hk, d) in enumerate(TINY_SHAPES):
        q = rnd((B, Sq, Hq, d), 10 + n)
        k = rnd((B, Sk, Hk, d), 20 + n)
        v = rnd((B, Sk, Hk, d), 30 + n)
        for causal in (False, True):
            scale = 0.37
            Ob, Lb = brute_force(q, k, v, causal, scale)
            O, L = attn(q, k, v, causal, scale)
            assert np.allclose(O, Ob, rtol=0, atol=1e-12), (n, causal)
            fin = np.isfinite(Lb)
            assert np.array_equal(fin, np.isfinite(L)), (n, causal)
            assert np.allclose(L[fin], Lb[fin], rtol=0, atol=1e-12), (n, causal)


# ------------------------------------------------------------- MHA identity

def pin_mha_identity(attn):
    B, Sq, Sk, Hk, d = 2, 11, 13, 2, 8
    for G in (1, 2, 3, 4):
        Hq = G * Hk
        q = rnd((B, Sq, Hq, d), 100 + G)
        k = rnd((B, Sk, Hk, d), 200 + G)
        v = rnd((B, Sk, Hk, d), 300 + G)
        kr = np.repeat(k, G, axis=2)    # KV head g repeated in place: heads gG..gG+G-1
        vr = np.repeat(v, G, axis=2)
        for causal in (False, True):
            O, L = attn(q, k, v, causal, 0.5)
            Om, Lm = attn(q, kr, vr, causal, 0.5)   # Hq == Hk: plain MHA
            assert np.allclose(O, Om, rtol=0, atol=1e-12)
            assert np.allclose(L, Lm, rtol=0, atol=1e-12)


def pin_sdpa_library(attn):
    """torch fp64 CPU scaled_dot_product_attention with enable_gqa, bottom-right causal mask."""
    cases = [(2, 9, 9, 6, 2, 16), (1, 12, 17, 8, 2, 8), (1, 1, 33, 4, 1, 32), (2, 16, 16, 4, 4, 8)]
    for n, (B, Sq, Sk, Hq, Hk, d) in enumerate(cases):
        q = rnd((B, Sq, Hq, d), 400 + n)
        k = rnd((B, Sk, Hk, d), 500 + n)
        v = rnd((B, Sk, Hk, d), 600 + n)
        for causal in (False, True):
            scale = 1.0 / math.sqrt(d)
            tq = torch.from_numpy(q).permute(0, 2, 1, 3)
            tk = torch.from_numpy(k).permute(0, 2, 1, 3)
            tv = torch.from_numpy(v).permute(0, 2, 1, 3)
            mask = None
            if causal:
                i = torch.arange(Sq)[:, None]
                j = torch.arange(Sk)[None, :]
                mask = j <= i + (Sk - Sq)
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                                 enable_gqa=True).permute(0, 2, 1, 3).numpy()
            O, _ = attn(q, k, v, causal, scale)
            assert np.allclose(O, ref, rtol=0, atol=1e-10), (n, causal)


def test_repeat_tile_is_not_the_head_map():
    """Tiling the KV heads (kv0, kv1, kv0, kv1, ...) is a different, wrong model for Hk=2, G=3."""
    B, Sq, Sk, Hq, Hk, d = 1, 5, 6, 6, 2, 4
    q, k, v = rnd((B, Sq, Hq, d), 1), rnd((B, Sk, Hk, d), 2), rnd((B, Sk, Hk, d), 3)
    O, _ = oracle.attention_fp64(q, k, v, False, 0.5)
    Ot, _ = oracle.attention_fp64(q, np.tile(k, (1, 1, 3, 1)), np.tile(v, (1, 1, 3, 1)), False, 0.5)
    assert not np.allclose(O, Ot, atol=1e-3)


# -------------------------------------------------------------- head map

def load_head_map():
    pairs = []
    with open(os.path.join(HERE, "golden", "head_map_hq6_hk2.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                pairs.append((int(a), int(b)))
    return pairs


def test_head_map_golden():
    pairs = load_head_map()
    assert len(pairs) == 6
    for h, g in pairs:
        assert oracle.kv_head_of(h, 6, 2) == g


def test_head_map_rejects_indivisible():
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


def pin_structured_head_map(attn):
    """V[b, j, g, :] = g + 1 for every key: O[b, i, h, :] must equal map(h) + 1 exactly."""
    pairs = load_head_map()
    B, Sq, Sk, Hq, Hk, d = 2, 7, 9, 6, 2, 4
    q, k = rnd((B, Sq, Hq, d), 7), rnd((B, Sk, Hk, d), 8)
    v = np.zeros((B, Sk, Hk, d))
    for g in range(Hk):
        v[:, :, g, :] = g + 1
    for causal in (False, True):
        O, _ = attn(q, k, v, causal, 0.5)
        for h, g in pairs:
            assert np.allclose(O[:, :, h, :], g + 1, rtol=0, atol=1e-12), (h, g)


# -------------------------------------------------------------- closed forms

def pin_closed_forms(attn):
    B, Sq, Sk, Hq, Hk, d = 1, 6, 6, 4, 2, 5
    k, v = rnd((B, Sk, Hk, d), 41), rnd((B, Sk, Hk, d), 42)
    G = Hq // Hk
    # Q = 0: uniform weights over the visible keys
    q0 = np.zeros((B, Sq, Hq, d))
    O, L = attn(q0, k, v, False, 0.3)
    for h in range(Hq):
        assert np.allclose(O[0, :, h, :], v[0, :, h // G, :].mean(axis=0)[None], atol=1e-12)
    assert np.allclose(L, math.log(Sk), atol=1e-12)
    O, L = attn(q0, k, v, True, 0.3)
    for i in range(Sq):
        for h in range(Hq):
            assert np.allclose(O[0, i, h], v[0, :i + 1, h // G].mean(axis=0), atol=1e-12)
            assert abs(L[0, h, i] - math.log(i + 1)) < 1e-12
    # scale = 0 behaves like Q = 0
    q = rnd((B, Sq, Hq, d), 43)
    O, L = attn(q, k, v, False, 0.0)
    assert np.allclose(L, math.log(Sk), atol=1e-12)
    # causal row 0 sees only key 0
    O, L = attn(q, k, v, True, 0.3)
    for h in range(Hq):
        g = h // G
        assert np.allclose(O[0, 0, h], v[0, 0, g], atol=1e-12)
        assert abs(L[0, h, 0] - 0.3 * float(q[0, 0, h] @ k[0, 0, g])) < 1e-12
    # one key: output is that value row, LSE is its score
    O, L = attn(q, k[:, :1], v[:, :1], False, 0.3)
    for h in range(Hq):
        assert np.allclose(O[0, :, h], v[0, 0, h // G][None], atol=1e-12)
    # causal with a single query row (decode): bottom-right alignment sees every key
    O1, L1 = attn(q[:, :1], k, v, True, 0.3)
    O2, L2 = attn(q[:, :1], k, v, False, 0.3)
    assert np.allclose(O1, O2, atol=1e-15) and np.allclose(L1, L2, atol=1e-15)


def test_fully_masked_rows():
    """Causal with Sq > Sk: the first Sq - Sk rows see no key -> O = 0, LSE = -inf."""
    B, Sq, Sk, Hq, Hk, d = 1, 7, 3, 2, 1, 4
    q, k, v = rnd((B, Sq, Hq, d), 1), rnd((B, Sk, Hk, d), 2), rnd((B, Sk, Hk, d), 3)
    O, L = oracle.attention_fp64(q, k, v, True, 0.5)
    assert np.all(O[0, :Sq - Sk] == 0)
    assert np.all(np.isneginf(L[0, :, :Sq - Sk]))
    assert np.all(np.isfinite(L[0, :, Sq - Sk:]))
    # row Sq-Sk sees exactly key 0
    assert np.allclose(O[0, Sq - Sk, 0], v[0, 0, 0], atol=1e-12)


# ---------------------------------------------------------------- invariants

def pin_invariants(attn):
    B, Sq, Sk, Hq, Hk, d = 2, 8, 10, 6, 3, 6
    q, k, v = rnd((B, Sq, Hq, d), 51), rnd((B, Sk, Hk, d), 52), rnd((B, Sk, Hk, d), 53)
    scale = 0.45
    for causal in (False, True):
        O, L, P = attn(q, k, v, causal, scale, return_p=True)
        assert np.allclose(P.sum(axis=-1), 1.0, atol=1e-12)
        vis = oracle.visible_keys(np.arange(Sq), Sq, Sk, causal)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hk)
                S = scale * (q[b, :, h] @ k[b, :, g].T)
                S = np.where(vis, S, -np.inf)
                m = S.max(axis=1)
                n = vis.sum(axis=1)
                assert np.all(m <= L[b, h] + 1e-12)
                assert np.all(L[b, h] <= m + np.log(n) + 1e-12)
                assert np.all(P[b, h][~vis] == 0)
        # shift every key by u: O unchanged, LSE_i moves by scale * q_i . u
        u = rnd((d,), 54)
        O2, L2 = attn(q, k + u, v, causal, scale)
        assert np.allclose(O2, O, atol=1e-11)
        shift = scale * np.einsum("bihc,c->bhi", q, u)
        assert np.allclose(L2, L + shift, atol=1e-11)
        # batches and heads computed alone agree with the full call
        Ob, Lb = attn(q, k, v, causal, scale, batches=[1], heads=[4])
        assert np.allclose(Ob[0, :, 0], O[1, :, 4], atol=1e-14)
        assert np.allclose(Lb[0, 0], L[1, 4], atol=1e-14)
    # non-causal: permuting the keys (and values alike) changes nothing
    perm = np.random.RandomState(55).permutation(Sk)
    O, L = attn(q, k, v, False, scale)
    O2, L2 = attn(q, k[:, perm], v[:, perm], False, scale)
    assert np.allclose(O2, O, atol=1e-12) and np.allclose(L2, L, atol=1e-12)


# ----------------------------------------------------------- split + combine

def pin_split_combine(attn, split_combine=None):
    split_combine = split_combine or oracle.split_combine_fp64
    B, Sq, Sk, Hq, Hk, d = 2, 9, 23, 4, 2, 5
    q, k, v = rnd((B, Sq, Hq, d), 61), rnd((B, Sk, Hk, d), 62), rnd((B, Sk, Hk, d), 63)
    scale = 0.4
    rs = random.Random(64)
    for causal in (False, True):
        Oref, Lref = attn(q, k, v, causal, scale)
        for ns in (1, 2, 3, 4, 8):
            partitions = [oracle.split_tiles(Sk, 4, ns)]
            cuts = sorted(rs.randint(0, Sk) for _ in range(ns - 1))
            bounds = [0] + cuts + [Sk]
            partitions.append([(bounds[s], bounds[s + 1]) for s in range(ns)])
            for part in partitions:
                O, L = split_combine(q, k, v, causal, scale, part)
                assert np.allclose(O, Oref, atol=1e-12), (causal, ns, part)
                assert np.allclose(L, Lref, atol=1e-12), (causal, ns, part)
    # causal with Sq > Sk: fully masked rows stay 0 / -inf through the combine
    q2 = rnd((1, 12, 4, 3), 65)
    k2, v2 = rnd((1, 5, 2, 3), 66), rnd((1, 5, 2, 3), 67)
    O, L = split_combine(q2, k2, v2, True, scale, [(0, 2), (2, 2), (2, 5)])
    Oref, Lref = attn(q2, k2, v2, True, scale)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lref))
    assert np.allclose(O, Oref, atol=1e-12)


def test_split_tiles_partition():
    for Sk in (1, 63, 64, 65, 77, 128, 8192):
        for bn in (32, 64, 128):
            T = -(-Sk // bn)
            for ns in (1, 2, 3, 4, 8, 16):
                r = oracle.split_tiles(Sk, bn, ns)
                assert len(r) == ns and r[0][0] == 0 and r[-1][1] == Sk
                for (a, b), (c, _) in zip(r, r[1:]):
                    assert b == c and a <= b
                sizes = [-(-(b - a) // bn) for a, b in r]
                assert max(sizes) - min(sizes) <= 1 + (1 if ns > T else 0)


# -------------------------------------------------------- pins on the oracle

PINS = [pin_brute_force, pin_mha_identity, pin_sdpa_library, pin_structured_head_map,
        pin_closed_forms, pin_invariants, pin_split_combine]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    pin(oracle.attention_fp64)


# --------------------------------------------- planted mistakes must be caught

def _fails_some_pin(attn, split_combine=None):
    for pin in PINS:
        try:
            if pin is pin_split_combine and split_combine is not None:
                pin(attn, split_combine)
            else:
                pin(attn)
        except AssertionError:
            return True
    return False


def test_planted_wrong_head_map(monkeypatch):
    monkeypatch.setattr(oatt, "kv_head_of", lambda h, Hq, Hk: h % Hk)
    assert _fails_some_pin(oatt.attention_fp64)


def test_planted_dropped_scale():
    assert _fails_some_pin(lambda q, k, v, c, s, **kw: oatt.attention_fp64(q, k, v, c, 1.0, **kw))


def test_planted_keys_as_values():
    assert _fails_some_pin(lambda q, k, v, c, s, **kw: oatt.attention_fp64(q, k, k, c, s, **kw))


def test_planted_causal_off_by_one(monkeypatch):
    def vis(i, Sq, Sk, causal):
        j = np.arange(Sk)[None, :]
        if not causal:
            return np.ones((len(i), Sk), dtype=bool)
        return j < (np.asarray(i)[:, None] + (Sk - Sq))
    monkeypatch.setattr(oatt, "visible_keys", vis)
    assert _fails_some_pin(oatt.attention_fp64)


def test_planted_top_left_causal(monkeypatch):
    def vis(i, Sq, Sk, causal):
        j = np.arange(Sk)[None, :]
        if not causal:
            return np.ones((len(i), Sk), dtype=bool)
        return j <= np.asarray(i)[:, None]
    monkeypatch.setattr(oatt, "visible_keys", vis)
    assert _fails_some_pin(oatt.attention_fp64)


def test_planted_log2_lse(monkeypatch):
    real = oatt._row_softmax

    def bad(S, vis):
        P, lse, m = real(S, vis)
        return P, np.where(np.isfinite(lse), m + (lse - m) / math.log(2), lse), m
    monkeypatch.setattr(oatt, "_row_softmax", bad)
    assert _fails_some_pin(oatt.attention_fp64)


def test_planted_unnormalised_combine():
    def bad_combine(q, k, v, causal, scale, parts, **sel):
        Os, Ls = oatt.split_partials_fp64(q, k, v, causal, scale, parts, **sel)
        M = Ls.max(axis=0)
        w = np.where(np.isfinite(Ls), np.exp(Ls - np.where(np.isfinite(M), M, 0)[None]), 0.0)
        O = (np.transpose(w, (0, 1, 3, 2))[..., None] * Os).sum(axis=0)   # weights not divided by their sum
        return O, M
    assert _fails_some_pin(oatt.attention_fp64, bad_combine)
