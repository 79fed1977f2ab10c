"""Pins of the variable-length oracle (CPU only).

* equal lengths: the packed layout gives the batched oracle's result
  (reshaped), causal and not;
* brute force: scalar loops over each sequence's own tokens with math.fsum /
  math.exp and the per-sequence bottom-right causal alignment;
* closed forms: a sequence without keys gives O = 0 and LSE = -inf, one
  without queries changes nothing; a sequence computed alone equals its rows
  of the full call.
Planted mistakes (keys of the neighbouring sequence visible, one causal
offset for all sequences) each fail a pin.
"""

import math

import numpy as np
import torch

import gqa_inputs as gi
import oracle
from oracle import varlen as ovl


def f64(t):
    return t.to(torch.float64).numpy()


def brute(q, k, v, cu_q, cu_k, causal, scale):
    total_q, Hq, d = q.shape
    Hk = k.shape[1]
    G = Hq // Hk
    O = np.zeros((total_q, Hq, d))
    L = np.full((Hq, total_q), -math.inf)
    for b in range(len(cu_q) - 1):
        nq, nk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(nq):
            t = cu_q[b] + i
            for h in range(Hq):
                g = h // G
                sc = []
                for j in range(nk):
                    if causal and j > i + nk - nq:
                        continue
                    kt = cu_k[b] + j
                    sc.append((kt, scale * math.fsum(float(q[t, h, c]) * float(k[kt, g, c]) for c in range(d))))
                if not sc:
                    continue
                mx = max(s for _, s in sc)
                w = [(kt, math.exp(s - mx)) for kt, s in sc]
                tot = math.fsum(x for _, x in w)
                L[h, t] = mx + math.log(tot)
                for c in range(d):
                    O[t, h, c] = math.fsum(x * float(v[kt, g, c]) for kt, x in w) / tot
    return O, L


def pin_brute(attn):
    for seed, lq, lk in ((1, [3, 1, 5], [4, 6, 2]), (2, [0, 4, 2], [3, 0, 7]), (3, [6], [6])):
        q, k, v, cq, ck = gi.varlen_batch(seed, lq, lk, 6, 2, 4)
        for causal in (False, True):
            Ob, Lb = brute(f64(q), f64(k), f64(v), cq.tolist(), ck.tolist(), causal, 0.45)
            O, L = attn(f64(q), f64(k), f64(v), cq.numpy(), ck.numpy(), causal, 0.45)
            assert np.allclose(O, Ob, rtol=0, atol=1e-12), (seed, causal)
            fin = np.isfinite(Lb)
            assert np.array_equal(fin, np.isfinite(L)) and np.allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def pin_equal_lengths(attn):
    B, S, Hq, Hk, d = 3, 9, 4, 2, 8
    q, k, v, cq, ck = gi.varlen_batch(4, [S] * B, [S] * B, Hq, Hk, d)
    for causal in (False, True):
        O, L = attn(f64(q), f64(k), f64(v), cq.numpy(), ck.numpy(), causal, 0.3)
        Ob, Lb = oracle.attention_fp64(f64(q).reshape(B, S, Hq, d), f64(k).reshape(B, S, Hk, d),
                                       f64(v).reshape(B, S, Hk, d), causal, 0.3)
        assert np.allclose(O, Ob.reshape(B * S, Hq, d), rtol=0, atol=1e-13)
        assert np.allclose(L, Lb.transpose(1, 0, 2).reshape(Hq, B * S), rtol=0, atol=1e-13)


def pin_closed_forms(attn):
    q, k, v, cq, ck = gi.varlen_batch(5, [2, 0, 3], [0, 4, 5], 4, 2, 4)
    for causal in (False, True):
        O, L = attn(f64(q), f64(k), f64(v), cq.numpy(), ck.numpy(), causal, 0.5)
        assert np.all(O[:2] == 0) and np.all(np.isneginf(L[:, :2]))     # sequence 0 has no key
        Oa, La = attn(f64(q), f64(k), f64(v), cq.numpy(), ck.numpy(), causal, 0.5, sequences=[2])
        assert np.array_equal(Oa[2:], O[2:]) and np.array_equal(La[:, 2:], L[:, 2:])


PINS = [pin_brute, pin_equal_lengths, pin_closed_forms]


def test_varlen_pins():
    for pin in PINS:
        pin(oracle.attention_varlen_fp64)


def _fails(attn):
    try:
        for pin in PINS:
            pin(attn)
    except AssertionError:
        return True
    return False


def test_planted_neighbour_keys_visible():
    def bad(q, k, v, cq, ck, causal, scale, sequences=None):
        ck2 = np.array(ck).copy()
        ck2[1:-1] += 1                       # each sequence also sees the next one's first key
        return ovl.attention_varlen_fp64(q, k, v, cq, ck2, causal, scale, sequences)
    assert _fails(bad)


def test_planted_one_causal_offset(monkeypatch):
    from oracle import attention as oatt
    real = oatt.visible_keys

    def vis(i, Sq, Sk, causal):
        return real(i, Sq, Sq, causal)[:, :Sk] if Sk <= Sq else np.pad(real(i, Sq, Sq, causal), ((0, 0), (0, Sk - Sq)))
    monkeypatch.setattr(oatt, "visible_keys", vis)
    assert _fails(oracle.attention_varlen_fp64)
