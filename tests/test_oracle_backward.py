"""Pins of the backward oracle to facts other than itself (CPU only).

* library routine: torch autograd in fp64 through the plain forward formula
  with the KV heads repeated in place (autograd sums the repeats' gradients:
  the GQA reduction), causal and not, Sq != Sk;
* finite differences: central differences of sum(dO * O) along random
  directions of Q, K and V on tiny inputs;
* closed forms: dO = 0 gives zero gradients; values equal for every key give
  O = that value, dS = 0 and so dQ = dK = 0 exactly, with dV_j = sum_i P_ij dO_i;
* invariants: the key gradients of each KV head sum to zero (shifting every
  key by the same vector leaves every softmax unchanged); the row dot D equals
  sum_j P_ij dP_ij.
Planted mistakes (the -D term dropped, only the first head of a group
counted, the scale missing from dQ) each fail a pin.
"""

import math

import numpy as np
import torch

import oracle
from oracle import backward as obw


def rnd(shape, seed, std=1.0):
    return np.random.RandomState(seed).standard_normal(shape) * std


def torch_grads(q, k, v, do, causal, scale):
    B, Sq, Hq, d = q.shape
    Sk, Hk = k.shape[1], k.shape[2]
    G = Hq // Hk
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kr = tk.repeat_interleave(G, dim=2)
    vr = tv.repeat_interleave(G, dim=2)
    s = torch.einsum("bihc,bjhc->bhij", tq, kr) * scale
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        s = s.masked_fill(~(j <= i + (Sk - Sq)), float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)
    o = torch.einsum("bhij,bjhc->bihc", p, vr)
    (o * torch.tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


SHAPES = [(1, 5, 5, 2, 1, 4), (2, 7, 9, 6, 2, 8), (1, 9, 4, 4, 2, 3), (1, 1, 11, 8, 2, 16), (2, 6, 6, 3, 3, 5)]


def pin_autograd(bwd):
    for n, (B, Sq, Sk, Hq, Hk, d) in enumerate(SHAPES):
        q, k, v = rnd((B, Sq, Hq, d), 10 + n), rnd((B, Sk, Hk, d), 20 + n), rnd((B, Sk, Hk, d), 30 + n)
        do = rnd((B, Sq, Hq, d), 40 + n)
        for causal in (False, True):
            if causal and Sq > Sk:
                continue  # rows without keys: torch's softmax of all -inf is NaN; covered by the closed forms
            ref = torch_grads(q, k, v, do, causal, 0.37)
            got = bwd(q, k, v, do, causal, 0.37)
            for r, g, name in zip(ref, got, ("dq", "dk", "dv")):
                assert np.allclose(g, r, rtol=0, atol=1e-11), (n, causal, name, np.abs(g - r).max())


def pin_finite_differences(bwd):
    B, Sq, Sk, Hq, Hk, d = 1, 4, 6, 4, 2, 3
    q, k, v = rnd((B, Sq, Hq, d), 51), rnd((B, Sk, Hk, d), 52), rnd((B, Sk, Hk, d), 53)
    do = rnd((B, Sq, Hq, d), 54)
    for causal in (False, True):
        grads = bwd(q, k, v, do, causal, 0.5)

        def loss(q_, k_, v_):
            O, _ = oracle.attention_fp64(q_, k_, v_, causal, 0.5)
            return float((O * do).sum())
        rs = np.random.RandomState(55)
        for which, x in enumerate((q, k, v)):
            for _ in range(3):
                u = rs.standard_normal(x.shape)
                eps = 1e-5
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which] = x + eps * u
                args_m[which] = x - eps * u
                fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                an = float((grads[which] * u).sum())
                assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, causal, fd, an)


def pin_closed_forms(bwd):
    B, Sq, Sk, Hq, Hk, d = 1, 5, 7, 4, 2, 6
    q, k = rnd((B, Sq, Hq, d), 61), rnd((B, Sk, Hk, d), 62)
    v = rnd((B, Sk, Hk, d), 63)
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, np.zeros((B, Sq, Hq, d)), causal, 0.4)
        assert not dq.any() and not dk.any() and not dv.any()
        vc = np.broadcast_to(rnd((1, 1, Hk, d), 64), (B, Sk, Hk, d)).copy()   # every key has the same value
        do = rnd((B, Sq, Hq, d), 65)
        dq, dk, dv = bwd(q, k, vc, do, causal, 0.4)
        assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
        O, L, P = oracle.attention_fp64(q, k, vc, causal, 0.4, return_p=True)
        G = Hq // Hk
        for g in range(Hk):
            ref = sum(P[0, h].T @ do[0, :, h] for h in range(g * G, (g + 1) * G))
            assert np.allclose(dv[0, :, g], ref, atol=1e-12)


def pin_invariants(bwd):
    B, Sq, Sk, Hq, Hk, d = 2, 6, 8, 6, 2, 5
    q, k, v, do = rnd((B, Sq, Hq, d), 71), rnd((B, Sk, Hk, d), 72), rnd((B, Sk, Hk, d), 73), rnd((B, Sq, Hq, d), 74)
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, causal, 0.6)
        assert np.abs(dk.sum(axis=1)).max() < 1e-11          # sum over keys of each KV head's key gradient
        O, L, P = oracle.attention_fp64(q, k, v, causal, 0.6, return_p=True)
        D = oracle.row_dot_fp64(O, do)
        G = Hq // Hk
        for b in range(B):
            for h in range(Hq):
                dP = do[b, :, h] @ v[b, :, h // G].T
                assert np.allclose(D[b, h], (P[b, h] * dP).sum(axis=1), atol=1e-12)


PINS = [pin_autograd, pin_finite_differences, pin_closed_forms, pin_invariants]


def test_backward_pins():
    for pin in PINS:
        pin(oracle.attention_bwd_fp64)


def _fails(bwd):
    for pin in PINS:
        try:
            pin(bwd)
        except AssertionError:
            return True
    return False


def _variant(drop_d=False, first_head_only=False, dq_unscaled=False):
    from oracle.attention import _row_softmax, kv_head_of, visible_keys

    def bwd(q, k, v, do, causal, scale):
        B, Sq, Hq, d = q.shape
        _, Sk, Hk, _ = k.shape
        G = Hq // Hk
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        vis = visible_keys(np.arange(Sq), Sq, Sk, causal)
        for b in range(B):
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hk)
                Q, K, V, dO = q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h]
                P, _, _ = _row_softmax(scale * (Q @ K.T), vis)
                O = P @ V
                dP = dO @ V.T
                D = 0.0 if drop_d else (dO * O).sum(axis=1)[:, None]
                dS = P * (dP - D)
                dq[b, :, h] = (1.0 if dq_unscaled else scale) * (dS @ K)
                if not first_head_only or h % G == 0:
                    dv[b, :, g] += P.T @ dO
                    dk[b, :, g] += scale * (dS.T @ Q)
        return dq, dk, dv
    return bwd


def test_planted_mistakes():
    assert _fails(_variant(drop_d=True))
    assert _fails(_variant(first_head_only=True))
    assert _fails(_variant(dq_unscaled=True))
    assert not _fails(_variant())   # the unplanted copy passes
