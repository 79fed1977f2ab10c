"""CPU oracle for the backward pass of exact grouped-query attention (fp64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module. The GPU library never calls
it and shares no code with it; this module imports numpy and the plain
oracle only.

The pages benchmark the forward and backward passes of flash attention
together (batch-sensitivity article, "performance analysis" training
numbers) and name training among its uses; they do not write the gradients
out. They follow from the forward definition by the chain rule. With
P = softmax(scale * Q K^T) over the visible keys, O = P V and an upstream
gradient dO of O, for query head h of KV group g:

  dV_g  = sum over the heads h of g of P^T dO
  dP    = dO V^T,  D_i = sum_c dO[i,c] * O[i,c]  (= sum_j P_ij dP_ij)
  dS    = P * (dP - D)                     (elementwise, row i uses D_i)
  dQ_h  = scale * dS K_g
  dK_g  = scale * sum over the heads h of g of dS^T Q_h

Masked keys have P = 0 and so contribute nothing; a row with no visible
key has P = 0 and gradient 0. The heads of a group share K and V, so their
contributions to dK and dV add up (the GQA reduction).
"""

from __future__ import annotations

import numpy as np

from .attention import _row_softmax, kv_head_of, visible_keys


def attention_bwd_fp64(q, k, v, do, causal: bool, scale: float):
    """dQ [B,Sq,Hq,d], dK [B,Sk,Hk,d], dV [B,Sk,Hk,d] of sum(dO * O) with O the exact forward output."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Sq, Hq, d = q.shape
    _, Sk, Hk, _ = k.shape
    scale = float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    vis = visible_keys(np.arange(Sq), Sq, Sk, causal)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hk)
            Q, K, V, dO = q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h]
            P, _, _ = _row_softmax(scale * (Q @ K.T), vis)
            O = P @ V
            dv[b, :, g] += P.T @ dO
            dP = dO @ V.T
            D = (dO * O).sum(axis=1)
            dS = P * (dP - D[:, None])
            dq[b, :, h] = scale * (dS @ K)
            dk[b, :, g] += scale * (dS.T @ Q)
    return dq, dk, dv


def row_dot_fp64(o, do):
    """D = sum over the head dimension of dO * O, laid out [B, Hq, Sq] like the LSE."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.transpose((o * do).sum(axis=-1), (0, 2, 1))
