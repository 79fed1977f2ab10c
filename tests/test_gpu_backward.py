"""Backward pass (gqa_attn_bwd) against the fp64 backward oracle (GPU).

The forward call on the GPU provides O and the log-sum-exp, as in training;
the oracle differentiates the exact forward. Tolerances (per gradient tensor
X, relative to max|X_ref|): max|dX| <= 2e-2 and mean|dX| <= 2e-3. The GPU
rounds P and dS to bf16 for the matrix products (relative error 2^-9 each),
takes D from the bf16 forward output (error about 2^-9 |O| |dO|) and rounds
the gradients to bf16; summed over a contraction these errors stay a few
2^-9 of the largest entry, well inside the bound.
Cases: ragged lengths around the 128-row / 128-key / 64-key tiles, every
group size, Sq < Sk and Sq > Sk (rows without keys), decode-like single
queries, scale 0 and negative, both head dimensions, and a Llama-2-shaped
causal problem.
"""

import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import oracle
from _parity import f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_MAX, TOL_MEAN = 2e-2, 2e-3


def run_bwd(q, k, v, do, causal, scale):
    import grouped_query_exact_amd as g
    q, k, v, do = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    B, Sq, Hq, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd(q, k, v, out, lse, causal, scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    g.gqa_attn_bwd(q, k, v, out, lse, do, dq, dk, dv, causal, scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare(got, q, k, v, do, causal, scale, tag):
    ref = oracle.attention_bwd_fp64(f64(q), f64(k), f64(v), f64(do), causal, scale)
    for name, gx, rx in zip(("dq", "dk", "dv"), got, ref):
        gx = f64(gx)
        assert np.isfinite(gx).all(), f"{tag} {name}: non-finite"
        m = np.abs(rx).max()
        err = np.abs(gx - rx)
        if m == 0:
            assert err.max() == 0, f"{tag} {name}: expected exact zeros"
            continue
        assert err.max() <= TOL_MAX * m, f"{tag} {name}: max {err.max() / m:.3e} of max|ref| {m:.3e}"
        assert err.mean() <= TOL_MEAN * m, f"{tag} {name}: mean {err.mean() / m:.3e} of max|ref| {m:.3e}"


CASES = [
    # B, Sq, Sk, Hq, Hk, d
    (2, 100, 100, 8, 2, 128),
    (1, 77, 150, 6, 2, 64),
    (1, 150, 77, 4, 4, 128),
    (2, 256, 256, 16, 2, 128),
    (1, 1, 300, 32, 8, 128),
    (1, 129, 257, 8, 8, 64),
    (2, 33, 33, 2, 1, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_backward_parity(case):
    B, Sq, Sk, Hq, Hk, d = case
    seed = 6000 + sum(case)
    q, k, v = gi.random_bf16(seed, (B, Sq, Hq, d)), gi.random_bf16(seed + 1, (B, Sk, Hk, d)), gi.random_bf16(seed + 2, (B, Sk, Hk, d))
    do = gi.random_bf16(seed + 3, (B, Sq, Hq, d))
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (False, True):
        compare(run_bwd(q, k, v, do, causal, scale), q, k, v, do, causal, scale, tag=f"{case} causal={causal}")


@pytest.mark.parametrize("scale", [0.0, -0.1])
def test_backward_scale_corners(scale):
    B, Sq, Sk, Hq, Hk, d = 1, 70, 90, 8, 2, 64
    q, k, v = gi.random_bf16(6100, (B, Sq, Hq, d)), gi.random_bf16(6101, (B, Sk, Hk, d)), gi.random_bf16(6102, (B, Sk, Hk, d))
    do = gi.random_bf16(6103, (B, Sq, Hq, d))
    for causal in (False, True):
        got = run_bwd(q, k, v, do, causal, scale)
        if scale == 0.0:
            assert torch.all(got[0] == 0) and torch.all(got[1] == 0)   # dQ = dK = 0 exactly
        compare(got, q, k, v, do, causal, scale, tag=f"scale={scale} causal={causal}")


def test_backward_llama_shape():
    """Hq=32, Hk=8, d=128, causal, one sequence of 1024 tokens (all heads, full check)."""
    B, S, Hq, Hk, d = 1, 1024, 32, 8, 128
    q, k, v = gi.random_bf16(6200, (B, S, Hq, d)), gi.random_bf16(6201, (B, S, Hk, d)), gi.random_bf16(6202, (B, S, Hk, d))
    do = gi.random_bf16(6203, (B, S, Hq, d))
    scale = gi.fp32(1 / math.sqrt(d))
    compare(run_bwd(q, k, v, do, True, scale), q, k, v, do, True, scale, tag="llama 1024")


def test_backward_key_gradients_sum_to_zero_full_size():
    """Llama-2 prefill shape (B=4, S=2048): per KV head the key gradients sum to zero (every softmax is
    unchanged by a common shift of the keys), up to the rounding of the bf16 gradients."""
    B, S, Hq, Hk, d = 4, 2048, 32, 8, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(6300)
    q = torch.randn((B, S, Hq, d), generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, S, Hk, d), generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, S, Hk, d), generator=gen, device=DEV).to(torch.bfloat16)
    do = torch.randn((B, S, Hq, d), generator=gen, device=DEV).to(torch.bfloat16)
    dq, dk, dv = run_bwd(q, k, v, do, True, gi.fp32(1 / math.sqrt(d)))
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
    colsum = dk.double().sum(dim=1)                # [B, Hk, d]
    scale_ref = dk.double().abs().sum(dim=1)
    assert float((colsum.abs() / scale_ref).max()) < 2e-2


def test_backward_without_queries():
    """Sq = 0: no query sees any key, so dK = dV = 0 (written over NaN-filled outputs); the query-side
    tensors are empty (null pointers)."""
    import grouped_query_exact_amd as g
    B, Sk, Hq, Hk, d = 2, 50, 8, 2, 128
    q = torch.empty((B, 0, Hq, d), dtype=torch.bfloat16, device=DEV)
    k, v = gi.random_bf16(6400, (B, Sk, Hk, d)).to(DEV), gi.random_bf16(6401, (B, Sk, Hk, d)).to(DEV)
    out, do, dq = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, Hq, 0), dtype=torch.float32, device=DEV)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    for causal in (False, True):
        g.gqa_attn_bwd(q, k, v, out, lse, do, dq, dk, dv, causal, 0.125)
        torch.cuda.synchronize()
        assert torch.all(dk == 0) and torch.all(dv == 0), f"causal={causal}"
