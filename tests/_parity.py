"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (fp32 accumulation, bf16 inputs and outputs):
  max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <= 1e-3 against the fp64 oracle.

Variants (pack_gqa on/off, num_splits) against each other:
  * LSE within 1e-3 (it is computed from fp32 probabilities, so variants differ by ~1e-6);
  * O: both paths round the probabilities P to bf16 (relative error <= 2^-9) before the
    P.V product, each relative to its own running maximum, so an unsplit and a split
    result can differ by up to 2 * 2^-9 * max|V| in fp32 plus one bf16 step of the
    output rounding. Every element must stay within max(1e-3, that bound); in addition
    the mean difference must stay below 1e-4 and at most 0.1% of the elements may
    differ by more than 1e-3 (a dropped or doubled key would break both).
  pack_gqa on/off does the same arithmetic per row and is required to be bitwise equal.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

TOL_O_MAX = 2e-2
TOL_O_MEAN = 2e-3
TOL_LSE = 1e-3
TOL_VARIANT = 1e-3


def gpu_run(q, k, v, causal, scale, pack, ns, with_lse=True, device="cuda:0"):
    """q/k/v CPU or GPU bf16 tensors -> (O bf16 GPU, LSE fp32 GPU or None)."""
    import grouped_query_exact_amd as g
    q = q.to(device)
    k = k.to(device)
    v = v.to(device)
    B, Sq, Hq, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device) if with_lse else None
    g.gqa_attn_fwd(q, k, v, out, lse, causal, scale, pack, ns)
    torch.cuda.synchronize()
    return out, lse


def f64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def compare_to_oracle(O_gpu, L_gpu, q, k, v, causal, scale, batches=None, heads=None, rows=None, tag=""):
    """Compare GPU outputs (full tensors) with the oracle on the selected slice."""
    Or, Lr = oracle.attention_fp64(f64(q), f64(k), f64(v), causal, scale, batches=batches, heads=heads, rows=rows)
    bs = list(range(q.shape[0])) if batches is None else list(batches)
    hs = list(range(q.shape[2])) if heads is None else list(heads)
    rs = list(range(q.shape[1])) if rows is None else list(rows)
    Og = f64(O_gpu[bs][:, rs][:, :, hs])
    dO = np.abs(Og - Or)
    assert np.isfinite(Og).all(), f"{tag}: non-finite output"
    mx, mean = float(dO.max()) if dO.size else 0.0, float(dO.mean()) if dO.size else 0.0
    assert mx <= TOL_O_MAX, f"{tag}: max|dO| = {mx}"
    assert mean <= TOL_O_MEAN, f"{tag}: mean|dO| = {mean}"
    if L_gpu is not None:
        Lg = f64(L_gpu[bs][:, hs][:, :, rs])
        fin = np.isfinite(Lr)
        assert np.array_equal(fin, np.isfinite(Lg)), f"{tag}: -inf pattern of LSE differs"
        assert np.all(Lg[~fin] == -np.inf), f"{tag}: masked rows must have LSE = -inf"
        dl = float(np.abs(Lg[fin] - Lr[fin]).max()) if fin.any() else 0.0
        assert dl <= TOL_LSE, f"{tag}: max|dLSE| = {dl}"
        return mx, mean, dl
    return mx, mean, 0.0


def bf16_adjacent(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """True where two bf16 tensors hold the same or neighbouring representable values."""
    ia = a.view(torch.int16).to(torch.int32)
    ib = b.view(torch.int16).to(torch.int32)
    # map sign-magnitude to a monotone integer line
    ka = torch.where(ia < 0, -(ia & 0x7FFF), ia)
    kb = torch.where(ib < 0, -(ib & 0x7FFF), ib)
    return (ka - kb).abs() <= 1


def bf16_ulp(x: torch.Tensor) -> torch.Tensor:
    """Spacing of bf16 values at magnitude |x| (7 stored mantissa bits)."""
    ax = x.abs().clamp_min(2.0 ** -126)
    return torch.exp2(torch.floor(torch.log2(ax)) - 7)


def assert_variants_agree(Oa, La, Ob, Lb, vmax: float, tag=""):
    dmax, dsum, nbig, n = 0.0, 0.0, 0, 0
    for i in range(Oa.shape[0]):  # one batch element at a time bounds the temporaries
        a, b = Oa[i].float(), Ob[i].float()
        d = (a - b).abs()
        bound = torch.clamp_min(2.0 * 2.0 ** -9 * vmax + bf16_ulp(torch.maximum(a.abs(), b.abs())), TOL_VARIANT)
        worst = float((d - bound).max())
        assert worst <= 0, f"{tag}: variants differ by {float(d.max())} at batch {i}, beyond the rounding bound"
        dmax = max(dmax, float(d.max()))
        dsum += float(d.double().sum())
        nbig += int((d > TOL_VARIANT).sum())
        n += d.numel()
    mean, frac = dsum / n, nbig / n
    assert mean <= 1e-4, f"{tag}: mean variant difference {mean}"
    assert frac <= 1e-3, f"{tag}: {frac:.2e} of the elements differ by more than 1e-3"
    if La is not None and Lb is not None:
        fa, fb = torch.isfinite(La), torch.isfinite(Lb)
        assert torch.equal(fa, fb), f"{tag}: LSE -inf pattern differs"
        dl = float((La[fa] - Lb[fb]).abs().max()) if bool(fa.any()) else 0.0
        assert dl <= TOL_VARIANT, f"{tag}: LSE variants differ by {dl}"
    return dmax, mean, frac
