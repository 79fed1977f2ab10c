"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (fp32 accumulation, bf16 inputs and outputs):
  max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <= 1e-3 against the fp64 oracle.

Variants (pack_gqa on/off, num_splits) against each other:
  * LSE within 1e-3 (it is computed from fp32 probabilities, so variants differ by ~1e-6);
  * O: both paths round the probabilities P to bf16 (relative error <= 2^-9) before the
    P.V product, each relative to its own running maximum, so an unsplit and a split
    result can differ by up to 2 * 2^-9 * max|V| in fp32 plus one bf16 step of the
    output rounding. Every element must stay within max(1e-3, that bound); in addition
    the mean difference must stay below max(1e-4, 2^-9 * mean|O|), the size
    of one probability rounding relative to the outputs' own magnitude.
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


def rounding_bound(Or: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Per-element error bound of the GPU arithmetic against the exact result.

    Each probability P = 2^(s*c - m) carries a relative error of at most
    2^-9 from its bf16 rounding plus |scale| * gamma_d * sum_i |q_i k_i| from
    the fp32 accumulation of the score (gamma_d = d * 2^-24, the classical
    dot-product bound), so the fp32 output is within eps * max|V| of the
    exact one. Rounding the output to bf16 adds half a bf16 step at the
    largest magnitude the fp32 value can have; 1e-4 covers exp2 and the
    final normalisation. Used for stress inputs whose outputs reach
    magnitudes where the flat 2e-2 tolerance is below the output rounding.
    """
    d = q.shape[-1]
    qabs = np.abs(q).sum(axis=-1).max()
    kmax = np.abs(k).max()
    eps = 2.0 ** -9 + abs(scale) * d * 2.0 ** -24 * qabs * kmax
    vmax = float(np.abs(v).max())
    top = np.abs(Or) + eps * vmax + 1e-4
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(top, 2.0 ** -126))) - 8)
    return eps * vmax + half_ulp + 1e-4


def compare_to_oracle(O_gpu, L_gpu, q, k, v, causal, scale, batches=None, heads=None, rows=None, tag="",
                      derived_bound=False):
    """Compare GPU outputs (full tensors) with the oracle on the selected slice.

    derived_bound=True replaces the flat max tolerance by rounding_bound (stress inputs only).
    """
    Or, Lr = oracle.attention_fp64(f64(q), f64(k), f64(v), causal, scale, batches=batches, heads=heads, rows=rows)
    bs = list(range(q.shape[0])) if batches is None else list(batches)
    hs = list(range(q.shape[2])) if heads is None else list(heads)
    rs = list(range(q.shape[1])) if rows is None else list(rows)
    Og = f64(O_gpu[bs][:, rs][:, :, hs])
    dO = np.abs(Og - Or)
    assert np.isfinite(Og).all(), f"{tag}: non-finite output"
    mx, mean = float(dO.max()) if dO.size else 0.0, float(dO.mean()) if dO.size else 0.0
    if derived_bound:
        excess = float((dO - rounding_bound(Or, f64(q), f64(k), f64(v), scale)).max()) if dO.size else 0.0
        assert excess <= 0, f"{tag}: max|dO| = {mx} exceeds the rounding bound by {excess}"
    else:
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
    dmax, dsum, asum, nbig, n = 0.0, 0.0, 0.0, 0, 0
    for i in range(Oa.shape[0]):  # one batch element at a time bounds the temporaries
        a, b = Oa[i].float(), Ob[i].float()
        d = (a - b).abs()
        bound = torch.clamp_min(2.0 * 2.0 ** -9 * vmax + bf16_ulp(torch.maximum(a.abs(), b.abs())), TOL_VARIANT)
        worst = float((d - bound).max())
        assert worst <= 0, f"{tag}: variants differ by {float(d.max())} at batch {i}, beyond the rounding bound"
        dmax = max(dmax, float(d.max()))
        dsum += float(d.double().sum())
        asum += float(a.abs().double().sum())
        nbig += int((d > TOL_VARIANT).sum())
        n += d.numel()
    mean, frac = dsum / n, nbig / n
    assert mean <= max(1e-4, 2.0 ** -9 * asum / n), f"{tag}: mean variant difference {mean} (mean|O| {asum / n})"
    if La is not None and Lb is not None:
        fa, fb = torch.isfinite(La), torch.isfinite(Lb)
        assert torch.equal(fa, fb), f"{tag}: LSE -inf pattern differs"
        dl = float((La[fa] - Lb[fb]).abs().max()) if bool(fa.any()) else 0.0
        assert dl <= TOL_VARIANT, f"{tag}: LSE variants differ by {dl}"
    return dmax, mean, frac
