"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (fp32 accumulation, bf16 inputs and outputs):
  max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <= 1e-3 against the fp64 oracle.

Variants (pack_gqa on/off, num_splits, tiled against decode kernel) against each other.
The literal "variants agree within 1e-3" cannot hold for every bf16 output: where
|O| >= 0.25 one bf16 step is 2^-9 = 1.95e-3, and two tilings of a row sum their fp32
terms in another order, so a value near a rounding boundary can land one step apart.
Both sides round every probability against an integral running maximum (raised lazily,
to an integer, in every kernel), so the probabilities themselves agree up to the last bit of the exponent
argument; what remains are fp32 reassociation differences. Enforced:
  * every element: |dO| <= max(1e-3, 2 bf16 steps at max(|a|, |b|));
  * at most 0.1% of the elements differ by more than 1e-3;
  * mean |dO| <= 1e-4;
  * LSE within 1e-3 (same -inf pattern);
  * reported: the strict max |dO| and the counts of elements 1 and 2 bf16 steps apart.
  pack_gqa on/off does the same arithmetic per row and is required to be bitwise equal.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

class force_tiled:
    """Context manager: prefill calls inside it run on the 4-wavefront tiled kernel
    (GQA_ATTN_FORCE_TILED=1, read by the library's planner at every call)."""

    def __enter__(self):
        import os
        self._old = os.environ.get("GQA_ATTN_FORCE_TILED")
        os.environ["GQA_ATTN_FORCE_TILED"] = "1"
        return self

    def __exit__(self, *exc):
        import os
        if self._old is None:
            os.environ.pop("GQA_ATTN_FORCE_TILED", None)
        else:
            os.environ["GQA_ATTN_FORCE_TILED"] = self._old
        return False


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


def bf16_ulp(x: torch.Tensor) -> torch.Tensor:
    """Spacing of bf16 values at magnitude |x| (7 stored mantissa bits)."""
    ax = x.abs().clamp_min(2.0 ** -126)
    return torch.exp2(torch.floor(torch.log2(ax)) - 7)


def bf16_steps(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Number of representable bf16 values between a and b (0: equal, 1: neighbours)."""
    ia = a.view(torch.int16).to(torch.int32)
    ib = b.view(torch.int16).to(torch.int32)
    ka = torch.where(ia < 0, -(ia & 0x7FFF), ia)
    kb = torch.where(ib < 0, -(ib & 0x7FFF), ib)
    return (ka - kb).abs()


VARIANT_FRAC = 1e-3   # share of elements allowed beyond TOL_VARIANT
VARIANT_FAR = 1e-6    # share of elements allowed beyond max(1e-3, two bf16 steps)
VARIANT_MEAN = 1e-4


def assert_variants_agree(Oa, La, Ob, Lb, vmax: float, tag="", strict=False):
    """Compare two variants' bf16 outputs (and LSEs); returns a dict of the statistics.

    Both sides apply the same bf16 probabilities, except where the last bit of an
    exponent argument s*c - m rounds differently under the two running maxima and
    flips one probability P_j by one bf16 step (2^-8 of it at most). That moves the
    output by delta * (V_j - O) / l with O = p V_j + (1 - p) O_rest, p = P_j / l, so by at
    most 2^-8 * p * (1 - p) * |V_j - O_rest| <= 2^-9 * max|V|, plus one output rounding on
    each side. Enforced: every element within that bound; at most a share VARIANT_FAR of
    the elements beyond max(1e-3, two bf16 steps at max(|a|, |b|)); at most VARIANT_FRAC
    beyond 1e-3; mean |dO| <= VARIANT_MEAN; LSE within 1e-3. strict=True requires every
    element within 1e-3 (the literal reading, which holds where all outputs are below
    0.25, e.g. decode).
    """
    dmax, dsum, nbig, nfar, n1, n2, n = 0.0, 0.0, 0, 0, 0, 0, 0
    for i in range(Oa.shape[0]):  # one batch element at a time bounds the temporaries
        a, b = Oa[i].float(), Ob[i].float()
        d = (a - b).abs()
        two_steps = 2.0 * bf16_ulp(torch.maximum(a.abs(), b.abs()))
        near = torch.clamp_min(two_steps, TOL_VARIANT)
        worst = float((d - (2.0 ** -9 * vmax + two_steps + 1e-4)).max())
        assert worst <= 0, (f"{tag}: variants differ by {float(d.max())} at batch {i}, beyond one probability "
                            f"rounding step (2^-9 * max|V| = {2.0 ** -9 * vmax:.3e}) plus two bf16 steps")
        st = bf16_steps(Oa[i].contiguous(), Ob[i].contiguous())
        n1 += int((st == 1).sum())
        n2 += int((st == 2).sum())
        nfar += int((d > near).sum())
        dmax = max(dmax, float(d.max()))
        dsum += float(d.double().sum())
        nbig += int((d > TOL_VARIANT).sum())
        n += d.numel()
    mean, frac = dsum / n, nbig / n
    stats = {"max": dmax, "mean": mean, "frac_gt_1e-3": frac, "n_1step": n1, "n_2step": n2,
             "n_beyond_2steps": nfar, "n": n}
    print(f"[variants] {tag}: strict max|dO| {dmax:.3e}, mean {mean:.3e}, beyond 1e-3: {nbig} of {n} "
          f"({frac:.2e}), 1 bf16 step apart: {n1}, 2 steps: {n2}, beyond max(1e-3, 2 steps): {nfar}", flush=True)
    assert frac <= VARIANT_FRAC, f"{tag}: {frac:.2e} of the elements differ by more than 1e-3"
    assert nfar <= VARIANT_FAR * n, f"{tag}: {nfar} elements differ by more than max(1e-3, two bf16 steps)"
    assert mean <= VARIANT_MEAN, f"{tag}: mean variant difference {mean}"
    if strict:
        assert dmax <= TOL_VARIANT, f"{tag}: strict max|dO| {dmax} > 1e-3"
    if La is not None and Lb is not None:
        fa, fb = torch.isfinite(La), torch.isfinite(Lb)
        assert torch.equal(fa, fb), f"{tag}: LSE -inf pattern differs"
        dl = float((La[fa] - Lb[fb]).abs().max()) if bool(fa.any()) else 0.0
        assert dl <= TOL_VARIANT, f"{tag}: LSE variants differ by {dl}"
        stats["lse_max"] = dl
    return stats
