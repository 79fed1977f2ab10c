"""Forward with fp8 e4m3 Q and K on the fp8 matrix cores (gqa_attn_fwd_qk8) against the fp8 oracle (GPU).

The scores are products of e4m3 values, exact in the fp32 accumulation, and
P V runs on the bf16 products as in gqa_attn_fwd, so the bf16 path's
tolerances apply against the oracle over q_scale * Q and k_scale * K. On the
same decoded values the LSE must also agree with the bf16 path to 1e-4
(the two differ only in how the score partial sums are added: 64-term fp8
products against 16-term bf16 ones; measured 4.6e-5 on LSEs of about 6). Cases: ragged lengths around the 128-row and 64-key tiles, every
group size, both packings, splits, both head dimensions, negative and
fractional factors, scale 0, rows without visible keys (causal, Sq > Sk),
decode-shaped calls (which run on the tiled kernel here), and the Llama-2
prefill shape on sampled rows.
"""

import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import oracle
from _parity import TOL_LSE, TOL_O_MAX, TOL_O_MEAN, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_qk8(q8, k8, v, qs, ks, causal, scale, pack=-1, ns=0):
    import grouped_query_exact_amd as g
    B, Sq, Hq, d = q8.shape
    out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd_qk8(q8.to(DEV), k8.to(DEV), v.to(DEV), qs, ks, out, lse, causal, scale, pack, ns)
    torch.cuda.synchronize()
    return out, lse


def check(O, L, Or, Lr, tag):
    Og = f64(O)
    assert np.isfinite(Og).all(), f"{tag}: non-finite output"
    dO = np.abs(Og - Or)
    assert dO.max() <= TOL_O_MAX and dO.mean() <= TOL_O_MEAN, f"{tag}: max {dO.max()} mean {dO.mean()}"
    Lg = f64(L)
    fin = np.isfinite(Lr)
    assert np.array_equal(fin, np.isfinite(Lg)), f"{tag}: LSE -inf pattern"
    if fin.any():
        assert np.abs(Lg[fin] - Lr[fin]).max() <= TOL_LSE, f"{tag}: LSE"


CASES = [
    # B, Sq, Sk, Hq, Hk, d
    (2, 100, 100, 8, 2, 128),
    (1, 77, 150, 6, 2, 64),
    (1, 150, 77, 4, 4, 128),
    (2, 256, 200, 16, 2, 128),
    (1, 129, 257, 8, 8, 64),
    (3, 1, 300, 32, 8, 128),
    (2, 4, 1000, 8, 2, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_qk8_parity(case):
    B, Sq, Sk, Hq, Hk, d = case
    seed = 9500 + sum(case)
    q8, k8 = gi.random_fp8(seed, (B, Sq, Hq, d)), gi.random_fp8(seed + 1, (B, Sk, Hk, d))
    v = gi.random_bf16(seed + 2, (B, Sk, Hk, d))
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (False, True):
        for qs, ks, pack, ns in ((1.0, 1.0, -1, 0), (0.37, 2.5, 1, 3), (-0.5, 1.25, 0, 1), (1.0, -1.0, 1, 1)):
            O, L = run_qk8(q8, k8, v, qs, ks, causal, scale, pack, ns)
            Or, Lr = oracle.attention_qk8_fp64(q8.numpy(), k8.numpy(), f64(v), qs, ks, causal, scale)
            check(O, L, Or, Lr, f"{case} causal={causal} qs={qs} ks={ks} pack={pack} ns={ns}")


def test_qk8_matches_bf16_path_on_decoded_values():
    """Unit factors: the same operation as gqa_attn_fwd on bf16 tensors holding the decoded e4m3 values."""
    import grouped_query_exact_amd as g
    B, S, Hq, Hk, d = 2, 333, 16, 4, 128
    q8, k8 = gi.random_fp8(9600, (B, S, Hq, d)), gi.random_fp8(9601, (B, S, Hk, d))
    v = gi.random_bf16(9602, (B, S, Hk, d))
    qb = q8.view(torch.float8_e4m3fn).to(torch.bfloat16).to(DEV)
    kb = k8.view(torch.float8_e4m3fn).to(torch.bfloat16).to(DEV)
    for causal in (False, True):
        O8, L8 = run_qk8(q8, k8, v, 1.0, 1.0, causal, 0.0883883461356163)
        ob = torch.empty_like(O8)
        lb = torch.empty_like(L8)
        g.gqa_attn_fwd(qb, kb, v.to(DEV), ob, lb, causal, 0.0883883461356163)
        torch.cuda.synchronize()
        assert (L8 - lb).abs().max().item() <= 1e-4, f"causal={causal}: LSE differs from the bf16 path"
        assert (O8.float() - ob.float()).abs().max().item() <= 2 ** -7, f"causal={causal}: O differs"
        assert (O8 == ob).float().mean().item() > 0.9, f"causal={causal}: fewer than 90% of outputs identical"


def test_qk8_scale_zero_and_empty_rows():
    """scale 0: every visible key weighs the same (the mean of the visible values); causal with Sq > Sk:
    rows that see no key give O = 0 and LSE = -inf."""
    B, Sq, Sk, Hq, Hk, d = 1, 90, 40, 8, 2, 64
    q8, k8 = gi.random_fp8(9700, (B, Sq, Hq, d)), gi.random_fp8(9701, (B, Sk, Hk, d))
    v = gi.random_bf16(9702, (B, Sk, Hk, d))
    for scale in (0.0, 0.125):
        O, L = run_qk8(q8, k8, v, 0.75, 1.5, True, scale)
        Or, Lr = oracle.attention_qk8_fp64(q8.numpy(), k8.numpy(), f64(v), 0.75, 1.5, True, scale)
        check(O, L, Or, Lr, f"scale={scale}")
        assert torch.all(O[:, : Sq - Sk].float() == 0) and torch.all(torch.isneginf(L[:, :, : Sq - Sk]))


def test_qk8_llama_shape_sampled():
    """Llama-2 prefill shape (B=4, S=2048, Hq=32, Hk=8, d=128, causal), library's choice; oracle on sampled rows."""
    B, S, Hq, Hk, d = 4, 2048, 32, 8, 128
    q8, k8 = gi.random_fp8(9800, (B, S, Hq, d)), gi.random_fp8(9801, (B, S, Hk, d))
    v = gi.random_bf16(9802, (B, S, Hk, d))
    scale = gi.fp32(1 / math.sqrt(d))
    O, L = run_qk8(q8, k8, v, 0.5, 2.0, True, scale)
    assert torch.isfinite(O.float()).all()
    rows = [0, 1, 63, 64, 127, 128, 1000, 2046, 2047]
    for b in (0, 3):
        Or, Lr = oracle.attention_qk8_fp64(q8.numpy()[b:b + 1], k8.numpy()[b:b + 1], f64(v)[b:b + 1], 0.5, 2.0, True,
                                           scale, rows=rows)
        check(O[b:b + 1, rows].cpu(), L[b:b + 1, :, rows].cpu(), Or, Lr, f"llama b={b}")


def test_qk8_rejects_bad_factors():
    import grouped_query_exact_amd as g
    q8 = torch.zeros((1, 64, 4, 64), dtype=torch.uint8, device=DEV)
    k8 = torch.zeros((1, 64, 2, 64), dtype=torch.uint8, device=DEV)
    v = torch.zeros((1, 64, 2, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((1, 64, 4, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(g.GqaAttnError) as e:
        g.gqa_attn_fwd_qk8(q8, k8, v, float("nan"), 1.0, out, None, True, 0.125)
    assert e.value.status == g.GQA_ERR_INVALID_ARG


PP_SHAPES = [
    # B, Sq, Sk, Hq, Hk, pack: at least 512 items of 256 packed rows (the 8-wavefront kernel)
    (64, 256, 256, 8, 2, 1),
    (64, 200, 333, 8, 2, 1),   # ragged rows and keys, Sq != Sk
    (64, 300, 300, 6, 2, 1),   # G = 3
    (32, 512, 448, 8, 2, 0),   # unpacked
    (64, 300, 100, 8, 2, 1),   # causal: tokens 0..199 see no key
    (16, 1800, 1800, 8, 2, 1), # causal pairs with an odd middle tile
]


@pytest.mark.parametrize("shape", PP_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_qk8_8_wavefront_kernel(shape):
    """Large unsplit calls run on the 8-wavefront kernel with fp8 scores: bit for bit the
    4-wavefront kernel (GQA_ATTN_FORCE_TILED=1) at unit, fractional and negative factors, and the
    oracle on sampled rows (every row for the first shape)."""
    import grouped_query_exact_amd as g
    from _parity import force_tiled
    B, Sq, Sk0, Hq, Hk, pack = shape
    d = 128
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (True, False):
        Sk = Sk0 if causal or Sk0 > 8 * 64 else Sk0 + 576  # non-causal rows of <= 8 key tiles keep 4 wavefronts
        assert g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, causal, pack, 1)["threads"] == 512
        seed = 9900 + Sq + Sk + Hq
        q8, k8 = gi.random_fp8(seed, (B, Sq, Hq, d)), gi.random_fp8(seed + 1, (B, Sk, Hk, d))
        v = gi.random_bf16(seed + 2, (B, Sk, Hk, d))
        for qs, ks in ((1.0, 1.0), (0.37, -2.5)):
            O8, L8 = run_qk8(q8, k8, v, qs, ks, causal, scale, pack, 1)
            with force_tiled():
                O4, L4 = run_qk8(q8, k8, v, qs, ks, causal, scale, pack, 1)
            tag = f"{shape} causal={causal} qs={qs} ks={ks}"
            assert torch.equal(O8, O4) and torch.equal(L8, L4), f"{tag}: differs from the 4-wavefront kernel"
            if qs == 1.0:
                rows = None if shape == PP_SHAPES[0] else sorted({0, 1, Sq // 3, Sq // 2, Sq - 2, Sq - 1})
                bs = None if shape == PP_SHAPES[0] else [0, B - 1]
                Or, Lr = oracle.attention_qk8_fp64(q8.numpy(), k8.numpy(), f64(v), qs, ks, causal, scale, rows=rows,
                                                   batches=bs)
                Og = O8.cpu() if rows is None else O8.cpu()[bs][:, rows]
                Lg = L8.cpu() if rows is None else L8.cpu()[bs][:, :, rows]
                check(Og, Lg, Or, Lr, tag)


def test_qk8_random_shapes_bitwise():
    """Seeded random shapes that the plan sends to the 8-wavefront kernel (group sizes 1-8, query and
    key counts up to 3000, causal or not, paired and unpaired causal row tiles, three score
    factors): the fp8 Q/K call equals, bit for bit, the same call on the 4-wavefront kernel."""
    import numpy as np
    import grouped_query_exact_amd as g
    from _parity import force_tiled
    ran = 0
    d = 128
    for seed in range(120):
        rs = np.random.RandomState(81000 + seed)
        Hk = int(rs.choice([1, 2, 4, 8]))
        G = int(rs.choice([1, 2, 3, 4, 5, 8]))
        Hq = G * Hk
        Sq = int(rs.randint(1, 3000))
        Sk = int(rs.choice([Sq, rs.randint(1, 3000)]))
        causal = bool(rs.randint(0, 2))
        B = int(rs.randint(1, 25))
        if g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, causal, -1, 0)["threads"] != 512:
            continue
        if B * Sq * Hq * d > 2.5e8 or B * Sk * Hk * d > 2.5e8:
            continue
        ran += 1
        scale = float(rs.choice([1 / math.sqrt(d), 0.3, -0.05]))
        gen = torch.Generator(device=DEV)
        gen.manual_seed(seed)
        q8 = torch.randn((B, Sq, Hq, d), generator=gen, device=DEV).to(torch.float8_e4m3fn).view(torch.uint8)
        k8 = torch.randn((B, Sk, Hk, d), generator=gen, device=DEV).to(torch.float8_e4m3fn).view(torch.uint8)
        v = torch.randn((B, Sk, Hk, d), generator=gen, device=DEV).to(torch.bfloat16)
        O8, L8 = run_qk8(q8, k8, v, 1.0, 1.0, causal, scale)
        with force_tiled():
            O4, L4 = run_qk8(q8, k8, v, 1.0, 1.0, causal, scale)
        tag = f"seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hk={Hk} causal={causal}"
        assert torch.equal(O8, O4) and torch.equal(L8, L4), tag
    assert ran >= 30, ran
