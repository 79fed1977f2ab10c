"""The 8-wavefront prefill kernel against the fp64 oracle and, bit for bit,
against the 4-wavefront tiled kernel (GPU).

Unsplit bf16 calls at d=128 with at least two 256-row work items per compute
unit run on the 8-wavefront kernel. The shapes below sit just past that threshold (512
or more items on 256 compute units), so the oracle compares every element.
With GQA_ATTN_FORCE_TILED=1 every prefill call runs on the 4-wavefront kernel:
the same rows through it give that kernel's result, and since the two kernels
share their per-row arithmetic (tile order, operand order, softmax and
epilogue) they must agree bit for bit.
"""

import math

import pytest
import torch

import gqa_inputs as gi
from _parity import compare_to_oracle, force_tiled, gpu_run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, Sq, Sk, Hq, Hk, d, pack); every shape has >= 512 items of 256 packed rows
SHAPES = [
    (64, 256, 256, 8, 2, 128, 1),  # 4 full row tiles per group, 4 full key tiles
    (64, 200, 333, 8, 2, 128, 1),  # ragged rows (800 = 3 tiles + 32) and keys (5 tiles + 13), Sq != Sk
    (64, 300, 300, 6, 2, 128, 1),  # G = 3
    (32, 512, 448, 8, 2, 128, 0),  # unpacked: 2 row tiles per head
    (64, 300, 100, 8, 2, 128, 1),  # causal: tokens 0..199 see no key (bottom-right alignment)
    # causal launches pair row tile rt with row_tiles-1-rt in one workgroup:
    (16, 1800, 1800, 8, 2, 128, 1),  # 29 row tiles: the middle one runs alone; long heavy items
    (64, 2048, 40, 8, 2, 128, 1),   # every item has at most one key tile: the light items load their own Q
    (64, 2048, 150, 8, 2, 128, 1),  # heavy items of 2-3 key tiles: the light items' Q staged through LDS
]


def _keys(Sk, causal):
    """Non-causal calls whose rows read at most 8 key tiles keep the 4-wavefront kernel: those
    variants of the shapes get 576 more keys (9 more tiles, the raggedness kept)."""
    return Sk if causal or Sk > 8 * 64 else Sk + 576


def _qkv(seed, B, Sq, Sk, Hq, Hk, d):
    return (gi.random_bf16(seed, (B, Sq, Hq, d)), gi.random_bf16(seed + 1, (B, Sk, Hk, d)),
            gi.random_bf16(seed + 2, (B, Sk, Hk, d)))


def _assert_selected(B, Sq, Sk, Hq, Hk, d, causal, pack):
    import grouped_query_exact_amd as g
    p = g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, causal, pack, 1, 0)
    assert p["threads"] == 512 and p["block_m"] == 256, p


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}_Sq{s[1]}_Sk{s[2]}_G{s[3] // s[4]}_d{s[5]}_p{s[6]}" for s in SHAPES])
@pytest.mark.parametrize("causal", [True, False])
def test_oracle_parity(shape, causal):
    B, Sq, Sk, Hq, Hk, d, pack = shape
    Sk = _keys(Sk, causal)
    _assert_selected(B, Sq, Sk, Hq, Hk, d, causal, pack)
    q, k, v = _qkv(9700 + Sq + Sk + d, B, Sq, Sk, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    O, L = gpu_run(q, k, v, causal, scale, pack, 1)
    compare_to_oracle(O, L, q, k, v, causal, scale, tag=f"{shape} causal={causal}")


@pytest.mark.parametrize("scale", [-0.0883883461356163, 0.0, 0.5])
def test_scales(scale):
    """Negative factors (Q negated), 0 (uniform weights over the visible keys) and a
    large factor (peaked rows, many rescales of the running maximum). At 0.5 the rows
    put most weight on single keys, so |O| approaches |V| and the output is checked
    against the per-element rounding bound instead of the flat tolerance, as for the
    other stress inputs."""
    B, Sq, Sk, Hq, Hk, d, pack = SHAPES[1]
    Sk = _keys(Sk, False)
    q, k, v = _qkv(9800, B, Sq, Sk, Hq, Hk, d)
    for causal in (True, False):
        _assert_selected(B, Sq, Sk, Hq, Hk, d, causal, pack)
        O, L = gpu_run(q, k, v, causal, gi.fp32(scale), pack, 1)
        compare_to_oracle(O, L, q, k, v, causal, gi.fp32(scale), tag=f"scale={scale} causal={causal}",
                          derived_bound=abs(scale) > 0.1)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}_Sq{s[1]}_Sk{s[2]}_G{s[3] // s[4]}_d{s[5]}_p{s[6]}" for s in SHAPES])
def test_bitwise_equal_to_4_wavefront_kernel(shape):
    import grouped_query_exact_amd as g
    B, Sq, Sk0, Hq, Hk, d, pack = shape
    for causal in (True, False):
        Sk = _keys(Sk0, causal)
        q, k, v = _qkv(9900 + Sq + Sk + d, B, Sq, Sk, Hq, Hk, d)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        cq = torch.arange(0, (B + 1) * Sq, Sq, dtype=torch.int32, device=DEV)
        ck = torch.arange(0, (B + 1) * Sk, Sk, dtype=torch.int32, device=DEV)
        _assert_selected(B, Sq, Sk, Hq, Hk, d, causal, pack)
        scale = gi.fp32(1 / math.sqrt(d))
        O8, L8 = gpu_run(qd, kd, vd, causal, scale, pack, 1)
        O4 = torch.full((B * Sq, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        L4 = torch.full((Hq, B * Sq), float("nan"), dtype=torch.float32, device=DEV)
        with force_tiled():
            assert g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, causal, pack, 1)["threads"] == 256
            g.gqa_attn_fwd_varlen(qd.view(B * Sq, Hq, d), kd.view(B * Sk, Hk, d), vd.view(B * Sk, Hk, d), O4, L4, cq,
                                  ck, Sq, Sk, causal, scale, pack, 1)
            torch.cuda.synchronize()
        assert torch.equal(O8.view(B * Sq, Hq, d), O4), f"O {shape} causal={causal}"
        assert torch.equal(L8.permute(1, 0, 2).reshape(Hq, B * Sq), L4), f"LSE {shape} causal={causal}"


def test_without_lse():
    """lse = None: the kernel skips the LSE store and O is unchanged."""
    B, Sq, Sk, Hq, Hk, d, pack = SHAPES[0]
    q, k, v = _qkv(9950, B, Sq, Sk, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    Oa, _ = gpu_run(q, k, v, True, scale, pack, 1)
    Ob, Lb = gpu_run(q, k, v, True, scale, pack, 1, with_lse=False)
    assert Lb is None and torch.equal(Oa, Ob)


def test_random_shapes_bitwise():
    """Seeded random shapes that the plan sends to the 8-wavefront kernel (group sizes 1-8, query
    and key counts up to 3000 with Sq > Sk, Sq < Sk and Sq = Sk, causal or not, three score
    factors): the batched call (causal: paired row tiles) equals, bit for bit, the 4-wavefront
    kernel (the same tokens as an equal-length variable-length call with GQA_ATTN_FORCE_TILED=1)
    and the variable-length work list on the 8-wavefront kernel."""
    import numpy as np
    import grouped_query_exact_amd as g
    ran = 0
    for seed in range(160):
        rs = np.random.RandomState(70000 + seed)
        Hk = int(rs.choice([1, 2, 4, 8]))
        G = int(rs.choice([1, 2, 3, 4, 5, 8]))
        Hq, d = G * Hk, 128
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
        q = torch.randn((B, Sq, Hq, d), generator=gen, device=DEV).to(torch.bfloat16)
        k = torch.randn((B, Sk, Hk, d), generator=gen, device=DEV).to(torch.bfloat16)
        v = torch.randn((B, Sk, Hk, d), generator=gen, device=DEV).to(torch.bfloat16)
        ob = torch.full_like(q, float("nan"))
        lb = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd(q, k, v, ob, lb, causal, scale)
        cq = torch.arange(0, (B + 1) * Sq, Sq, dtype=torch.int32, device=DEV)
        ck = torch.arange(0, (B + 1) * Sk, Sk, dtype=torch.int32, device=DEV)
        tag = f"seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hk={Hk} causal={causal}"
        for tiled in (True, False):
            ov = torch.full((B * Sq, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
            lv = torch.full((Hq, B * Sq), float("nan"), dtype=torch.float32, device=DEV)
            call = lambda: g.gqa_attn_fwd_varlen(q.view(B * Sq, Hq, d), k.view(B * Sk, Hk, d), v.view(B * Sk, Hk, d),
                                                 ov, lv, cq, ck, Sq, Sk, causal, scale)
            if tiled:
                with force_tiled():
                    call()
            else:
                call()
            torch.cuda.synchronize()
            assert torch.equal(ov.view(B, Sq, Hq, d), ob), f"{tag} tiled={tiled}: O"
            assert torch.equal(lv.view(Hq, B, Sq).permute(1, 0, 2), lb), f"{tag} tiled={tiled}: LSE"
    assert ran >= 50, ran


@pytest.mark.parametrize("shape", [(1, 2048, 8192, 32, 8, 128, 1), (2, 1000, 3000, 32, 8, 128, 1)],
                         ids=["chunk2048_vs_8192", "B2_ragged1000_vs_3000"])
def test_causal_unpaired_row_tiles(shape):
    """Causal calls whose mirrored pairs of row tiles would not give every compute unit one (a
    chunk of new tokens against a longer context) run one row tile per workgroup, heaviest
    first: bit for bit the 4-wavefront kernel, and the oracle on sampled rows."""
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d, pack = shape
    p = g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, True, pack, 1, 256)
    assert p["threads"] == 512 and p["grid"] == B * Hk * p["row_tiles"], p
    q, k, v = _qkv(9990 + Sq, B, Sq, Sk, Hq, Hk, d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = gi.fp32(1 / math.sqrt(d))
    O8, L8 = gpu_run(qd, kd, vd, True, scale, pack, 1)
    with force_tiled():
        O4, L4 = gpu_run(qd, kd, vd, True, scale, pack, 1)
    assert torch.equal(O8, O4) and torch.equal(L8, L4), f"{shape}: differs from the 4-wavefront kernel"
    compare_to_oracle(O8, L8, q, k, v, True, scale, rows=[0, 1, 255, 256, Sq // 2, Sq - 1], tag=f"{shape}")
