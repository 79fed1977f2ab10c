"""The 8-wavefront prefill kernel against the fp64 oracle and, bit for bit,
against the 4-wavefront tiled kernel (GPU).

Unsplit bf16 calls at d=128 with at least two 256-row work items per compute
unit run on the 8-wavefront kernel. The shapes below sit just past that threshold (512
or more items on 256 compute units), so the oracle compares every element.
Variable-length calls always use the 4-wavefront kernel: a batch of
equal-length sequences through gqa_attn_fwd_varlen gives that kernel's result
for the same rows, and since the two kernels share their per-row arithmetic
(tile order, operand order, softmax and epilogue) they must agree bit for bit.
"""

import math

import pytest
import torch

import gqa_inputs as gi
from _parity import compare_to_oracle, gpu_run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, Sq, Sk, Hq, Hk, d, pack); every shape has >= 512 items of 256 packed rows
SHAPES = [
    (64, 256, 256, 8, 2, 128, 1),  # 4 full row tiles per group, 4 full key tiles
    (64, 200, 333, 8, 2, 128, 1),  # ragged rows (800 = 3 tiles + 32) and keys (5 tiles + 13), Sq != Sk
    (64, 300, 300, 6, 2, 128, 1),  # G = 3
    (32, 512, 448, 8, 2, 128, 0),  # unpacked: 2 row tiles per head
    (64, 300, 100, 8, 2, 128, 1),  # causal: tokens 0..199 see no key (bottom-right alignment)
]


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
    _assert_selected(B, Sq, Sk, Hq, Hk, d, True, pack)
    q, k, v = _qkv(9800, B, Sq, Sk, Hq, Hk, d)
    for causal in (True, False):
        O, L = gpu_run(q, k, v, causal, gi.fp32(scale), pack, 1)
        compare_to_oracle(O, L, q, k, v, causal, gi.fp32(scale), tag=f"scale={scale} causal={causal}",
                          derived_bound=abs(scale) > 0.1)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}_Sq{s[1]}_Sk{s[2]}_G{s[3] // s[4]}_d{s[5]}_p{s[6]}" for s in SHAPES])
def test_bitwise_equal_to_4_wavefront_kernel(shape):
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d, pack = shape
    q, k, v = _qkv(9900 + Sq + Sk + d, B, Sq, Sk, Hq, Hk, d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    cq = torch.arange(0, (B + 1) * Sq, Sq, dtype=torch.int32, device=DEV)
    ck = torch.arange(0, (B + 1) * Sk, Sk, dtype=torch.int32, device=DEV)
    for causal in (True, False):
        _assert_selected(B, Sq, Sk, Hq, Hk, d, causal, pack)
        scale = gi.fp32(1 / math.sqrt(d))
        O8, L8 = gpu_run(qd, kd, vd, causal, scale, pack, 1)
        O4 = torch.full((B * Sq, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        L4 = torch.full((Hq, B * Sq), float("nan"), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd_varlen(qd.view(B * Sq, Hq, d), kd.view(B * Sk, Hk, d), vd.view(B * Sk, Hk, d), O4, L4, cq, ck,
                              Sq, Sk, causal, scale, pack, 1)
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
