"""Decode with fp8 e4m3 K/V (gqa_attn_fwd_kv8, gqa_attn_fwd_paged_kv8) against the fp8 oracle (GPU).

The kernel converts each fp8 tile exactly to bf16 and then runs the bf16
arithmetic, so with k_scale = v_scale = 1 its result must equal, bit for
bit, the bf16 path on K/V holding the same values; with other factors it
must match the oracle over k_scale * K and v_scale * V to the same
tolerances as the bf16 path. Cases: one and four new tokens, ragged and
tile-multiple key lengths, causal and not, both head dimensions, splits,
negative and fractional factors, paged pools with NaN in every unused row,
and the full-size decode shape on sampled sequences.
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


def run_kv8(q, k8, v8, ks, vs, causal, scale, pack=-1, ns=0):
    import grouped_query_exact_amd as g
    B, Sq, Hq, d = q.shape
    out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd_kv8(q.to(DEV), k8.to(DEV), v8.to(DEV), ks, vs, out, lse, causal, scale, pack, ns)
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


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sk", [1, 33, 96, 1000])
def test_kv8_parity(d, Sk):
    B, Hq, Hk = 3, 8, 2
    k8, v8 = gi.random_fp8(8000 + Sk + d, (B, Sk, Hk, d)), gi.random_fp8(8100 + Sk + d, (B, Sk, Hk, d))
    scale = gi.fp32(1 / math.sqrt(d))
    for Sq in (1, 4):
        q = gi.random_bf16(8200 + Sk + d + Sq, (B, Sq, Hq, d))
        for causal in (False, True):
            for ks, vs, ns in ((1.0, 1.0, 1), (0.37, 2.5, 3), (-0.5, 1.0, 2)):
                O, L = run_kv8(q, k8, v8, ks, vs, causal, scale, 1, ns)
                Or, Lr = oracle.attention_kv8_fp64(f64(q), k8.numpy(), v8.numpy(), ks, vs, causal, scale)
                check(O, L, Or, Lr, f"d={d} Sk={Sk} Sq={Sq} causal={causal} ks={ks} vs={vs} ns={ns}")


def test_kv8_equals_bf16_path_bitwise():
    """k_scale = v_scale = 1: the same products as the bf16 path on the decoded values."""
    import grouped_query_exact_amd as g
    B, Sk, Hq, Hk, d = 4, 777, 32, 8, 128
    k8, v8 = gi.random_fp8(8300, (B, Sk, Hk, d)), gi.random_fp8(8301, (B, Sk, Hk, d))
    kb = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = v8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    q = gi.random_bf16(8302, (B, 1, Hq, d))
    for causal in (False, True):
        for ns in (1, 4):
            O8, L8 = run_kv8(q, k8, v8, 1.0, 1.0, causal, 0.0883883461356163, 1, ns)
            out = torch.empty_like(O8)
            lse = torch.empty_like(L8)
            g.gqa_attn_fwd(q.to(DEV), kb.to(DEV), vb.to(DEV), out, lse, causal, 0.0883883461356163, 1, ns)
            torch.cuda.synchronize()
            assert torch.equal(O8, out) and torch.equal(L8, lse), f"causal={causal} ns={ns}"


def test_paged_kv8_parity_and_bitwise():
    import grouped_query_exact_amd as g
    lens = [0, 1, 31, 33, 200, 1000]
    kv = gi.paged_kv(8400, lens, 32, 2, 128, spare_pages=3)
    k8, v8 = gi.to_fp8_bytes(kv.k_cache), gi.to_fp8_bytes(kv.v_cache)
    q = gi.random_bf16(8401, (len(lens), 2, 8, 128))
    qd, k8d, v8d = q.to(DEV), k8.to(DEV), v8.to(DEV)
    tab, sl = kv.block_table.to(DEV), kv.seqlens_k.to(DEV)
    scale = gi.fp32(1 / math.sqrt(128))
    for causal in (False, True):
        for ks, vs, ns in ((1.0, 1.0, 1), (0.8, 1.5, 3)):
            out = torch.empty((len(lens), 2, 8, 128), dtype=torch.bfloat16, device=DEV)
            lse = torch.empty((len(lens), 8, 2), dtype=torch.float32, device=DEV)
            g.gqa_attn_fwd_paged_kv8(qd, k8d, v8d, ks, vs, tab, sl, out, lse, causal, scale, 1, ns)
            torch.cuda.synchronize()
            Or, Lr = oracle.attention_paged_kv8_fp64(f64(q), k8.numpy(), v8.numpy(), kv.block_table.numpy(),
                                                     kv.seqlens_k.numpy(), ks, vs, causal, scale)
            check(out, lse, Or, Lr, f"paged causal={causal} ks={ks} ns={ns}")
            if ks == 1.0 and vs == 1.0:   # same values as a bf16 pool: bitwise equal
                kb = k8.view(torch.float8_e4m3fn).to(torch.bfloat16).to(DEV)
                vb = v8.view(torch.float8_e4m3fn).to(torch.bfloat16).to(DEV)
                ob = torch.empty_like(out)
                lb = torch.empty_like(lse)
                g.gqa_attn_fwd_paged(qd, kb, vb, tab, sl, ob, lb, causal, scale, 1, ns)
                torch.cuda.synchronize()
                assert torch.equal(out, ob) and torch.equal(lse, lb), f"paged bitwise causal={causal}"


def test_kv8_full_size_sampled():
    """The decode workload's shape (B=64, Sk=8192, Hq=32, Hk=8, d=128) with fp8 K/V, library's choice."""
    B, Sk, Hq, Hk, d = 64, 8192, 32, 8, 128
    k8 = gi.random_fp8(8500, (B, Sk, Hk, d))
    v8 = gi.random_fp8(8501, (B, Sk, Hk, d))
    q = gi.random_bf16(8502, (B, 1, Hq, d))
    O, L = run_kv8(q, k8, v8, 0.5, 2.0, False, gi.fp32(1 / math.sqrt(d)))
    assert torch.isfinite(O.float()).all()
    bs = [0, 21, 63]
    Or, Lr = oracle.attention_kv8_fp64(f64(q[bs]), k8[bs].numpy(), v8[bs].numpy(), 0.5, 2.0, False,
                                       gi.fp32(1 / math.sqrt(d)))
    check(O[bs], L[bs], Or, Lr, "full size")


def test_kv8_rejects_prefill_shapes():
    import grouped_query_exact_amd as g
    q = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device=DEV)
    k8 = torch.zeros((1, 64, 2, 64), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(g.GqaAttnError) as e:
        g.gqa_attn_fwd_kv8(q, k8, k8, 1.0, 1.0, out, None, True, 0.125)
    assert e.value.status == g.GQA_ERR_UNSUPPORTED


def test_kv8_one_sequence_long():
    """One sequence of 32 query heads over 8 fp8 KV heads against 16389 keys with the
    automatic split count (128 on 256 compute units: the one-workgroup-per-row merge)
    and with 128 splits asked for explicitly."""
    B, Sq, Sk, Hq, Hk, d = 1, 1, 16384 + 5, 32, 8, 128
    k8, v8 = gi.random_fp8(8700, (B, Sk, Hk, d)), gi.random_fp8(8701, (B, Sk, Hk, d))
    q = gi.random_bf16(8702, (B, Sq, Hq, d))
    scale = gi.fp32(1 / math.sqrt(d))
    for ks, vs, ns in ((1.0, 1.0, 0), (0.37, 2.5, 0), (1.0, 1.0, 128)):
        O, L = run_kv8(q, k8, v8, ks, vs, False, scale, -1, ns)
        Or, Lr = oracle.attention_kv8_fp64(f64(q), k8.numpy(), v8.numpy(), ks, vs, False, scale)
        check(O, L, Or, Lr, f"ks={ks} vs={vs} ns={ns}")


def test_kv8_many_split_workgroups():
    """fp8 K/V with many more split workgroups than the GPU keeps resident (64 x 8 x 24 = 12288):
    bit for bit the bf16 path on the same values at the same split count, and the oracle."""
    B, Sq, Sk, Hq, Hk, d = 64, 2, 2000, 32, 8, 128
    k8, v8 = gi.random_fp8(8800, (B, Sk, Hk, d)), gi.random_fp8(8801, (B, Sk, Hk, d))
    q = gi.random_bf16(8802, (B, Sq, Hq, d))
    scale = gi.fp32(1 / math.sqrt(d))
    kb = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = v8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    for causal in (False, True):
        O8, L8 = run_kv8(q, k8, v8, 1.0, 1.0, causal, scale, 1, 24)
        import grouped_query_exact_amd as g
        ob = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
        lb = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd(q.to(DEV), kb.to(DEV), vb.to(DEV), ob, lb, causal, scale, 1, 24)
        torch.cuda.synchronize()
        assert torch.equal(O8, ob) and torch.equal(L8, lb), f"causal={causal}"
        sel = [0, 31, 63]
        Or, Lr = oracle.attention_kv8_fp64(f64(q[sel]), k8[sel].numpy(), v8[sel].numpy(), 1.0, 1.0, causal, scale)
        check(O8[sel], L8[sel], Or, Lr, f"kv8 many items causal={causal}")
