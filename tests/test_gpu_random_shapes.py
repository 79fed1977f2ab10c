"""Seeded random shapes against the fp64 oracle (GPU): the bf16 forward, the fp8 Q/K forward, the fp8 K/V
decode path, the backward, variable-length batches and paged decode and prefill, each on shapes drawn from seeded
generators (batch 1-3, lengths 0-900 around the tile sizes, G in 1..8, Hk in 1..4, d in {64, 128}, causal
or not, packing, splits, page sizes and factors drawn too). Every case is small enough for the oracle to
finish in well under a second; tolerances as elsewhere. A last group draws shapes with enough work items
for the 8-wavefront prefill kernel (the batch size follows from the drawn lengths and heads) and checks
it bit for bit against the 4-wavefront kernel and against the oracle on two batch elements.
"""

import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import oracle
from _parity import TOL_LSE, TOL_O_MAX, TOL_O_MEAN, f64, force_tiled

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw(seed):
    rs = np.random.RandomState(seed)
    B = int(rs.randint(1, 4))
    Hk = int(rs.randint(1, 5))
    G = int(rs.choice([1, 2, 3, 4, 5, 8]))
    d = int(rs.choice([64, 128]))
    Sq = int(rs.choice([1, 2, 7, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 300]))
    Sk = int(rs.choice([1, 5, 32, 63, 64, 65, 128, 129, 257, 300]))
    causal = bool(rs.randint(0, 2))
    pack = int(rs.choice([-1, 0, 1]))
    ns = int(rs.choice([0, 1, 2, 3, 5]))
    return B, Sq, Sk, G * Hk, Hk, d, causal, pack, ns


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


@pytest.mark.parametrize("seed", range(24))
def test_random_forward_bf16_and_fp8_qk(seed):
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d, causal, pack, ns = draw(11000 + seed)
    tag = f"seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hk={Hk} d={d} causal={causal} pack={pack} ns={ns}"
    scale = gi.fp32(1 / math.sqrt(d))
    q, k, v = gi.random_bf16(seed, (B, Sq, Hq, d)), gi.random_bf16(seed + 100, (B, Sk, Hk, d)), gi.random_bf16(seed + 200, (B, Sk, Hk, d))
    out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, causal, scale, pack, ns)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention_fp64(f64(q), f64(k), f64(v), causal, scale)
    check(out, lse, Or, Lr, "bf16 " + tag)
    q8, k8 = gi.to_fp8_bytes(q), gi.to_fp8_bytes(k)
    qs, ks = 0.75, -1.5
    g.gqa_attn_fwd_qk8(q8.to(DEV), k8.to(DEV), v.to(DEV), qs, ks, out, lse, causal, scale, pack, ns)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention_qk8_fp64(q8.numpy(), k8.numpy(), f64(v), qs, ks, causal, scale)
    check(out, lse, Or, Lr, "fp8 Q/K " + tag)


@pytest.mark.parametrize("seed", range(12))
def test_random_decode_fp8_kv(seed):
    import grouped_query_exact_amd as g
    rs = np.random.RandomState(12000 + seed)
    B, Hk, G = int(rs.randint(1, 5)), int(rs.randint(1, 5)), int(rs.choice([1, 2, 4, 8]))
    d = int(rs.choice([64, 128]))
    Sq = int(rs.choice([1, 2, 4])) if G <= 8 else 1
    Sq = min(Sq, 32 // G)
    Sk = int(rs.randint(1, 900))
    causal, ns = bool(rs.randint(0, 2)), int(rs.choice([0, 1, 3]))
    Hq = G * Hk
    tag = f"seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hk={Hk} d={d} causal={causal} ns={ns}"
    q = gi.random_bf16(seed + 300, (B, Sq, Hq, d))
    k8, v8 = gi.random_fp8(seed + 400, (B, Sk, Hk, d)), gi.random_fp8(seed + 500, (B, Sk, Hk, d))
    out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd_kv8(q.to(DEV), k8.to(DEV), v8.to(DEV), 0.6, 1.7, out, lse, causal, gi.fp32(1 / math.sqrt(d)), -1, ns)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention_kv8_fp64(f64(q), k8.numpy(), v8.numpy(), 0.6, 1.7, causal, gi.fp32(1 / math.sqrt(d)))
    check(out, lse, Or, Lr, tag)


@pytest.mark.parametrize("seed", range(10))
def test_random_backward(seed):
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d, causal, _, _ = draw(13000 + seed)
    tag = f"seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hk={Hk} d={d} causal={causal}"
    scale = gi.fp32(1 / math.sqrt(d))
    q, k, v = gi.random_bf16(seed + 600, (B, Sq, Hq, d)), gi.random_bf16(seed + 700, (B, Sk, Hk, d)), gi.random_bf16(seed + 800, (B, Sk, Hk, d))
    do = gi.random_bf16(seed + 900, (B, Sq, Hq, d))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd(qd, kd, vd, out, lse, causal, scale)
    grads = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
    g.gqa_attn_bwd(qd, kd, vd, out, lse, do.to(DEV), *grads, causal, scale)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_fp64(f64(q), f64(k), f64(v), f64(do), causal, scale)
    for name, gx, rx in zip(("dq", "dk", "dv"), grads, ref):
        gx = f64(gx)
        assert np.isfinite(gx).all(), f"{tag} {name}: non-finite"
        m = np.abs(rx).max()
        err = np.abs(gx - rx)
        if m == 0:
            assert err.max() == 0, f"{tag} {name}: expected zeros"
            continue
        assert err.max() <= 2e-2 * m and err.mean() <= 2e-3 * m, f"{tag} {name}: max {err.max() / m:.3e} mean {err.mean() / m:.3e}"


@pytest.mark.parametrize("seed", range(8))
def test_random_varlen(seed):
    """Packed sequences with drawn lengths (empty ones included), chunked-prefill lengths (fewer queries
    than keys) and decode-shaped batches, drawn packing and splits."""
    import grouped_query_exact_amd as g
    rs = np.random.RandomState(14000 + seed)
    nseq = int(rs.randint(1, 7))
    Hk, G, d = int(rs.randint(1, 4)), int(rs.choice([1, 2, 3, 4, 8])), int(rs.choice([64, 128]))
    lk = [int(x) for x in rs.choice([0, 1, 17, 64, 65, 130, 300], size=nseq)]
    if rs.randint(0, 2):
        lq = [min(x, int(rs.choice([1, 2, 4]))) for x in lk]  # decode-shaped / short chunks
    else:
        lq = [int(min(x, rs.randint(0, x + 1))) for x in lk]  # chunked prefill: up to the key count
    if max(lk) == 0:
        lk[0] = 5
    causal, pack, ns = bool(rs.randint(0, 2)), int(rs.choice([-1, 0, 1])), int(rs.choice([0, 1, 3]))
    Hq = G * Hk
    q, k, v, cq, ck = gi.varlen_batch(14000 + seed, lq, lk, Hq, Hk, d)
    tag = f"seed={seed} lq={lq} lk={lk} Hq={Hq} Hk={Hk} d={d} causal={causal} pack={pack} ns={ns}"
    if sum(lq) == 0:
        return
    scale = gi.fp32(1 / math.sqrt(d))
    out = torch.empty((sum(lq), Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((Hq, sum(lq)), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, cq.to(DEV), ck.to(DEV), max(max(lq), 1),
                          max(max(lk), 1), causal, scale, pack, ns)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention_varlen_fp64(f64(q), f64(k), f64(v), cq.tolist(), ck.tolist(), causal, scale)
    check(out, lse, Or, Lr, tag)


@pytest.mark.parametrize("seed", range(8))
def test_random_paged_decode(seed):
    import grouped_query_exact_amd as g
    rs = np.random.RandomState(15000 + seed)
    nseq = int(rs.randint(1, 6))
    Hk, G, d = int(rs.randint(1, 4)), int(rs.choice([1, 2, 4, 8])), int(rs.choice([64, 128]))
    Sq = min(int(rs.choice([1, 2, 4])), 32 // G)
    ps = int(rs.choice([16, 32, 48, 64, 128]))
    lens = [int(x) for x in rs.randint(0, 700, size=nseq)]
    causal, ns = bool(rs.randint(0, 2)), int(rs.choice([0, 1, 3]))
    Hq = G * Hk
    kv = gi.paged_kv(15000 + seed, lens, ps, Hk, d, spare_pages=int(rs.randint(0, 4)))
    q = gi.random_bf16(15100 + seed, (nseq, Sq, Hq, d))
    tag = f"seed={seed} lens={lens} ps={ps} Sq={Sq} Hq={Hq} Hk={Hk} d={d} causal={causal} ns={ns}"
    kvd = kv.to(DEV)
    out = torch.empty((nseq, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((nseq, Hq, Sq), dtype=torch.float32, device=DEV)
    scale = gi.fp32(1 / math.sqrt(d))
    g.gqa_attn_fwd_paged(q.to(DEV), kvd.k_cache, kvd.v_cache, kvd.block_table, kvd.seqlens_k, out, lse, causal, scale,
                         -1, ns)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention_paged_fp64(f64(q), f64(kv.k_cache), f64(kv.v_cache), kv.block_table.numpy(),
                                         kv.seqlens_k.numpy(), causal, scale)
    check(out, lse, Or, Lr, tag)


@pytest.mark.parametrize("seed", range(8))
def test_random_paged_prefill(seed):
    """Chunks of 33-200 new tokens over a paged cache (the prefill kernels' page lookups)."""
    import grouped_query_exact_amd as g
    rs = np.random.RandomState(15500 + seed)
    nseq = int(rs.randint(1, 5))
    Hk, G, d = int(rs.randint(1, 4)), int(rs.choice([1, 2, 3, 4])), int(rs.choice([64, 128]))
    Sq = int(rs.choice([33, 40, 77, 130, 200]))
    ps = int(rs.choice([16, 32, 48, 64, 128]))
    lens = [int(x) for x in rs.randint(0, 700, size=nseq)]
    causal, pack, ns = bool(rs.randint(0, 2)), int(rs.choice([-1, 0, 1])), int(rs.choice([0, 1, 3]))
    Hq = G * Hk
    kv = gi.paged_kv(15500 + seed, lens, ps, Hk, d, spare_pages=int(rs.randint(0, 4)))
    q = gi.random_bf16(15600 + seed, (nseq, Sq, Hq, d))
    tag = f"seed={seed} lens={lens} ps={ps} Sq={Sq} Hq={Hq} Hk={Hk} d={d} causal={causal} pack={pack} ns={ns}"
    kvd = kv.to(DEV)
    out = torch.empty((nseq, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((nseq, Hq, Sq), dtype=torch.float32, device=DEV)
    scale = gi.fp32(1 / math.sqrt(d))
    g.gqa_attn_fwd_paged(q.to(DEV), kvd.k_cache, kvd.v_cache, kvd.block_table, kvd.seqlens_k, out, lse, causal, scale,
                         pack, ns)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention_paged_fp64(f64(q), f64(kv.k_cache), f64(kv.v_cache), kv.block_table.numpy(),
                                         kv.seqlens_k.numpy(), causal, scale)
    check(out, lse, Or, Lr, tag)


def draw8(seed):
    """A shape with at least 512 items of 256 packed rows (the 8-wavefront prefill kernel)."""
    rs = np.random.RandomState(seed)
    Hk = int(rs.choice([1, 2, 4]))
    G = int(rs.choice([1, 2, 3, 4, 8]))
    d = 128  # the 8-wavefront kernel runs at d=128 only
    Sq = int(rs.choice([200, 255, 256, 257, 300, 511, 512, 513, 700, 1025]))
    Sk = int(rs.choice([63, 64, 65, 199, 300, 511, 513, 1024, 1100]))
    causal = bool(rs.randint(0, 2))
    if not causal and Sk <= 8 * 64:  # non-causal rows of at most 8 key tiles keep the 4-wavefront kernel
        Sk += 576
    pack = 1 if G > 1 and rs.randint(0, 3) else 0
    units = Hk if pack else G * Hk
    rt8 = -(-(Sq * (G if pack else 1)) // 256)
    B = -(-512 // (units * rt8)) + int(rs.randint(0, 3))
    return B, Sq, Sk, G * Hk, Hk, d, causal, pack


@pytest.mark.parametrize("seed", range(16))
def test_random_forward_8_wavefront(seed):
    """The 8-wavefront kernel (d=128) on seeded shapes: bit for bit the 4-wavefront kernel (the same rows
    with GQA_ATTN_FORCE_TILED=1) on every row, the oracle on two batch elements."""
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d, causal, pack = draw8(12000 + seed)
    tag = f"seed={seed} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hk={Hk} d={d} causal={causal} pack={pack}"
    assert g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, causal, pack, 1, 0)["threads"] == 512, tag
    scale = gi.fp32(1 / math.sqrt(d))
    q, k, v = gi.random_bf16(seed + 300, (B, Sq, Hq, d)), gi.random_bf16(seed + 400, (B, Sk, Hk, d)), gi.random_bf16(seed + 500, (B, Sk, Hk, d))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd(qd, kd, vd, out, lse, causal, scale, pack, 1)
    o4 = torch.empty((B * Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
    l4 = torch.empty((Hq, B * Sq), dtype=torch.float32, device=DEV)
    cq = torch.arange(0, (B + 1) * Sq, Sq, dtype=torch.int32, device=DEV)
    ck = torch.arange(0, (B + 1) * Sk, Sk, dtype=torch.int32, device=DEV)
    with force_tiled():
        g.gqa_attn_fwd_varlen(qd.view(B * Sq, Hq, d), kd.view(B * Sk, Hk, d), vd.view(B * Sk, Hk, d), o4, l4, cq, ck,
                              Sq, Sk, causal, scale, pack, 1)
        torch.cuda.synchronize()
    assert torch.equal(out.view(B * Sq, Hq, d), o4), "O " + tag
    assert torch.equal(lse.permute(1, 0, 2).reshape(Hq, B * Sq), l4), "LSE " + tag
    sel = sorted({0, B - 1})
    Or, Lr = oracle.attention_fp64(f64(q[sel]), f64(k[sel]), f64(v[sel]), causal, scale)
    check(out[sel], lse[sel], Or, Lr, tag)
