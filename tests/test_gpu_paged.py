"""Decode and chunked prefill over a paged KV cache (gqa_attn_fwd_paged) against the paged
fp64 oracle (GPU).

The cache is a pool of pages handed out in a seeded random order; sequences
have their own key lengths (empty ones included) and the unused page rows,
unused pages and unused table entries hold NaN / -1, so any read outside the
sequences shows up as a non-finite output. Cases: page sizes 16 to 256 around
the 32-key tile, lengths around page and tile boundaries, causal and not, one
and four new tokens (decode kernel) and chunks of 40 and 200 tokens (tiled
kernel), both head dimensions and several split counts; the paged path
against the contiguous path (bitwise, same tile order, decode and prefill);
and the full-size decode workload on sampled sequences.
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


def run_paged(q, kv, causal, scale, pack=-1, ns=0):
    import grouped_query_exact_amd as g
    q = q.to(DEV)
    kvd = kv.to(DEV)
    B, Sq, Hq, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd_paged(q, kvd.k_cache, kvd.v_cache, kvd.block_table, kvd.seqlens_k, out, lse, causal, scale,
                         pack, ns)
    torch.cuda.synchronize()
    return out, lse


def compare_paged(O, L, q, kv, causal, scale, batches=None, tag=""):
    bs = list(range(q.shape[0])) if batches is None else list(batches)
    Or, Lr = oracle.attention_paged_fp64(f64(q), f64(kv.k_cache), f64(kv.v_cache), kv.block_table.numpy(),
                                         kv.seqlens_k.numpy(), causal, scale, batches=bs)
    Og = f64(O[bs])
    assert np.isfinite(Og).all(), f"{tag}: non-finite output (a read outside the sequences?)"
    dO = np.abs(Og - Or)
    assert dO.max() <= TOL_O_MAX and dO.mean() <= TOL_O_MEAN, f"{tag}: max {dO.max()} mean {dO.mean()}"
    Lg = f64(L[bs])
    fin = np.isfinite(Lr)
    assert np.array_equal(fin, np.isfinite(Lg)), f"{tag}: -inf pattern of LSE differs"
    if fin.any():
        assert np.abs(Lg[fin] - Lr[fin]).max() <= TOL_LSE, f"{tag}: LSE"


LENGTHS = [0, 1, 15, 16, 17, 31, 32, 33, 100, 257, 1000]


@pytest.mark.parametrize("page_size", [16, 32, 48, 64, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_paged_decode_parity(page_size, d):
    """Ragged and empty sequences, causal and not, 1 and 4 new tokens, ns 1 / 3 / 8."""
    Hq, Hk = 8, 2
    kv = gi.paged_kv(7000 + page_size + d, LENGTHS, page_size, Hk, d, spare_pages=3)
    scale = gi.fp32(1 / math.sqrt(d))
    for Sq in (1, 4):
        q = gi.random_bf16(7100 + page_size + d + Sq, (len(LENGTHS), Sq, Hq, d))
        for causal in (False, True):
            for ns in (1, 3, 8):
                O, L = run_paged(q, kv, causal, scale, 1, ns)
                compare_paged(O, L, q, kv, causal, scale, tag=f"ps={page_size} d={d} Sq={Sq} causal={causal} ns={ns}")


def test_paged_unpacked_and_auto():
    """One head per workgroup (pack 0, 4 rows of one head) and the library's own choice."""
    kv = gi.paged_kv(7200, [300, 64, 5], 64, 2, 128)
    q = gi.random_bf16(7201, (3, 4, 8, 128))
    for pack, ns in ((0, 1), (0, 2), (-1, 0)):
        O, L = run_paged(q, kv, True, 0.0883883461356163, pack, ns)
        compare_paged(O, L, q, kv, True, 0.0883883461356163, tag=f"pack={pack} ns={ns}")


PREFILL_LENGTHS = [0, 1, 63, 64, 65, 200, 517, 1000]


@pytest.mark.parametrize("page_size", [16, 48, 64, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_paged_prefill_parity(page_size, d):
    """Chunks of 40 and 200 new tokens (more than 32 rows per head unit: the tiled kernel)
    against ragged and empty cached sequences; causal (with rows that see no key where the
    chunk is longer than the cache) and not; packed with 1 split, unpacked with 3, and the
    library's choice."""
    import grouped_query_exact_amd as g
    Hq, Hk = 8, 2
    kv = gi.paged_kv(7500 + page_size + d, PREFILL_LENGTHS, page_size, Hk, d, spare_pages=3)
    scale = gi.fp32(1 / math.sqrt(d))
    for Sq in (40, 200):
        q = gi.random_bf16(7600 + page_size + d + Sq, (len(PREFILL_LENGTHS), Sq, Hq, d))
        for causal in (False, True):
            for pack, ns in ((1, 1), (0, 3), (-1, 0)):
                plan = g.gqa_attn_plan(len(PREFILL_LENGTHS), Sq, kv.block_table.shape[1] * page_size, Hq, Hk, d,
                                       causal, pack, ns, 256)
                assert plan["block_m"] != 32, plan
                O, L = run_paged(q, kv, causal, scale, pack, ns)
                compare_paged(O, L, q, kv, causal, scale,
                              tag=f"prefill ps={page_size} d={d} Sq={Sq} causal={causal} pack={pack} ns={ns}")


def test_paged_prefill_equals_contiguous_bitwise():
    """A 300-token chunk against 1000 cached keys per sequence, pages in order: the tiled
    kernel reads the same keys in the same tile order as the contiguous call."""
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d, ps = 3, 300, 1000, 32, 8, 128, 64
    P = -(-Sk // ps)
    q, k, v = gi.random_bf16(7700, (B, Sq, Hq, d)), gi.random_bf16(7701, (B, Sk, Hk, d)), gi.random_bf16(7702, (B, Sk, Hk, d))
    kc = torch.zeros((B * P, ps, Hk, d), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc.view(B, P * ps, Hk, d)[:, :Sk] = k
    vc.view(B, P * ps, Hk, d)[:, :Sk] = v
    kv = gi.PagedKV(kc, vc, torch.arange(B * P, dtype=torch.int32).view(B, P), torch.full((B,), Sk, dtype=torch.int32))
    for causal in (False, True):
        for pack, ns in ((1, 1), (0, 1), (1, 3)):
            Op, Lp = run_paged(q, kv, causal, 0.0883883461356163, pack, ns)
            out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
            lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
            g.gqa_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, causal, 0.0883883461356163, pack, ns)
            torch.cuda.synchronize()
            assert torch.equal(Op, out) and torch.equal(Lp, lse), f"causal={causal} pack={pack} ns={ns}"


def test_paged_prefill_8_wavefront():
    """16 sequences, 512-token chunks, 32 query heads over 8 KV heads (1024 items of 256 packed
    rows: the 8-wavefront kernel), ragged cached lengths (one shorter than the chunk, so causal
    rows that see no key), pages of 64 in random pool order: oracle on sampled sequences. With
    equal lengths and pages in order: bitwise equal to the contiguous call."""
    import grouped_query_exact_amd as g
    B, Sq, Hq, Hk, d, ps = 16, 512, 32, 8, 128, 64
    rs = np.random.RandomState(7800)
    lens = [int(x) for x in rs.randint(300, 2000, size=B)]
    lens[0], lens[1] = 100, 2048
    kv = gi.paged_kv(7800, lens, ps, Hk, d, spare_pages=3)
    q = gi.random_bf16(7801, (B, Sq, Hq, d))
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (True, False):
        plan = g.gqa_attn_plan(B, Sq, kv.block_table.shape[1] * ps, Hq, Hk, d, causal, -1, 1, 256)
        assert plan["threads"] == 512, plan
        O, L = run_paged(q, kv, causal, scale, -1, 1)
        assert torch.isfinite(O.float()).all()
        compare_paged(O, L, q, kv, causal, scale, batches=[0, 1, 9], tag=f"8-wavefront causal={causal}")
    Sk = 1024
    P = Sk // ps
    k, v = gi.random_bf16(7802, (B, Sk, Hk, d)), gi.random_bf16(7803, (B, Sk, Hk, d))
    kvc = gi.PagedKV(k.reshape(B * P, ps, Hk, d).contiguous(), v.reshape(B * P, ps, Hk, d).contiguous(),
                     torch.arange(B * P, dtype=torch.int32).view(B, P), torch.full((B,), Sk, dtype=torch.int32))
    for causal in (True, False):
        Op, Lp = run_paged(q, kvc, causal, scale, -1, 1)
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, causal, scale, -1, 1)
        torch.cuda.synchronize()
        assert torch.equal(Op, out) and torch.equal(Lp, lse), f"causal={causal}"


def test_paged_equals_contiguous_bitwise():
    """Pages laid out in order (page b*P + p holds keys p*ps.. of sequence b) and equal lengths:
    the paged kernel reads the same keys in the same tile order as the contiguous call."""
    import grouped_query_exact_amd as g
    B, Sk, Hq, Hk, d, ps = 4, 1000, 32, 8, 128, 64
    P = -(-Sk // ps)
    q, k, v = gi.random_bf16(7300, (B, 1, Hq, d)), gi.random_bf16(7301, (B, Sk, Hk, d)), gi.random_bf16(7302, (B, Sk, Hk, d))
    kc = torch.zeros((B * P, ps, Hk, d), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc.view(B, P * ps, Hk, d)[:, :Sk] = k
    vc.view(B, P * ps, Hk, d)[:, :Sk] = v
    kv = gi.PagedKV(kc, vc, torch.arange(B * P, dtype=torch.int32).view(B, P), torch.full((B,), Sk, dtype=torch.int32))
    for causal in (False, True):
        for ns in (1, 4):
            Op, Lp = run_paged(q, kv, causal, 0.0883883461356163, 1, ns)
            out = torch.empty((B, 1, Hq, d), dtype=torch.bfloat16, device=DEV)
            lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=DEV)
            g.gqa_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, causal, 0.0883883461356163, 1, ns)
            torch.cuda.synchronize()
            assert torch.equal(Op, out) and torch.equal(Lp, lse), f"causal={causal} ns={ns}"


def test_paged_decode_full_size_sampled():
    """The decode workload's shape (B=64, Hq=32, Hk=8, d=128) with sequence lengths up to 8192
    in pages of 256 keys, library's choice of pack and splits; oracle on 6 sampled sequences."""
    rs = np.random.RandomState(7400)
    lens = [int(x) for x in rs.randint(1, 8193, size=64)]
    lens[0], lens[1] = 8192, 1
    kv = gi.paged_kv(7400, lens, 256, 8, 128, spare_pages=5)
    q = gi.random_bf16(7401, (64, 1, 32, 128))
    O, L = run_paged(q, kv, False, gi.fp32(1 / math.sqrt(128)))
    assert torch.isfinite(O.float()).all()
    compare_paged(O, L, q, kv, False, gi.fp32(1 / math.sqrt(128)), batches=[0, 1, 17, 33, 48, 63], tag="full size")


def test_paged_decode_many_split_workgroups():
    """Paged decode with many more split workgroups than the GPU keeps resident (48 x 8 x 20),
    pages of 16 keys in random pool order: bit for bit the contiguous call at the same splits."""
    import grouped_query_exact_amd as g
    B, Sq, Hq, Hk, d, ps = 48, 1, 32, 8, 128, 16
    lens = [700 + 13 * b for b in range(B)]
    kv = gi.paged_kv(7700, lens, ps, Hk, d).to(DEV)
    q = gi.random_bf16(7701, (B, Sq, Hq, d)).to(DEV)
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (False, True):
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd_paged(q, kv.k_cache, kv.v_cache, kv.block_table, kv.seqlens_k, out, lse, causal, scale, 1, 20)
        torch.cuda.synchronize()
        for b in (0, 23, 47):
            kb, vb = gi.batch_slice(7700, b, 1, lens[b], Hq, Hk, d)[1:]
            ob = torch.empty((1, Sq, Hq, d), dtype=torch.bfloat16, device=DEV)
            lb = torch.empty((1, Hq, Sq), dtype=torch.float32, device=DEV)
            g.gqa_attn_fwd(q[b:b + 1], kb[None].to(DEV), vb[None].to(DEV), ob, lb, causal, scale, 1, 20)
            torch.cuda.synchronize()
            assert torch.equal(out[b:b + 1], ob) and torch.equal(lse[b:b + 1], lb), f"b={b} causal={causal}"


@pytest.mark.parametrize("Sq", [1, 40])
def test_paged_malformed_tables_stay_in_the_pool(Sq):
    """Block-table entries below 0 or past the pool and key lengths below 0 or past the table's
    capacity: the kernels clamp pages into [0, num_pages) and lengths into [0, capacity], so every
    read stays in the pool. The pool sits between NaN guard pages and holds only finite values, so
    a read outside it would show up as a non-finite output. Decode (Sq=1) and chunked prefill (40
    new tokens), bf16 and fp8 pools, causal and not, unsplit and split."""
    import grouped_query_exact_amd as g
    B, Hq, Hk, d, ps, max_pages, num_pages, gp = 6, 8, 2, 128, 32, 6, 10, 3
    rs = np.random.default_rng(77)
    table = torch.from_numpy(rs.integers(-4, num_pages + 4, (B, max_pages)).astype(np.int32)).to(DEV)
    seqlens = torch.tensor([-7, 0, 5, 100, max_pages * ps, max_pages * ps + 500], dtype=torch.int32, device=DEV)
    q = gi.random_bf16(9960, (B, Sq, Hq, d)).to(DEV)
    scale = gi.fp32(1 / math.sqrt(d))
    for fp8 in (False, True):
        if fp8 and Sq > 1:
            continue  # fp8 pools take decode-shaped calls only
        dt = torch.uint8 if fp8 else torch.bfloat16
        pools = []
        for seed in (9961, 9962):
            big = torch.full((num_pages + 2 * gp, ps, Hk, d), float("nan"), dtype=torch.float32, device=DEV)
            big[gp:gp + num_pages] = gi.random_bf16(seed, (num_pages, ps, Hk, d)).float().to(DEV)
            big = big.to(torch.float8_e4m3fn).view(torch.uint8) if fp8 else big.to(torch.bfloat16)
            assert big.dtype == dt
            pools.append(big[gp:gp + num_pages])
        kc, vc = pools
        for causal in (False, True):
            for ns in (1, 3):
                out = torch.empty_like(q)
                lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
                if fp8:
                    g.gqa_attn_fwd_paged_kv8(q, kc, vc, 1.0, 1.0, table, seqlens, out, lse, causal, scale, -1, ns)
                else:
                    g.gqa_attn_fwd_paged(q, kc, vc, table, seqlens, out, lse, causal, scale, -1, ns)
                torch.cuda.synchronize()
                tag = f"Sq={Sq} fp8={fp8} causal={causal} ns={ns}"
                assert torch.isfinite(out.float()).all(), f"{tag}: a read left the pool"
                assert not torch.isnan(lse).any(), tag
                # the two sequences without keys (length <= 0) give O = 0
                assert torch.all(out[:2].float() == 0), tag
