"""The decode kernel (at most 32 query rows per head unit) against the fp64 oracle (GPU).

Decode-shaped work -- one or a few new tokens per sequence against a long KV
cache, the pages' memory-bound regime -- runs on its own kernel: one
wavefront per workgroup, 32-key tiles, a ring of LDS stages. These cases
cover what is particular to it: the ring's head and tail (splits of 1 to 5
tiles), ragged key lengths around the 32-key tile, the 32-row capacity on
both sides of the boundary with the tiled kernel, causal rows that see no key
at all, both head dimensions and every split count up to one tile per split.
"""

import math

import pytest
import torch

import gqa_inputs as gi
from _parity import assert_variants_agree, compare_to_oracle, gpu_run

pytestmark = pytest.mark.gpu


def _qkv(seed, B, Sq, Sk, Hq, Hk, d):
    return (gi.random_bf16(seed, (B, Sq, Hq, d)), gi.random_bf16(seed + 1, (B, Sk, Hk, d)),
            gi.random_bf16(seed + 2, (B, Sk, Hk, d)))


def _plan(q, k, causal, pack, ns):
    import grouped_query_exact_amd as g
    B, Sq, Hq, d = q.shape
    Sk, Hk = k.shape[1], k.shape[2]
    return g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, causal, pack, ns, 256)


# Sk around the 32-key tile: 1 .. 5 tiles, full and ragged last tiles
SK_RING = [1, 31, 32, 33, 64, 95, 96, 97, 160, 161]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sk", SK_RING)
def test_one_token_ring_head_and_tail(d, Sk):
    """One new token of 3 groups of 4 heads: every tile count of the ring, causal and not, ns 1 and 2."""
    q, k, v = _qkv(9000 + Sk + d, 2, 1, Sk, 12, 3, d)
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (False, True):
        for ns in (1, 2):
            plan = _plan(q, k, causal, 1, ns)
            assert plan["block_m"] == 32 and plan["block_n"] == 32
            O, L = gpu_run(q, k, v, causal, scale, 1, ns)
            compare_to_oracle(O, L, q, k, v, causal, scale, tag=f"d={d} Sk={Sk} causal={causal} ns={ns}")


@pytest.mark.parametrize("Sq,G,pack", [(8, 4, 1), (4, 8, 1), (32, 4, 0), (3, 3, 1), (2, 1, 0)])
def test_rows_up_to_capacity(Sq, G, pack):
    """Up to 32 rows per head unit (packed and not), causal with Sq > 1, ragged Sk, several splits."""
    Hk = 2
    for Sk in (40, 129, 1000):
        q, k, v = _qkv(9100 + Sq * 10 + G + Sk, 2, Sq, Sk, G * Hk, Hk, 64 if Sq % 2 else 128)
        d = q.shape[-1]
        scale = gi.fp32(1 / math.sqrt(d))
        for causal in (False, True):
            for ns in (1, 3, 7):
                plan = _plan(q, k, causal, pack, ns)
                assert plan["block_m"] == 32, plan
                O, L = gpu_run(q, k, v, causal, scale, pack, ns)
                compare_to_oracle(O, L, q, k, v, causal, scale,
                                  tag=f"Sq={Sq} G={G} pack={pack} Sk={Sk} causal={causal} ns={ns}")


def test_capacity_boundary_between_kernels():
    """Sq=9, G=4: packed rows (36) go to the tiled kernel, unpacked rows (9) to the decode
    kernel; both match the oracle and agree with each other within the variant bound."""
    q, k, v = _qkv(9200, 3, 9, 700, 16, 4, 128)
    scale = gi.fp32(1 / math.sqrt(128))
    for causal in (False, True):
        assert _plan(q, k, causal, 1, 1)["block_m"] == 128
        assert _plan(q, k, causal, 0, 1)["block_m"] == 32
        Ot, Lt = gpu_run(q, k, v, causal, scale, 1, 1)
        Od, Ld = gpu_run(q, k, v, causal, scale, 0, 1)
        compare_to_oracle(Ot, Lt, q, k, v, causal, scale, tag=f"tiled causal={causal}")
        compare_to_oracle(Od, Ld, q, k, v, causal, scale, tag=f"decode causal={causal}")
        assert_variants_agree(Ot, Lt, Od, Ld, float(v.float().abs().max()), tag=f"tiled vs decode causal={causal}")


def test_causal_rows_that_see_no_key():
    """Bottom-right causal with Sq > Sk: the first Sq - Sk tokens see no key (O = 0, LSE = -inf)."""
    q, k, v = _qkv(9300, 2, 8, 3, 8, 2, 64)
    for pack, ns in ((1, 1), (0, 1), (1, 2)):
        O, L = gpu_run(q, k, v, True, 0.125, pack, ns)
        compare_to_oracle(O, L, q, k, v, True, 0.125, tag=f"pack={pack} ns={ns}")
        assert torch.all(O[:, :5].float() == 0)
        assert torch.all(torch.isneginf(L[:, :, :5]))
        assert torch.all(torch.isfinite(L[:, :, 5:]))


def test_one_tile_per_split():
    """As many splits as tiles (every split holds exactly one tile), and more splits than tiles."""
    q, k, v = _qkv(9400, 1, 1, 32 * 16, 8, 2, 128)
    scale = gi.fp32(1 / math.sqrt(128))
    for ns in (16, 40):
        plan = _plan(q, k, False, 1, ns)
        assert plan["num_splits"] == 16
        O, L = gpu_run(q, k, v, False, scale, 1, ns)
        compare_to_oracle(O, L, q, k, v, False, scale, tag=f"ns={ns}")


@pytest.mark.parametrize("d", [64, 128])
def test_many_splits(d):
    """Split counts on both sides of the switch to the one-workgroup-per-row merge
    (16 splits): 15, 16, 64, one 32-key tile per split (129) and more splits than
    tiles (200, clamped to 129); one and four new tokens, causal and not."""
    import grouped_query_exact_amd as g
    B, Hq, Hk, Sk = 2, 8, 2, 4096 + 7
    scale = gi.fp32(1 / math.sqrt(d))
    for Sq in (1, 4):
        q, k, v = _qkv(9600 + d + Sq, B, Sq, Sk, Hq, Hk, d)
        for causal in (False, True):
            for ns in (15, 16, 64, 129, 200):
                plan = _plan(q, k, causal, 1, ns)
                assert plan["block_m"] == 32 and plan["num_splits"] == min(ns, 129), plan
                O, L = gpu_run(q, k, v, causal, scale, 1, ns)
                compare_to_oracle(O, L, q, k, v, causal, scale, tag=f"d={d} Sq={Sq} causal={causal} ns={ns}")


@pytest.mark.parametrize("d", [64, 128])
def test_many_splits_tiled_empty_rows(d):
    """The tiled kernel split 16 and 33 ways (one 64-key tile per split) with causal
    rows for which the last splits hold no visible key, and -- with more query
    tokens than keys -- rows that see no key in any split (O = 0, LSE = -inf)."""
    B, Hq, Hk = 1, 4, 1
    scale = gi.fp32(1 / math.sqrt(d))
    for Sq, Sk in ((300, 2048 + 13), (2100, 2061)):
        q, k, v = _qkv(9650 + d + Sq, B, Sq, Sk, Hq, Hk, d)
        for ns in (16, 33):
            plan = _plan(q, k, True, 0, ns)
            assert plan["block_m"] != 32 and plan["num_splits"] == ns, plan
            O, L = gpu_run(q, k, v, True, scale, 0, ns)
            compare_to_oracle(O, L, q, k, v, True, scale, tag=f"d={d} Sq={Sq} Sk={Sk} ns={ns}")
            if Sq > Sk:
                dead = Sq - Sk
                assert torch.all(O[:, :dead].float() == 0)
                assert torch.all(torch.isneginf(L[:, :, :dead]))
                assert torch.all(torch.isfinite(L[:, :, dead:]))


def _many_items_check(O, L, Or, Lr, vmax, tag):
    """A launch of many split workgroups against the same call unsplit: the strict variant gate."""
    assert_variants_agree(Or, Lr, O, L, vmax, tag=tag, strict=True)


@pytest.mark.parametrize("d", [64, 128])
def test_many_split_workgroups(d):
    """Many more (head unit, split) workgroups than the GPU keeps resident (64 sequences x 8 KV
    groups x 16 splits = 8192, up to 47 splits): against the oracle and, strictly, the unsplit call;
    causal and not, pack on and off."""
    B, Sq, Sk, Hq, Hk = 64, 1, 1500, 32, 8
    q, k, v = _qkv(9900 + d, B, Sq, Sk, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    vmax = float(v.float().abs().max())
    for causal in (False, True):
        Or, Lr = gpu_run(q, k, v, causal, scale, 1, 1)
        compare_to_oracle(Or, Lr, q, k, v, causal, scale, batches=[0, 37, 63], tag=f"d={d} unsplit")
        for pack, ns in ((1, 16), (0, 3), (1, 47)):
            O, L = gpu_run(q, k, v, causal, scale, pack, ns)
            compare_to_oracle(O, L, q, k, v, causal, scale, batches=[0, 37, 63], tag=f"d={d} pack={pack} ns={ns}")
            _many_items_check(O, L, Or, Lr, vmax, f"d={d} causal={causal} pack={pack} ns={ns}")


def test_many_splits_varlen_with_empty_sequences():
    """Variable-length decode with empty key and query sequences among many split workgroups."""
    import grouped_query_exact_amd as g
    import oracle
    import numpy as np
    rs = np.random.default_rng(5)
    lk = [int(x) for x in rs.integers(0, 3000, 96)]
    lk[3] = 0
    lk[50] = 0
    lq = [1 + (b % 3) for b in range(96)]
    lq[7] = 0
    Hq, Hk, d = 32, 8, 128
    q, k, v, cq, ck = gi.varlen_batch(9950, lq, lk, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    res = {}
    for ns in (1, 9, 24):
        out = torch.full((q.shape[0], Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.full((Hq, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda:0")
        g.gqa_attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), out, lse, cq.cuda(), ck.cuda(), max(lq), max(lk), True,
                              scale, 1, ns)
        torch.cuda.synchronize()
        res[ns] = (out, lse)
        Or, Lr = oracle.attention_varlen_fp64(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                              cq.tolist(), ck.tolist(), True, scale, sequences=[0, 3, 7, 50, 95])
        cols = np.concatenate([np.arange(int(cq[b]), int(cq[b + 1])) for b in (0, 3, 7, 50, 95)])
        Og = out.double().cpu().numpy()[cols]
        assert np.abs(Og - Or[cols]).max() <= 2e-2, f"ns={ns}"
        fin = np.isfinite(Lr[:, cols])
        Lg = lse.double().cpu().numpy()[:, cols]
        assert np.array_equal(fin, np.isfinite(Lg)) and np.abs(Lg[fin] - Lr[:, cols][fin]).max() <= 1e-3, f"ns={ns}"
    for ns in (9, 24):
        assert_variants_agree(res[1][0].unsqueeze(0), None, res[ns][0].unsqueeze(0), None,
                              float(v.float().abs().max()), tag=f"varlen ns={ns}", strict=True)
