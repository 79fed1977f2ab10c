"""Variable-length (packed) batches, gqa_attn_fwd_varlen, against the fp64 oracle (GPU).

Cases: prefill length mixes around the 128-row and 64-key tiles with empty
sequences, causal and not, both packings, splits and both head dimensions;
chunked prefill (fewer queries than keys, per-sequence bottom-right
alignment); decode-shaped batches (one or a few new tokens per sequence) on
the decode kernel; equal lengths against the batched call (bit for bit);
and a Llama-2-shaped mix of long sequences on sampled rows.
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


def run_varlen(q, k, v, cq, ck, causal, scale, pack=-1, ns=0):
    import grouped_query_exact_amd as g
    total_q, Hq, d = q.shape
    lq = (cq[1:] - cq[:-1]).tolist()
    lk = (ck[1:] - ck[:-1]).tolist()
    out = torch.empty((total_q, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=DEV)
    g.gqa_attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, cq.to(DEV), ck.to(DEV), max(lq), max(max(lk), 1),
                          causal, scale, pack, ns)
    torch.cuda.synchronize()
    return out, lse


def check(O, L, q, k, v, cq, ck, causal, scale, sequences=None, tag=""):
    Or, Lr = oracle.attention_varlen_fp64(f64(q), f64(k), f64(v), cq.tolist(), ck.tolist(), causal, scale,
                                          sequences=sequences)
    cols = slice(None)
    if sequences is not None:
        cols = np.concatenate([np.arange(int(cq[b]), int(cq[b + 1])) for b in sequences])
    Og, Lg = f64(O)[cols], f64(L)[:, cols]
    Or, Lr = Or[cols], Lr[:, cols]
    assert np.isfinite(Og).all(), f"{tag}: non-finite output"
    dO = np.abs(Og - Or)
    assert dO.max() <= TOL_O_MAX and dO.mean() <= TOL_O_MEAN, f"{tag}: max {dO.max()} mean {dO.mean()}"
    fin = np.isfinite(Lr)
    assert np.array_equal(fin, np.isfinite(Lg)), f"{tag}: LSE -inf pattern"
    if fin.any():
        assert np.abs(Lg[fin] - Lr[fin]).max() <= TOL_LSE, f"{tag}: LSE"


MIX = [1, 77, 128, 0, 129, 300, 513]


@pytest.mark.parametrize("G,d", [(4, 128), (3, 64)])
def test_varlen_prefill_mix(G, d):
    Hk = 2
    q, k, v, cq, ck = gi.varlen_batch(9000 + G + d, MIX, MIX, G * Hk, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (False, True):
        for pack, ns in ((1, 1), (0, 1), (1, 3), (-1, 0)):
            O, L = run_varlen(q, k, v, cq, ck, causal, scale, pack, ns)
            check(O, L, q, k, v, cq, ck, causal, scale, tag=f"G={G} d={d} causal={causal} pack={pack} ns={ns}")


def test_varlen_chunked_prefill():
    """Fewer queries than keys (a new chunk against its cached prefix), and a sequence without keys."""
    lq, lk = [5, 64, 200, 3, 9], [100, 64, 700, 0, 1]
    q, k, v, cq, ck = gi.varlen_batch(9100, lq, lk, 8, 2, 128)
    scale = gi.fp32(1 / math.sqrt(128))
    for causal in (False, True):
        for pack, ns in ((1, 1), (1, 4), (0, 2)):
            O, L = run_varlen(q, k, v, cq, ck, causal, scale, pack, ns)
            check(O, L, q, k, v, cq, ck, causal, scale, tag=f"causal={causal} pack={pack} ns={ns}")
            assert torch.all(O[cq[3]:cq[4]].float() == 0) and torch.all(torch.isneginf(L[:, cq[3]:cq[4]]))


def test_varlen_decode_shaped():
    """One or a few new tokens per sequence (packed rows <= 32: the decode kernel)."""
    import grouped_query_exact_amd as g
    lk = [1, 31, 32, 33, 500, 2000, 0, 64]
    for nq in (1, 4):
        lq = [nq] * len(lk)
        q, k, v, cq, ck = gi.varlen_batch(9200 + nq, lq, lk, 32, 8, 128)
        assert g.gqa_attn_plan(len(lk), nq, max(lk), 32, 8, 128, True, -1, 0, 256)["block_m"] == 32
        scale = gi.fp32(1 / math.sqrt(128))
        for causal in (False, True):
            for ns in (0, 1, 3):
                O, L = run_varlen(q, k, v, cq, ck, causal, scale, -1, ns)
                check(O, L, q, k, v, cq, ck, causal, scale, tag=f"nq={nq} causal={causal} ns={ns}")


def test_varlen_equal_lengths_match_batched_bitwise():
    import grouped_query_exact_amd as g
    B, S, Hq, Hk, d = 3, 300, 8, 2, 128
    q, k, v, cq, ck = gi.varlen_batch(9300, [S] * B, [S] * B, Hq, Hk, d)
    for causal in (False, True):
        for pack, ns in ((1, 1), (0, 2)):
            O, L = run_varlen(q, k, v, cq, ck, causal, 0.0883883461356163, pack, ns)
            ob = torch.empty((B, S, Hq, d), dtype=torch.bfloat16, device=DEV)
            lb = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
            g.gqa_attn_fwd(q.view(B, S, Hq, d).to(DEV), k.view(B, S, Hk, d).to(DEV), v.view(B, S, Hk, d).to(DEV), ob, lb,
                           causal, 0.0883883461356163, pack, ns)
            torch.cuda.synchronize()
            assert torch.equal(O.view(B, S, Hq, d), ob), f"O causal={causal} pack={pack} ns={ns}"
            assert torch.equal(L, lb.permute(1, 0, 2).reshape(Hq, B * S)), f"LSE causal={causal} pack={pack} ns={ns}"


def test_varlen_llama_mix_sampled():
    """Hq=32, Hk=8, d=128, causal, eight sequences of 33 to 2048 tokens; oracle on four of them."""
    lens = [2048, 1500, 1000, 700, 512, 300, 100, 33]
    q, k, v, cq, ck = gi.varlen_batch(9400, lens, lens, 32, 8, 128)
    scale = gi.fp32(1 / math.sqrt(128))
    O, L = run_varlen(q, k, v, cq, ck, True, scale)
    assert torch.isfinite(O.float()).all()
    check(O, L, q, k, v, cq, ck, True, scale, sequences=[1, 4, 6, 7], tag="llama mix")


@pytest.mark.parametrize("lq,lk,max_sq", [([40, 100, 7], [1100, 1200, 50], 64),   # tiled kernel
                                          ([1, 3, 2], [700, 1500, 90], 2)])        # decode kernel
def test_varlen_split_leaves_unwritten_tokens_untouched(lq, lk, max_sq):
    """Tokens past max_seqlen_q of a longer sequence and padding tokens after the last
    sequence are written by no path: unsplit, split with the per-row combine, or split
    with the one-workgroup-per-row combine (>= 16 splits). NaN guard values stay."""
    import grouped_query_exact_amd as g
    Hq, Hk, d, pad = 8, 2, 64, 13
    q, k, v, cq, ck = gi.varlen_batch(9500 + max_sq, lq, lk, Hq, Hk, d)
    total_q = int(cq[-1]) + pad
    qp = torch.cat([q, gi.random_bf16(9599, (pad, Hq, d))]).to(DEV)
    written = torch.zeros(total_q, dtype=torch.bool)
    for b, n in enumerate(lq):
        written[int(cq[b]):int(cq[b]) + min(n, max_sq)] = True
    scale = gi.fp32(1 / math.sqrt(d))
    for causal in (False, True):
        for ns in (1, 3, 17):
            out = torch.full((total_q, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
            lse = torch.full((Hq, total_q), float("nan"), dtype=torch.float32, device=DEV)
            g.gqa_attn_fwd_varlen(qp, k.to(DEV), v.to(DEV), out, lse, cq.to(DEV), ck.to(DEV), max_sq, max(lk), causal,
                                  scale, 1, ns)
            torch.cuda.synchronize()
            tag = f"lq={lq} causal={causal} ns={ns}"
            assert torch.isnan(out[~written.to(DEV)].float()).all(), f"{tag}: unwritten tokens were written"
            assert torch.isnan(lse[:, ~written.to(DEV)]).all(), f"{tag}: unwritten LSE entries were written"
            assert torch.isfinite(out[written.to(DEV)].float()).all(), f"{tag}: written tokens not finite"
            ok = [b for b, n in enumerate(lq) if n <= max_sq]  # sequences within max_seqlen_q: exact results
            check(out, lse, q, k, v, cq, ck, causal, scale, sequences=ok, tag=tag)



def test_varlen_work_list_many_sequences():
    """1500 short sequences (more than the scheduling kernel's 1024 threads), empty ones, and one
    sequence whose 70000 keys put its row tiles in the top cost bin; causal with more keys than
    queries, splits and not. Sampled sequences against the oracle."""
    import numpy as np
    rs = np.random.default_rng(12)
    B = 1500
    lq = [int(x) for x in rs.integers(0, 61, B)]
    lk = [n + int(x) for n, x in zip(lq, rs.integers(0, 101, B))]
    lq[10], lk[10] = 0, 0
    lq[11] = 0
    lq[700], lk[700] = 100, 70000
    q, k, v, cq, ck = gi.varlen_batch(9700, lq, lk, 8, 2, 64)
    scale = gi.fp32(1 / math.sqrt(64))
    sel = [0, 10, 11, 12, 700, 1023, 1024, 1499]
    for causal in (False, True):
        for pack, ns in ((1, 1), (1, 3)):
            O, L = run_varlen(q, k, v, cq, ck, causal, scale, pack, ns)
            check(O, L, q, k, v, cq, ck, causal, scale, sequences=sel, tag=f"causal={causal} ns={ns}")


@pytest.mark.parametrize("lens", [[300, 280, 290, 120],    # >= 3/4 of B * max_seqlen_q tokens: the plain grid
                                  [300, 20, 290, 1]])      # fewer: the work list
def test_varlen_grid_and_work_list_paths(lens):
    """Both ways of laying out variable-length prefill items, causal and not, both packings
    and a split, against the oracle on every sequence."""
    q, k, v, cq, ck = gi.varlen_batch(9800 + len(lens) + lens[1], lens, lens, 8, 2, 128)
    scale = gi.fp32(1 / math.sqrt(128))
    for causal in (False, True):
        for pack, ns in ((1, 1), (0, 1), (1, 2)):
            O, L = run_varlen(q, k, v, cq, ck, causal, scale, pack, ns)
            check(O, L, q, k, v, cq, ck, causal, scale, tag=f"lens={lens} causal={causal} pack={pack} ns={ns}")


def test_varlen_llama_mix_8_wavefront_kernel_full():
    """Llama-2 heads, 16 sequences of 40 to 940 tokens: the work list on the 8-wavefront kernel
    (enough 256-row items); every sequence against the oracle."""
    lens = [40 + 60 * i for i in range(16)]
    q, k, v, cq, ck = gi.varlen_batch(9900, lens, lens, 32, 8, 128)
    scale = gi.fp32(1 / math.sqrt(128))
    for causal in (True, False):
        O, L = run_varlen(q, k, v, cq, ck, causal, scale)
        check(O, L, q, k, v, cq, ck, causal, scale, tag=f"causal={causal}")


def test_varlen_8_wavefront_pairs_unequal_key_counts():
    """Causal calls on the 8-wavefront kernel take pairs of a sequence's row tiles (R-1-i and i)
    from the work list. Sequences of 40 to 940 tokens (one to 15 row tiles, odd and even) with
    300 cached keys before the chunk, half as many keys as queries (the first rows see no key)
    or as many; every sequence against the oracle."""
    lq = [40 + 60 * i for i in range(16)]
    lk = [n + 300 if i % 3 == 0 else (n // 2 if i % 3 == 1 else n) for i, n in enumerate(lq)]
    q, k, v, cq, ck = gi.varlen_batch(9905, lq, lk, 32, 8, 128)
    scale = gi.fp32(1 / math.sqrt(128))
    O, L = run_varlen(q, k, v, cq, ck, True, scale)
    check(O, L, q, k, v, cq, ck, True, scale, tag="causal pairs, unequal key counts")


@pytest.mark.parametrize("shape", ["small", "8-wavefront"])
def test_varlen_malformed_offsets_stay_in_bounds(shape):
    """Offsets that decrease, overlap, start below 0 or run past total_q/total_k: the kernels
    clamp every sequence into [0, total_q) x [0, total_k), so the call succeeds and nothing
    outside out and lse is written (guard rows around them keep their NaNs). Results for such
    offsets are unspecified; each path (plain grid, work list, splits) must stay in bounds."""
    import grouped_query_exact_amd as g
    if shape == "small":
        Hq, Hk, d, total_q, total_k, max_sq, max_sk = 8, 2, 128, 300, 400, 128, 400
        cqs = [[0, 100, 50, 300], [-20, 250, 1000, 1000], [0, 300, 300, 300]]
        cks = [[0, 150, 100, 400], [-5, 200, 5000, 7], [0, 0, 400, 10]]
    else:  # enough 256-row items for the 8-wavefront kernel with a work list
        Hq, Hk, d, total_q, total_k, max_sq, max_sk = 32, 8, 128, 8192, 8192, 512, 1024
        B = 64
        base = np.linspace(0, total_q, B + 1).astype(int)
        bad_q = base.copy(); bad_q[10] = base[30]; bad_q[40] = -100; bad_q[B] = total_q + 900
        bad_k = base.copy(); bad_k[5] = base[9]; bad_k[20] = total_k + 50
        cqs, cks = [bad_q.tolist()], [bad_k.tolist()]
    q = gi.random_bf16(9950, (total_q, Hq, d)).to(DEV)
    k = gi.random_bf16(9951, (total_k, Hk, d)).to(DEV)
    v = gi.random_bf16(9952, (total_k, Hk, d)).to(DEV)
    scale = gi.fp32(1 / math.sqrt(d))
    pad = 48
    for cq, ck in zip(cqs, cks):
        cq_t = torch.tensor(cq, dtype=torch.int32, device=DEV)
        ck_t = torch.tensor(ck, dtype=torch.int32, device=DEV)
        for causal in (False, True):
            for pack, ns in ((1, 1), (0, 1), (1, 3), (-1, 0)):
                big_o = torch.full((total_q + 2 * pad, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
                big_l = torch.full((Hq * total_q + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
                out = big_o[pad:pad + total_q]
                lse = big_l[pad:pad + Hq * total_q].view(Hq, total_q)
                g.gqa_attn_fwd_varlen(q, k, v, out, lse, cq_t, ck_t, max_sq, max_sk, causal, scale, pack, ns)
                torch.cuda.synchronize()
                tag = f"{shape} cq={cq[:4]} causal={causal} pack={pack} ns={ns}"
                assert torch.isnan(big_o[:pad].float()).all() and torch.isnan(big_o[pad + total_q:].float()).all(), tag
                assert torch.isnan(big_l[:pad]).all() and torch.isnan(big_l[pad + Hq * total_q:]).all(), tag


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_work_list_equals_plain_grid_bitwise(d):
    """The same sequences called with max_seqlen_q = the longest sequence (tokens fill over 3/4 of
    the grid: the plain grid) and with a larger bound (the work list): the tiled kernel's per-row
    arithmetic does not depend on the order it takes the items in, so outputs and LSE are equal
    bit for bit, unsplit and split."""
    import grouped_query_exact_amd as g
    lens = [300, 280, 290, 120]
    Hq, Hk = 6, 2
    q, k, v, cq, ck = gi.varlen_batch(9990 + d, lens, lens, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    total = sum(lens)
    for causal in (False, True):
        for pack, ns in ((1, 1), (0, 1), (1, 3)):
            res = []
            for max_q in (max(lens), 2 * max(lens)):
                out = torch.empty((total, Hq, d), dtype=torch.bfloat16, device=DEV)
                lse = torch.empty((Hq, total), dtype=torch.float32, device=DEV)
                g.gqa_attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, cq.to(DEV), ck.to(DEV), max_q,
                                      max(lens), causal, scale, pack, ns)
                torch.cuda.synchronize()
                res.append((out, lse))
            tag = f"d={d} causal={causal} pack={pack} ns={ns}"
            assert torch.equal(res[0][0], res[1][0]), f"{tag}: O"
            assert torch.equal(res[0][1], res[1][1]), f"{tag}: LSE"


def test_varlen_8_wavefront_work_list_equals_batched_bitwise():
    """Eight sequences of 2048 tokens (Llama-2 heads, causal and not): the batched call runs on the
    8-wavefront kernel's plain grid; the same tokens as a variable-length call with max_seqlen_q =
    4096 run on that kernel from the work list. Same per-row arithmetic: equal bit for bit."""
    import grouped_query_exact_amd as g
    B, S, Hq, Hk, d = 8, 2048, 32, 8, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9995)
    q = torch.randn((B, S, Hq, d), generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, S, Hk, d), generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, S, Hk, d), generator=gen, device=DEV).to(torch.bfloat16)
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device=DEV)
    scale = gi.fp32(1 / math.sqrt(d))
    assert g.gqa_attn_plan(B, S, S, Hq, Hk, d, True, -1, 0, 256)["threads"] == 512  # 8-wavefront kernel
    for causal in (True, False):
        ob = torch.empty_like(q)
        lb = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd(q, k, v, ob, lb, causal, scale)
        ov = torch.empty((B * S, Hq, d), dtype=torch.bfloat16, device=DEV)
        lv = torch.empty((Hq, B * S), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd_varlen(q.view(B * S, Hq, d), k.view(B * S, Hk, d), v.view(B * S, Hk, d), ov, lv, cu, cu,
                              2 * S, S, causal, scale)
        torch.cuda.synchronize()
        assert torch.equal(ov.view(B, S, Hq, d), ob), f"O causal={causal}"
        assert torch.equal(lv, lb.permute(1, 0, 2).reshape(Hq, B * S)), f"LSE causal={causal}"
