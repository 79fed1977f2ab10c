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
