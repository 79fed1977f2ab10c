"""Long sequences against the fp64 oracle (GPU).

The largest key and row counts the other tests reach are a few thousand. Here:
a causal prefill of 32768 tokens (8-wavefront kernel, 512 key tiles per row
tile at the end, checked on sampled rows including the last ones), decode
against 131072 keys (decode kernel, automatic and single split), and a chunk
of 128 new tokens against a 65536-key context (split keys and the combine,
bottom-right causal alignment), checked on every row.
"""

import math
import random

import pytest

import gqa_inputs as gi
from _parity import compare_to_oracle, gpu_run

pytestmark = pytest.mark.gpu


def _qkv(seed, B, Sq, Sk, Hq, Hk, d):
    return (gi.random_bf16(seed, (B, Sq, Hq, d)), gi.random_bf16(seed + 1, (B, Sk, Hk, d)),
            gi.random_bf16(seed + 2, (B, Sk, Hk, d)))


def test_prefill_causal_32k():
    import grouped_query_exact_amd as g
    B, S, Hq, Hk, d = 1, 32768, 32, 8, 128
    assert g.gqa_attn_plan(B, S, S, Hq, Hk, d, True, -1, 0, 0)["threads"] == 512
    q, k, v = _qkv(9500, B, S, S, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    O, L = gpu_run(q, k, v, True, scale, -1, 0)
    rows = sorted({0, 1, 63, 64, 255, 256, 16383, 16384, S - 65, S - 64, S - 2, S - 1}
                  | set(random.Random(5).sample(range(S), 12)))
    compare_to_oracle(O, L, q, k, v, True, scale, heads=[0, 3, 4, 31], rows=rows, tag="causal 32k")


@pytest.mark.parametrize("ns", [0, 1])
def test_decode_128k_keys(ns):
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d = 4, 1, 131072, 32, 8, 128
    plan = g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, False, -1, ns, 0)
    assert plan["block_m"] == 32 and (ns == 1) == (plan["num_splits"] == 1), plan
    q, k, v = _qkv(9520, B, Sq, Sk, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    O, L = gpu_run(q, k, v, False, scale, -1, ns)
    compare_to_oracle(O, L, q, k, v, False, scale, tag=f"decode 128k ns={plan['num_splits']}")


def test_chunk_against_64k_context():
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d = 1, 128, 65536, 32, 8, 128
    plan = g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, True, -1, 0, 0)
    assert plan["num_splits"] > 1 and plan["threads"] == 256, plan
    q, k, v = _qkv(9540, B, Sq, Sk, Hq, Hk, d)
    scale = gi.fp32(1 / math.sqrt(d))
    O, L = gpu_run(q, k, v, True, scale, -1, 0)
    compare_to_oracle(O, L, q, k, v, True, scale, tag=f"chunk vs 64k ns={plan['num_splits']}")
