"""Forward calls captured in a HIP graph (GPU).

An unsplit forward call launches one kernel on the caller's stream and makes
no allocation, memset or synchronisation, so it can be captured. Each graph
is replayed several times; between replays the inputs are rewritten in place
and eager work runs on the same stream, and every replay must equal, bit for
bit, an eager call on the inputs it saw. Covered: the 4-wavefront tiled
kernel, the 8-wavefront prefill kernel and the decode kernel.
"""

import math

import pytest
import torch

import gqa_inputs as gi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, Sq, Sk, Hq, Hk, d, causal, threads of the kernel the plan picks)
CASES = [
    (2, 300, 300, 8, 2, 128, True, 256),   # 4-wavefront tiled kernel
    (64, 256, 256, 8, 2, 128, True, 512),  # 8-wavefront prefill kernel
    (16, 1, 1000, 32, 8, 128, False, 64),  # decode kernel
]


@pytest.mark.parametrize("case", CASES, ids=[f"threads{c[-1]}" for c in CASES])
def test_forward_graph_replays(case):
    import grouped_query_exact_amd as g
    B, Sq, Sk, Hq, Hk, d, causal, threads = case
    assert g.gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, causal, 1, 1, 0)["threads"] == threads
    scale = gi.fp32(1 / math.sqrt(d))
    q = gi.random_bf16(9600, (B, Sq, Hq, d)).to(DEV)
    k = gi.random_bf16(9601, (B, Sk, Hk, d)).to(DEV)
    v = gi.random_bf16(9602, (B, Sk, Hk, d)).to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)

    def eager(qx, kx, vx):
        o = torch.empty_like(qx)
        l = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
        g.gqa_attn_fwd(qx, kx, vx, o, l, causal, scale, 1, 1)
        torch.cuda.synchronize()
        return o, l

    g.gqa_attn_fwd(q, k, v, out, lse, causal, scale, 1, 1)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            g.gqa_attn_fwd(q, k, v, out, lse, causal, scale, 1, 1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        # new inputs in place, then eager work on the same stream before the replay
        q.copy_(gi.random_bf16(9610 + rep, (B, Sq, Hq, d)).to(DEV))
        v.mul_(-1.0 if rep % 2 else 1.0)
        ref_o, ref_l = eager(q, k, v)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: O differs from the eager call"
        assert torch.equal(lse, ref_l), f"replay {rep}: LSE differs from the eager call"
