"""Kept split-KV workspaces (GPU).

Split calls of up to 64 MiB of workspace reuse one buffer per (device, stream)
instead of allocating and releasing per call. These tests drive that buffer
through growth (small, larger, small again on one stream), through two streams
whose calls interleave without any synchronisation between them, and past the
64 MiB limit (per-call allocation). Every output must equal, bit for bit, the
same call through gqa_attn_fwd_noalloc (same kernels and plan, the partials in
the fixed scratch array) or, past the limit, an unsplit call within the variant
gate, and stay within the oracle's tolerances on sampled rows.
"""

import pytest
import torch

import gqa_inputs as gi
from _parity import assert_variants_agree, compare_to_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bufs(q):
    B, Sq, Hq, _ = q.shape
    return (torch.full_like(q, float("nan")),
            torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=q.device))


def _cases():
    return [
        (gi.TINY.with_(B=2, Sq=1, Sk=3000, Hq=8, Hk=2, d=64, causal=False, seed=11), 1, 4),
        (gi.DECODE.with_(B=16, seed=12), 1, 8),              # ~2 MB of partials: grows the buffer
        (gi.TINY.with_(B=3, Sq=70, Sk=900, Hq=12, Hk=4, d=128, causal=True, seed=13), 0, 3),
    ]


def test_kept_workspace_grows_and_shrinks_on_one_stream():
    import grouped_query_exact_amd as g
    s = torch.cuda.Stream(device=DEV)
    for w, pack, ns in _cases() + _cases()[:1]:
        q, k, v = gi.make_qkv(w)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, pack, ns)
        assert plan["num_splits"] == ns and plan["workspace_bytes"] <= g.GQA_NOALLOC_SCRATCH_BYTES
        torch.cuda.synchronize()
        Ok, Lk = _bufs(qd)
        with torch.cuda.stream(s):
            g.gqa_attn_fwd(qd, kd, vd, Ok, Lk, w.causal, w.scale, pack, ns)
        s.synchronize()
        On, Ln = _bufs(qd)
        g.gqa_attn_fwd_noalloc(qd, kd, vd, On, Ln, w.causal, w.scale, pack, ns)
        torch.cuda.synchronize()
        assert torch.equal(Ok, On) and torch.equal(Lk, Ln), f"{w.name} ns={ns}: differs from noalloc"
        compare_to_oracle(Ok, Lk, q, k, v, w.causal, w.scale, rows=list(range(min(w.Sq, 24))),
                          tag=f"kept {w.name} ns={ns}")


def test_kept_workspaces_of_two_streams_interleaved():
    import grouped_query_exact_amd as g
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    cases = _cases()
    inputs = []
    for w, pack, ns in cases:
        q, k, v = gi.make_qkv(w)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        ref = _bufs(qd)
        g.gqa_attn_fwd_noalloc(qd, kd, vd, ref[0], ref[1], w.causal, w.scale, pack, ns)
        inputs.append((w, pack, ns, qd, kd, vd, ref))
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):  # each stream runs every case, in another order, with no waits between
        for si, s in enumerate(streams):
            order = inputs if (rep + si) % 2 == 0 else inputs[::-1]
            with torch.cuda.stream(s):
                for w, pack, ns, qd, kd, vd, ref in order:
                    O, L = _bufs(qd)
                    g.gqa_attn_fwd(qd, kd, vd, O, L, w.causal, w.scale, pack, ns)
                    outs.append((w, ns, O, L, ref))
    torch.cuda.synchronize()
    for w, ns, O, L, ref in outs:
        assert torch.equal(O, ref[0]) and torch.equal(L, ref[1]), f"{w.name} ns={ns}: interleaved streams differ"


def test_workspace_past_the_kept_limit_is_per_call():
    import grouped_query_exact_amd as g
    # 1 x 2048 queries x 32 heads at d=128, 3 splits: 3 * 65536 * 520 B = 102 MB of partials (> 64 MiB)
    w = gi.LLAMA_PREFILL.with_(B=1, causal=True, seed=14)
    q, k, v = gi.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, 1, 3)
    assert plan["workspace_bytes"] > 64 << 20
    O3, L3 = _bufs(qd)
    O1, L1 = _bufs(qd)
    for _ in range(2):
        g.gqa_attn_fwd(qd, kd, vd, O3, L3, w.causal, w.scale, 1, 3)
    with torch.cuda.stream(torch.cuda.Stream(device=DEV)):
        g.gqa_attn_fwd(qd, kd, vd, O1, L1, w.causal, w.scale, 1, 1)
    torch.cuda.synchronize()
    assert_variants_agree(O3, L3, O1, L1, float(v.float().abs().max()), tag="ns=3 per-call workspace vs unsplit")
    compare_to_oracle(O3, L3, q, k, v, w.causal, w.scale, rows=[0, 1, 777, 2047], tag="ns=3 per-call")


def test_kept_workspace_shared_by_host_threads():
    """Host threads that enqueue split calls of different sizes on one stream at the same time:
    a call holds its stream's buffer from the lookup until its kernels are enqueued, so a growth by
    another thread never releases a buffer between a call's lookup and its launches. Every output
    equals the no-allocation entry point's, bit for bit."""
    import threading
    import grouped_query_exact_amd as g
    s = torch.cuda.Stream(device=DEV)
    cases = _cases()
    inputs = []
    for w, pack, ns in cases:
        q, k, v = gi.make_qkv(w)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        ref = _bufs(qd)
        g.gqa_attn_fwd_noalloc(qd, kd, vd, ref[0], ref[1], w.causal, w.scale, pack, ns)
        inputs.append((w, pack, ns, qd, kd, vd, ref))
    outs = [[] for _ in range(4)]
    bufs = [[_bufs(x[3]) for _ in range(6) for x in inputs] for _ in range(4)]  # allocated up front
    torch.cuda.synchronize()  # the NaN fills run on the default stream
    errors = []

    def worker(i):
        try:
            for r in range(6):
                order = list(range(len(inputs))) if (i + r) % 2 == 0 else list(range(len(inputs)))[::-1]
                for j in order:
                    w, pack, ns, qd, kd, vd, ref = inputs[j]
                    O, L = bufs[i][r * len(inputs) + j]
                    g.gqa_attn_fwd(qd, kd, vd, O, L, w.causal, w.scale, pack, ns, stream=s)
                    outs[i].append((w, ns, O, L, ref))
        except Exception as e:  # reported below, on the test's own thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for per in outs:
        for w, ns, O, L, ref in per:
            assert torch.equal(O, ref[0]) and torch.equal(L, ref[1]), f"{w.name} ns={ns}: threads sharing a stream differ"
