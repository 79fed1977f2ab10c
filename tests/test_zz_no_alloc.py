"""gqa_attn_fwd_noalloc: the forward pass without any allocation (GPU).

Split calls keep their partials in the library's fixed per-GPU scratch array.
Two calls in a row (the second smaller, so it reuses the array the first
filled) must give exactly what gqa_attn_fwd gives on the same inputs and
launch plan (same kernels, same arithmetic), and stay within the oracle's
tolerances; a call whose workspace exceeds the array is refused before any
launch and leaves its outputs untouched.
"""

import pytest
import torch

import gqa_inputs as gi
from _parity import compare_to_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(entry, q, k, v, causal, scale, pack, ns):
    B, Sq, Hq, _ = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV)
    entry(q, k, v, out, lse, causal, scale, pack, ns)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_allocating_call_twice_in_a_row():
    import grouped_query_exact_amd as g
    cases = [
        # the decode workload at 8 splits: 8.5 MB of partials
        (gi.DECODE, 1, 8),
        # a smaller, ragged causal prefill next: 3 splits over fewer rows
        (gi.TINY.with_(B=3, Sq=100, Sk=700, Hq=8, Hk=2, d=64, causal=True, seed=77), 1, 3),
    ]
    for w, pack, ns in cases:
        q, k, v = gi.make_qkv(w)
        plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, pack, ns)
        assert plan["num_splits"] == ns and 0 < plan["workspace_bytes"] <= g.GQA_NOALLOC_SCRATCH_BYTES
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        On, Ln = _run(g.gqa_attn_fwd_noalloc, qd, kd, vd, w.causal, w.scale, pack, ns)
        Oa, La = _run(g.gqa_attn_fwd, qd, kd, vd, w.causal, w.scale, pack, ns)
        assert torch.equal(On, Oa) and torch.equal(Ln, La), f"{w.name}: differs from gqa_attn_fwd"
        rows = list(range(min(w.Sq, 40)))
        compare_to_oracle(On, Ln, q, k, v, w.causal, w.scale, rows=rows, tag=f"noalloc {w.name} ns={ns}")


def test_noalloc_unsplit_call_needs_no_scratch():
    import grouped_query_exact_amd as g
    w = gi.RAGGED
    q, k, v = (t.to(DEV) for t in gi.make_qkv(w))
    On, Ln = _run(g.gqa_attn_fwd_noalloc, q, k, v, w.causal, w.scale, 1, 1)
    Oa, La = _run(g.gqa_attn_fwd, q, k, v, w.causal, w.scale, 1, 1)
    assert torch.equal(On, Oa) and torch.equal(Ln, La)


def test_noalloc_refuses_oversized_workspace():
    import grouped_query_exact_amd as g
    B, S, Hq, Hk, d = 4, 2048, 32, 8, 128
    plan = g.gqa_attn_plan(B, S, S, Hq, Hk, d, True, 1, 2)
    assert plan["workspace_bytes"] > g.GQA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, S, Hq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, S, Hk, d), dtype=torch.bfloat16, device=DEV)
    out, lse = _run(lambda *a: None, q, k, k, True, 0.1, 1, 2)  # NaN-filled buffers
    with pytest.raises(g.GqaAttnError) as e:
        g.gqa_attn_fwd_noalloc(q, k, k, out, lse, True, 0.1, 1, 2)
    assert e.value.status == g.GQA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()
