"""The seeded input generator: deterministic, chunkable per batch element, bf16 from N(0,1)."""

import torch

import gqa_inputs as gi


def test_deterministic_and_chunkable():
    w = gi.TINY.with_(B=3)
    q, k, v = gi.make_qkv(w)
    q2, k2, v2 = gi.make_qkv(w)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    qb, kb, vb = gi.make_qkv(w, batches=[2])
    assert torch.equal(qb[0], q[2]) and torch.equal(kb[0], k[2]) and torch.equal(vb[0], v[2])
    assert q.dtype == torch.bfloat16 and q.shape == (3, w.Sq, w.Hq, w.d)
    assert k.shape == (3, w.Sk, w.Hk, w.d)
    # q, k, v streams and batch elements are distinct
    assert not torch.equal(q[0, :, :2], k[0, :, :2])
    assert not torch.equal(q[0], q[1])


def test_distribution():
    q, _, _ = gi.make_qkv(gi.TINY)
    x = q.float()
    assert abs(x.mean().item()) < 0.02 and abs(x.std().item() - 1.0) < 0.02


def test_workloads():
    names = [w.name for w in gi.ALL]
    assert len(set(names)) == len(names)
    for w in gi.ALL:
        assert w.Hq % w.Hk == 0 and w.d in (64, 128)
    assert gi.RAGGED.B == 16384 // 77
    assert abs(gi.LLAMA_PREFILL.flops - 4 * 4 * 32 * 2048 * 2048 * 128 / 2) < 1
    assert gi.sweep(64).scale == gi.fp32(1 / 128 ** 0.5)
