"""Pins of the fp8 oracle to facts other than itself (CPU only).

* the e4m3 decoding of all 256 codes equals torch's float8_e4m3fn (a library
  routine), NaN codes included, and the format's landmarks: 1.0 = 0x38,
  448 = 0x7E (largest finite), 2^-6 = 0x08 (smallest normal), 2^-9 = 0x01
  (smallest subnormal), -0 = 0x80, NaN = 0x7F and 0xFF;
* the factor identities: attention over k_scale * K equals attention over K
  with scale * k_scale, and v_scale multiplies the output and leaves the LSE;
* the paged fp8 oracle equals the contiguous one on gathered sequences;
* fp8 queries and keys: attention over q_scale * Q and k_scale * K equals
  attention over the decoded Q and K with scale * q_scale * k_scale (signs
  included), and unit factors give the plain attention of the decoded values.
Planted mistakes (exponent bias 8, a factor applied to the wrong tensor,
q_scale applied to V) each fail a pin.
"""

import math

import numpy as np
import torch

import gqa_inputs as gi
import oracle
from oracle import fp8 as ofp8

CODES = np.arange(256)


def pin_decode(decode):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode(CODES)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert decode(np.array([0x38]))[0] == 1.0
    assert decode(np.array([0x7E]))[0] == 448.0
    assert decode(np.array([0x08]))[0] == 2.0 ** -6
    assert decode(np.array([0x01]))[0] == 2.0 ** -9
    z = decode(np.array([0x80]))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0
    assert np.isnan(decode(np.array([0x7F, 0xFF]))).all()


def pin_factors(attn_kv8):
    B, Sq, Sk, Hq, Hk, d = 2, 3, 37, 8, 2, 16
    q = gi.random_bf16(1, (B, Sq, Hq, d)).to(torch.float64).numpy()
    k8, v8 = gi.random_fp8(2, (B, Sk, Hk, d)).numpy(), gi.random_fp8(3, (B, Sk, Hk, d)).numpy()
    K, V = ofp8.e4m3_to_float(k8), ofp8.e4m3_to_float(v8)
    for causal in (False, True):
        O1, L1 = attn_kv8(q, k8, v8, 1.0, 1.0, causal, 0.25)
        O0, L0 = oracle.attention_fp64(q, K, V, causal, 0.25)
        assert np.allclose(O1, O0, rtol=0, atol=1e-13) and np.allclose(L1, L0, rtol=0, atol=1e-13)
        Ok, Lk = attn_kv8(q, k8, v8, 0.375, 1.0, causal, 0.25)
        Os, Ls = oracle.attention_fp64(q, K, V, causal, 0.25 * 0.375)
        assert np.allclose(Ok, Os, rtol=0, atol=1e-12) and np.allclose(Lk, Ls, rtol=0, atol=1e-12)
        Ov, Lv = attn_kv8(q, k8, v8, 1.0, -2.5, causal, 0.25)
        assert np.allclose(Ov, -2.5 * O0, rtol=0, atol=1e-12) and np.allclose(Lv, L0, rtol=0, atol=1e-13)


def test_decode_pin():
    pin_decode(ofp8.e4m3_to_float)


def test_factor_pin():
    pin_factors(oracle.attention_kv8_fp64)


def test_paged_fp8_matches_contiguous():
    lens, ps, Hq, Hk, d = [40, 3, 17], 16, 4, 2, 8
    kv = gi.paged_kv(11, lens, ps, Hk, d)
    k8, v8 = gi.to_fp8_bytes(kv.k_cache).numpy(), gi.to_fp8_bytes(kv.v_cache).numpy()
    q = gi.random_bf16(12, (3, 2, Hq, d)).to(torch.float64).numpy()
    O, L = oracle.attention_paged_kv8_fp64(q, k8, v8, kv.block_table.numpy(), kv.seqlens_k.numpy(), 0.5, 3.0,
                                           True, 0.3)
    for b, n in enumerate(lens):
        rows_k = [k8[kv.block_table[b, j // ps], j % ps] for j in range(n)]
        rows_v = [v8[kv.block_table[b, j // ps], j % ps] for j in range(n)]
        Oc, Lc = oracle.attention_kv8_fp64(q[b:b + 1], np.stack(rows_k)[None], np.stack(rows_v)[None], 0.5, 3.0,
                                           True, 0.3)
        assert np.allclose(O[b], Oc[0], rtol=0, atol=1e-13) and np.allclose(L[b], Lc[0], rtol=0, atol=1e-13)


def test_planted_exponent_bias_8():
    def bad(codes):
        c = np.asarray(codes).astype(np.int64) & 0xFF
        e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
        val = np.where(e == 0, m * 2.0 ** -10, (1 + m / 8) * np.exp2(e - 8.0))
        return np.where(c >> 7, -val, val)
    try:
        pin_decode(bad)
    except AssertionError:
        return
    raise AssertionError("the planted decoding passed")


def test_planted_factor_on_wrong_tensor():
    def bad(q, k8, v8, k_scale, v_scale, causal, scale, **kw):
        return oracle.attention_kv8_fp64(q, k8, v8, v_scale, k_scale, causal, scale, **kw)
    try:
        pin_factors(bad)
    except AssertionError:
        return
    raise AssertionError("the planted factor swap passed")


def pin_qk_factors(attn_qk8):
    B, Sq, Sk, Hq, Hk, d = 2, 5, 29, 6, 2, 16
    q8, k8 = gi.random_fp8(21, (B, Sq, Hq, d)).numpy(), gi.random_fp8(22, (B, Sk, Hk, d)).numpy()
    v = gi.random_bf16(23, (B, Sk, Hk, d)).to(torch.float64).numpy()
    Q, K = ofp8.e4m3_to_float(q8), ofp8.e4m3_to_float(k8)
    for causal in (False, True):
        O1, L1 = attn_qk8(q8, k8, v, 1.0, 1.0, causal, 0.25)
        O0, L0 = oracle.attention_fp64(Q, K, v, causal, 0.25)
        assert np.allclose(O1, O0, rtol=0, atol=1e-13) and np.allclose(L1, L0, rtol=0, atol=1e-13)
        for qs, ks in ((0.5, -1.25), (-3.0, 0.125)):
            Of, Lf = attn_qk8(q8, k8, v, qs, ks, causal, 0.25)
            Os, Ls = oracle.attention_fp64(Q, K, v, causal, 0.25 * qs * ks)
            assert np.allclose(Of, Os, rtol=0, atol=1e-12) and np.allclose(Lf, Ls, rtol=0, atol=1e-12)


def test_qk_factor_pin():
    pin_qk_factors(oracle.attention_qk8_fp64)


def test_planted_q_scale_on_values():
    def bad(q8, k8, v, q_scale, k_scale, causal, scale, **kw):
        return oracle.attention_qk8_fp64(q8, k8, np.asarray(v) * q_scale, 1.0, k_scale, causal, scale, **kw)
    try:
        pin_qk_factors(bad)
    except AssertionError:
        return
    raise AssertionError("the planted factor on V passed")
