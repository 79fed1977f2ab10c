"""CPU oracle for attention over fp8 e4m3 keys and values (fp64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module. The GPU library never calls
it and shares no code with it; this module imports numpy and the plain
oracle only.

The pages name FP8 e4m3 as the way to halve the bandwidth pressure of
inference (rise-and-fall tuning article, "verification and further
directions"). Reading taken here: K and V are given as e4m3 bytes with one
fp32 factor per tensor, so the operation is the plain attention over
K = k_scale * decode(k8) and V = v_scale * decode(v8). The e4m3 decoding
follows the OCP 8-bit floating point format: 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent 0 encodes subnormals m * 2^-9; the
code S.1111.111 is NaN and there is no infinity, so the largest finite
magnitude is 1.75 * 2^8 = 448.

The same reading for fp8 queries and keys (the compute-bound prefill case):
Q and K given as e4m3 bytes with factors q_scale and k_scale, V in bf16; the
operation is the plain attention over Q = q_scale * decode(q8),
K = k_scale * decode(k8) and V.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_fp64
from .paged import attention_paged_fp64


def e4m3_to_float(codes) -> np.ndarray:
    """Decode e4m3 bytes (any integer array) into float64 values."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = m * 2.0 ** -9
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


def attention_kv8_fp64(q, k8, v8, k_scale: float, v_scale: float, causal: bool, scale: float, **select):
    """Exact GQA forward over K = k_scale * decode(k8), V = v_scale * decode(v8)."""
    K = e4m3_to_float(k8) * float(k_scale)
    V = e4m3_to_float(v8) * float(v_scale)
    return attention_fp64(q, K, V, causal, scale, **select)


def attention_paged_kv8_fp64(q, k8_cache, v8_cache, block_table, seqlens_k, k_scale: float, v_scale: float,
                             causal: bool, scale: float, **select):
    """attention_paged_fp64 over fp8 page pools with per-tensor factors."""
    K = e4m3_to_float(k8_cache) * float(k_scale)
    V = e4m3_to_float(v8_cache) * float(v_scale)
    return attention_paged_fp64(q, K, V, block_table, seqlens_k, causal, scale, **select)


def attention_qk8_fp64(q8, k8, v, q_scale: float, k_scale: float, causal: bool, scale: float, **select):
    """Exact GQA forward over Q = q_scale * decode(q8), K = k_scale * decode(k8) and V."""
    Q = e4m3_to_float(q8) * float(q_scale)
    K = e4m3_to_float(k8) * float(k_scale)
    return attention_fp64(Q, K, np.asarray(v, dtype=np.float64), causal, scale, **select)
