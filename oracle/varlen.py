"""CPU oracle for variable-length batches in packed layout (fp64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module. The GPU library never calls
it and shares no code with it; this module imports numpy and the plain
oracle only.

The pages list variable-length sequences among the uses of grouped-query
attention (batch-sensitivity article, "applicable scenarios") and continuous
batching of generation requests (Llama-2 GQA article, section 4.1), without
a layout. Reading taken here: the sequences of a batch are packed along the
token axis, q [total_q, Hq, d] and k, v [total_k, Hk, d], and sequence b
owns query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key tokens
cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (both arrays non-decreasing, length
B+1, starting at 0). Each sequence is an independent attention problem with
its own lengths and its own bottom-right causal alignment. Outputs are
O [total_q, Hq, d] and LSE [Hq, total_q]; a sequence with no key gives
O = 0 and LSE = -inf for its tokens.
"""

from __future__ import annotations

import numpy as np

from .attention import NEG_INF, attention_fp64


def attention_varlen_fp64(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool, scale: float, sequences=None):
    """Exact GQA forward of every packed sequence (or only the listed ones; other rows stay 0 / -inf)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    total_q, Hq, d = q.shape
    cu_q = [int(x) for x in cu_seqlens_q]
    cu_k = [int(x) for x in cu_seqlens_k]
    B = len(cu_q) - 1
    O = np.zeros((total_q, Hq, d))
    LSE = np.full((Hq, total_q), NEG_INF)
    for b in (range(B) if sequences is None else sequences):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0:
            continue
        Ob, Lb = attention_fp64(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], causal, scale)
        O[q0:q1] = Ob[0]
        LSE[:, q0:q1] = Lb[0]
    return O, LSE
