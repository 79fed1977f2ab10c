"""CPU oracle (test infrastructure only): plain fp64 grouped-query attention.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may use this package. The GPU library neither imports nor links it.

Every function is pinned by the CPU tests (brute force on tiny inputs, the
MHA identity, a library routine, closed forms and invariants; for the paged
cache also a gather of known draws and a brute force that looks every key up
in the pool; for fp8 the e4m3 decoding against torch's float8_e4m3fn and the
format's printed landmarks); no function here is "parity unpinned".
"""

from .attention import (NEG_INF, attention_fp64, combine_fp64, kv_head_of,
                        split_combine_fp64, split_partials_fp64, split_tiles,
                        visible_keys)
from .paged import attention_paged_fp64, gather_pages
from .fp8 import attention_kv8_fp64, attention_paged_kv8_fp64, attention_qk8_fp64, e4m3_to_float
from .varlen import attention_varlen_fp64
from .backward import attention_bwd_fp64, row_dot_fp64

__all__ = ["NEG_INF", "attention_bwd_fp64", "attention_fp64", "attention_kv8_fp64", "attention_paged_fp64", "attention_paged_kv8_fp64", "attention_qk8_fp64",
           "attention_varlen_fp64", "combine_fp64", "e4m3_to_float", "gather_pages", "row_dot_fp64",
           "kv_head_of", "split_combine_fp64", "split_partials_fp64", "split_tiles", "visible_keys"]
