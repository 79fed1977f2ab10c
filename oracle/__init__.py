"""CPU oracle (test infrastructure only): plain fp64 grouped-query attention.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may use this package. The GPU library neither imports nor links it.

Every function is pinned by the CPU tests (brute force on tiny inputs, the
MHA identity, a library routine, closed forms and invariants); no function
here is "parity unpinned".
"""

from .attention import (NEG_INF, attention_fp64, combine_fp64, kv_head_of,
                        split_combine_fp64, split_partials_fp64, split_tiles,
                        visible_keys)

__all__ = ["NEG_INF", "attention_fp64", "combine_fp64", "kv_head_of", "split_combine_fp64",
           "split_partials_fp64", "split_tiles", "visible_keys"]
