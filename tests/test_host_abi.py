"""CPU tests of the C-ABI library: exported symbols, status strings, the
heuristic and launch plan, and argument checks that return before any HIP call.

No compute is launched here (there is no GPU in this environment): every
gqa_attn_fwd call below carries an invalid argument and must be rejected by
the host-side checks.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")
LIB = os.path.join(ROOT, "grouped_query_exact_amd", "libgqa_attn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libgqa_attn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gqa_attn_\w+)\s*\(", text, flags=re.M)))


def lib():
    import grouped_query_exact_amd as g
    return g.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == ["gqa_attn_bwd", "gqa_attn_choose", "gqa_attn_fwd", "gqa_attn_fwd_kv8", "gqa_attn_fwd_noalloc",
                     "gqa_attn_fwd_paged",
                     "gqa_attn_fwd_paged_kv8", "gqa_attn_fwd_qk8", "gqa_attn_fwd_varlen", "gqa_attn_plan",
                     "gqa_attn_strerror"]


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
    for name in declared_functions():
        assert hasattr(lib(), name)


def test_strerror():
    import grouped_query_exact_amd as g
    assert g.gqa_attn_strerror(0) == "success"
    for st in (g.GQA_ERR_INVALID_ARG, g.GQA_ERR_UNSUPPORTED, g.GQA_ERR_NOMEM, g.GQA_ERR_HIP, g.GQA_ERR_SCRATCH):
        assert g.gqa_attn_strerror(st) not in ("success", "unknown status")
    assert g.gqa_attn_strerror(12345) == "unknown status"


def _fwd(q=1, k=1, v=1, out=1, lse=None, B=1, Sq=4, Sk=4, Hq=2, Hk=1, d=64, causal=0, scale=0.125,
         pack=-1, ns=0):
    """Call gqa_attn_fwd with fake (never dereferenced) pointers; only invalid calls are allowed."""
    L = lib()
    P = lambda x: None if x is None else ctypes.c_void_p(x * 4096)
    return L.gqa_attn_fwd(P(q), P(k), P(v), P(out), P(lse), B, Sq, Sk, Hq, Hk, d, causal, scale, pack, ns, None)


@pytest.mark.parametrize("kw", [
    dict(Hq=6, Hk=4),           # Hq not a multiple of Hk (the pages' divisibility rule)
    dict(Hk=0),
    dict(Hq=-2),
    dict(B=-1),
    dict(Sq=-1),
    dict(Sk=-3),
    dict(Sk=0),                 # queries but no keys
    dict(pack=2),
    dict(pack=-2),
    dict(ns=-1),
    dict(scale=float("inf")),
    dict(scale=float("nan")),
    dict(q=None),
    dict(k=None),
    dict(v=None),
    dict(out=None),
])
def test_invalid_arguments_are_rejected(kw):
    import grouped_query_exact_amd as g
    assert _fwd(**kw) == g.GQA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Hq=6, Hk=4), dict(Sk=0), dict(pack=2), dict(ns=-1), dict(q=None),
                                dict(scale=float("nan"))])
def test_noalloc_invalid_arguments_are_rejected(kw):
    """The no-allocation entry point runs gqa_attn_fwd's checks before anything else."""
    import grouped_query_exact_amd as g
    L = lib()
    a = dict(q=1, k=1, v=1, out=1, B=1, Sq=4, Sk=4, Hq=2, Hk=1, d=64, causal=0, scale=0.125, pack=-1, ns=0)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x * 4096)
    st = L.gqa_attn_fwd_noalloc(P(a["q"]), P(a["k"]), P(a["v"]), P(a["out"]), None, a["B"], a["Sq"], a["Sk"],
                                a["Hq"], a["Hk"], a["d"], a["causal"], a["scale"], a["pack"], a["ns"], None)
    assert st == g.GQA_ERR_INVALID_ARG


def test_noalloc_scratch_size_matches_header():
    import grouped_query_exact_amd as g
    text = open(HEADER).read()
    assert re.search(r"#define GQA_NOALLOC_SCRATCH_BYTES \(64LL << 20\)", text)
    assert g.GQA_NOALLOC_SCRATCH_BYTES == 64 << 20


@pytest.mark.parametrize("d", [0, 32, 96, 256])
def test_unsupported_head_dim(d):
    import grouped_query_exact_amd as g
    assert _fwd(d=d) == g.GQA_ERR_UNSUPPORTED


def test_misaligned_pointer_is_unsupported():
    import grouped_query_exact_amd as g
    L = lib()
    st = L.gqa_attn_fwd(ctypes.c_void_p(4096 + 8), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                        ctypes.c_void_p(8192), None, 1, 4, 4, 2, 1, 64, 0, 0.125, 1, 1, None)
    assert st == g.GQA_ERR_UNSUPPORTED


def _paged(q=1, kc=1, vc=1, bt=1, sl=1, out=1, lse=None, B=2, Sq=1, Hq=8, Hk=2, d=128, num_pages=10,
           page_size=32, max_pages=4, causal=0, scale=0.125, pack=-1, ns=0):
    """Call gqa_attn_fwd_paged with fake (never dereferenced) pointers; only invalid calls are allowed."""
    L = lib()
    P = lambda x: None if x is None else ctypes.c_void_p(x * 4096)
    return L.gqa_attn_fwd_paged(P(q), P(kc), P(vc), P(bt), P(sl), P(out), P(lse), B, Sq, Hq, Hk, d,
                                num_pages, page_size, max_pages, causal, scale, pack, ns, None)


def _paged8(q=1, kc=1, vc=1, bt=1, sl=1, out=1, lse=None, B=2, Sq=1, Hq=8, Hk=2, d=128, num_pages=10,
            page_size=32, max_pages=4, causal=0, scale=0.125, pack=-1, ns=0):
    """gqa_attn_fwd_paged_kv8 with fake pointers and unit factors; only invalid calls are allowed."""
    L = lib()
    P = lambda x: None if x is None else ctypes.c_void_p(x * 4096)
    return L.gqa_attn_fwd_paged_kv8(P(q), P(kc), P(vc), 1.0, 1.0, P(bt), P(sl), P(out), P(lse), B, Sq, Hq, Hk, d,
                                    num_pages, page_size, max_pages, causal, scale, pack, ns, None)


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=0), "INVALID_ARG"),
    (dict(page_size=-16), "INVALID_ARG"),
    (dict(max_pages=0), "INVALID_ARG"),
    (dict(num_pages=0), "INVALID_ARG"),
    (dict(max_pages=2 ** 30), "INVALID_ARG"),      # table capacity overflows int
    (dict(bt=None), "INVALID_ARG"),
    (dict(sl=None), "INVALID_ARG"),
    (dict(kc=None), "INVALID_ARG"),
    (dict(Hq=6, Hk=4), "INVALID_ARG"),
    (dict(scale=float("nan")), "INVALID_ARG"),
    (dict(page_size=24), "UNSUPPORTED"),            # not a multiple of 16
    (dict(page_size=8), "UNSUPPORTED"),
    (dict(d=96), "UNSUPPORTED"),
    (dict(Sq=9, pack=0), "OK_OR_DEVICE"),           # 9 unpacked rows per head: accepted up to the launch
])
def test_paged_argument_checks(kw, status):
    import grouped_query_exact_amd as g
    st = _paged(**kw)
    if status == "OK_OR_DEVICE":
        assert st in (g.GQA_OK, g.GQA_ERR_HIP)  # no GPU here: the first HIP call fails
    else:
        assert st == getattr(g, "GQA_ERR_" + status), (kw, st)


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=24), "UNSUPPORTED"),            # not a multiple of 16
    (dict(Sq=9, Hq=8, Hk=2), "UNSUPPORTED"),        # 36 packed rows: fp8 pools take decode shapes only
    (dict(Sq=33, Hq=2, Hk=2), "UNSUPPORTED"),       # 33 rows of one head
    (dict(max_pages=0), "INVALID_ARG"),
])
def test_paged_kv8_argument_checks(kw, status):
    import grouped_query_exact_amd as g
    assert _paged8(**kw) == getattr(g, "GQA_ERR_" + status), kw


@pytest.mark.parametrize("kw,status", [
    (dict(total_q=-1), "INVALID_ARG"),
    (dict(total_k=-1), "INVALID_ARG"),
    (dict(msk=0), "INVALID_ARG"),                   # queries but no key anywhere
    (dict(cq=None), "INVALID_ARG"),
    (dict(ck=None), "INVALID_ARG"),
    (dict(Hq=6, Hk=4), "INVALID_ARG"),
    (dict(d=32), "UNSUPPORTED"),
    (dict(cq=1.0005), "UNSUPPORTED"),              # offsets not 4-byte aligned
])
def test_varlen_argument_checks(kw, status):
    import grouped_query_exact_amd as g
    a = dict(q=1, k=1, v=1, out=1, lse=None, cq=1, ck=1, B=2, msq=9, msk=9, total_q=12, total_k=12, Hq=4, Hk=2,
             d=64, causal=0, scale=0.125, pack=-1, ns=0)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(int(x * 4096))
    st = lib().gqa_attn_fwd_varlen(P(a["q"]), P(a["k"]), P(a["v"]), P(a["out"]), P(a["lse"]), P(a["cq"]), P(a["ck"]),
                                   a["B"], a["msq"], a["msk"], a["total_q"], a["total_k"], a["Hq"], a["Hk"], a["d"],
                                   a["causal"], a["scale"], a["pack"], a["ns"], None)
    assert st == getattr(g, "GQA_ERR_" + status), (kw, st)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hk=4), "INVALID_ARG"),
    (dict(Sk=0), "INVALID_ARG"),
    (dict(lse=None), "INVALID_ARG"),
    (dict(dq=None), "INVALID_ARG"),
    (dict(scale=float("inf")), "INVALID_ARG"),
    (dict(d=96), "UNSUPPORTED"),
    (dict(lse=1.0005), "UNSUPPORTED"),
    (dict(dk=1.0005), "UNSUPPORTED"),
    (dict(Sq=0, q=None, out=None, lse=None, do=None, dq=None, k=None), "INVALID_ARG"),   # no rows: k still needed
    (dict(Sq=0, q=None, out=None, lse=None, do=None, dq=None, dv=1.0005), "UNSUPPORTED"),
])
def test_backward_argument_checks(kw, status):
    import grouped_query_exact_amd as g
    a = dict(q=1, k=1, v=1, out=1, lse=1, do=1, dq=1, dk=1, dv=1, B=1, Sq=8, Sk=8, Hq=4, Hk=2, d=64, causal=1,
             scale=0.125)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(int(x * 4096))
    st = lib().gqa_attn_bwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["out"]), P(a["lse"]), P(a["do"]), P(a["dq"]),
                            P(a["dk"]), P(a["dv"]), a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hk"], a["d"], a["causal"],
                            a["scale"], None)
    assert st == getattr(g, "GQA_ERR_" + status), (kw, st)


@pytest.mark.parametrize("kw,status", [
    (dict(qs=float("nan")), "INVALID_ARG"),
    (dict(ks=float("inf")), "INVALID_ARG"),
    (dict(Hq=6, Hk=4), "INVALID_ARG"),
    (dict(scale=float("nan")), "INVALID_ARG"),
    (dict(q=None), "INVALID_ARG"),
    (dict(d=96), "UNSUPPORTED"),
    (dict(k=1.0005), "UNSUPPORTED"),
    (dict(q=None, k=None, v=None, out=None, B=0), "OK"),
])
def test_qk8_argument_checks(kw, status):
    import grouped_query_exact_amd as g
    a = dict(q=1, k=1, v=1, qs=1.0, ks=1.0, out=1, lse=None, B=1, Sq=8, Sk=8, Hq=4, Hk=2, d=64, causal=1,
             scale=0.125, pack=-1, ns=0)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(int(x * 4096))
    st = lib().gqa_attn_fwd_qk8(P(a["q"]), P(a["k"]), P(a["v"]), a["qs"], a["ks"], P(a["out"]), P(a["lse"]), a["B"],
                                a["Sq"], a["Sk"], a["Hq"], a["Hk"], a["d"], a["causal"], a["scale"], a["pack"],
                                a["ns"], None)
    want = g.GQA_OK if status == "OK" else getattr(g, "GQA_ERR_" + status)
    assert st == want, (kw, st)


def test_paged_misaligned_table_is_unsupported():
    import grouped_query_exact_amd as g
    L = lib()
    st = L.gqa_attn_fwd_paged(ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                              ctypes.c_void_p(4096 + 2), ctypes.c_void_p(4096), ctypes.c_void_p(8192), None,
                              2, 1, 8, 2, 128, 10, 32, 4, 0, 0.125, -1, 0, None)
    assert st == g.GQA_ERR_UNSUPPORTED


def test_paged_empty_problem_is_a_no_op():
    import grouped_query_exact_amd as g
    assert _paged(q=None, kc=None, vc=None, bt=None, sl=None, out=None, B=0) == g.GQA_OK


def test_empty_problem_is_a_no_op():
    import grouped_query_exact_amd as g
    # B*Sq == 0: nothing to do, no pointer is touched (null pointers allowed)
    assert _fwd(q=None, k=None, v=None, out=None, B=0) == g.GQA_OK
    assert _fwd(q=None, k=None, v=None, out=None, Sq=0) == g.GQA_OK


def test_choose_heuristic_shapes():
    import grouped_query_exact_amd as g
    # prefill: long sequences, plenty of tiles -> pack, no split
    assert g.gqa_attn_choose(128, 2048, 2048, 32, 8, 128, True, 256) == (1, 1)
    assert g.gqa_attn_choose(4, 2048, 2048, 32, 8, 128, True, 256) == (1, 1)
    # short ragged sequences (Sq=77 fills 60% of a 128-row tile, 3 heads packed fill 90%)
    assert g.gqa_attn_choose(212, 77, 77, 6, 2, 64, False, 256)[0] == 1
    # decode: one query row per head -> pack; 64 x 8 groups already give two
    # workgroups per compute unit; fewer groups split the keys up to one
    # workgroup per compute unit (8 x 8 groups: 4 splits), up to 64 splits
    assert g.gqa_attn_choose(64, 1, 8192, 32, 8, 128, False, 256) == (1, 1)
    pk, ns = g.gqa_attn_choose(8, 1, 8192, 32, 8, 128, False, 256)
    assert pk == 1 and ns == 4
    assert g.gqa_attn_choose(4, 1, 131072, 32, 8, 128, False, 256) == (1, 8)
    assert g.gqa_attn_choose(1, 1, 131072, 32, 8, 128, False, 256) == (1, 32)
    assert g.gqa_attn_choose(1, 1, 131072, 4, 4, 128, False, 256) == (0, 64)
    # ... but at least two 32-key tiles per split
    assert g.gqa_attn_choose(1, 1, 1024, 32, 8, 128, False, 256) == (1, 16)
    # MHA: nothing to pack
    assert g.gqa_attn_choose(8, 512, 512, 8, 8, 64, True, 256)[0] == 0
    # invalid sizes are reported
    with pytest.raises(g.GqaAttnError):
        g.gqa_attn_choose(1, 4, 4, 6, 4, 64, False, 256)


def test_plan_force_tiled_switch(monkeypatch):
    """GQA_ATTN_FORCE_TILED=1 keeps prefill calls on the 4-wavefront kernel (128-row tiles, every row
    tile its own workgroup); "0" or an empty value leaves the choice to the plan."""
    import grouped_query_exact_amd as g
    args = (128, 2048, 2048, 32, 8, 128, True, 1, 1, 256)
    assert g.gqa_attn_plan(*args)["threads"] == 512
    monkeypatch.setenv("GQA_ATTN_FORCE_TILED", "1")
    p = g.gqa_attn_plan(*args)
    assert (p["threads"], p["block_m"], p["grid"]) == (256, 128, 128 * 8 * 64)
    for off in ("0", ""):
        monkeypatch.setenv("GQA_ATTN_FORCE_TILED", off)
        assert g.gqa_attn_plan(*args)["threads"] == 512


def test_plan_grid_and_workspace():
    import grouped_query_exact_amd as g
    p = g.gqa_attn_plan(128, 2048, 2048, 32, 8, 128, True, 1, 1, 256)
    assert p["pack_gqa"] == 1 and p["num_splits"] == 1 and p["workspace_bytes"] == 0
    assert p["block_n"] == 64
    assert p["row_tiles"] * p["block_m"] >= 2048 * 4
    # large unsplit bf16 calls: 8 wavefronts, 256-row tiles, one workgroup per compute unit; causal
    # launches pair each row tile with its mirror, so the grid holds half the row tiles
    assert (p["block_m"], p["threads"], p["row_tiles"], p["grid"]) == (256, 512, 32, 128 * 8 * 16)
    p = g.gqa_attn_plan(128, 2048, 2048, 32, 8, 128, False, 1, 1, 256)
    assert (p["block_m"], p["threads"], p["row_tiles"], p["grid"]) == (256, 512, 32, 128 * 8 * 32)
    p = g.gqa_attn_plan(64, 1800, 1800, 32, 8, 128, True, 1, 1, 256)  # odd row tiles: the middle one alone
    assert (p["threads"], p["row_tiles"], p["grid"]) == (512, 29, 64 * 8 * 15)
    # a chunk of 2048 tokens against 65536 keys: 256 row tiles would make only 128 pairs on
    # 256 compute units, so each row tile gets its own workgroup
    p = g.gqa_attn_plan(1, 2048, 65536, 32, 8, 128, True, 1, 1, 256)
    assert (p["threads"], p["row_tiles"], p["grid"]) == (512, 32, 8 * 32)
    # ... only with at least two such items per compute unit (212 * 2 = 424 < 512 here)
    p = g.gqa_attn_plan(212, 77, 77, 6, 2, 64, False, 1, 1, 256)
    assert (p["block_m"], p["threads"], p["grid"]) == (128, 256, 212 * 2 * 2)
    assert g.gqa_attn_plan(212, 77, 77, 6, 2, 128, True, 1, 1, 128)["threads"] == 512
    assert g.gqa_attn_plan(212, 77, 77, 6, 2, 128, False, 1, 1, 128)["threads"] == 256  # 2 key tiles
    # d=64 keeps the 4-wavefront kernel
    assert g.gqa_attn_plan(212, 77, 77, 6, 2, 64, False, 1, 1, 128)["threads"] == 256
    assert g.gqa_attn_plan(64, 2048, 2048, 32, 8, 64, True, 1, 1, 256)["threads"] == 256
    # one item per compute unit suffices when the items are long (an average of >= 32 key tiles):
    # a 2048-token chunk against 65536 keys and a non-causal 2048 x 2048 call do, a causal one does not
    assert g.gqa_attn_plan(1, 2048, 65536, 32, 8, 128, True, 1, 1, 256)["threads"] == 512
    assert g.gqa_attn_plan(1, 2048, 2048, 32, 8, 128, False, 1, 1, 256)["threads"] == 512
    assert g.gqa_attn_plan(1, 2048, 2048, 32, 8, 128, True, 1, 1, 256)["threads"] == 256
    # non-causal calls whose rows read at most 8 key tiles keep the 4-wavefront kernel; causal ones do not
    assert g.gqa_attn_plan(32, 384, 384, 32, 8, 128, False, 1, 1, 256)["threads"] == 256
    assert g.gqa_attn_plan(64, 512, 512, 32, 8, 128, False, 1, 1, 256)["threads"] == 256
    assert g.gqa_attn_plan(24, 768, 768, 32, 8, 128, False, 1, 1, 256)["threads"] == 512
    assert g.gqa_attn_plan(64, 256, 256, 32, 8, 128, True, 1, 1, 256)["threads"] == 512
    # split calls stay on the 4-wavefront kernel
    assert g.gqa_attn_plan(128, 2048, 2048, 32, 8, 128, True, 1, 2, 256)["threads"] == 256
    p = g.gqa_attn_plan(16, 2048, 2048, 32, 8, 128, True, 0, 4, 256)
    assert p["pack_gqa"] == 0 and p["num_splits"] == 4
    assert p["grid"] == 16 * 32 * p["row_tiles"] * 4
    assert p["workspace_bytes"] == 4 * 16 * 2048 * 32 * (128 * 4 + 8)  # O_s, LSE_s, W_s
    # the split count is clamped to the number of key tiles (decode tiles: 32 keys)
    p = g.gqa_attn_plan(1, 1, 100, 4, 4, 64, False, 0, 16, 256)
    assert p["num_splits"] == 4 and p["key_tiles"] == 4
    assert p["block_m"] == 32 and p["block_n"] == 32 and p["grid"] == 4 * 4
    p = g.gqa_attn_plan(1, 40, 100, 4, 4, 64, False, 0, 16, 256)
    assert p["num_splits"] == 2 and p["key_tiles"] == 2 and p["block_m"] == 128
    # decode-shaped work (at most 32 query rows per head unit) uses 32 x 32 tiles
    p = g.gqa_attn_plan(64, 1, 8192, 32, 8, 128, False, -1, 0, 256)
    assert (p["block_m"], p["block_n"], p["key_tiles"], p["grid"], p["threads"]) == (32, 32, 256, 512, 64)
    p = g.gqa_attn_plan(2, 9, 300, 32, 8, 128, True, 1, 1, 256)
    assert p["block_m"] == 128 and p["row_tiles"] == 1  # 36 packed rows
    # a single-head group never packs
    assert g.gqa_attn_plan(2, 300, 300, 4, 4, 64, False, 1, 1, 256)["pack_gqa"] == 0


CPP_TEST = r"""
#include "host_logic.h"
#include "../../include/gqa_attn.h"
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
using namespace gqa;
int main() {
    long long checked = 0;
    for (uint32_t d = 1; d <= 64; ++d) {
        FastDiv f = make_fastdiv(d);
        for (uint32_t n = 0; n < (1u << 20); ++n) {
            if (fastdiv_host(n, f) != n / d) { std::printf("FAIL d=%u n=%u\n", d, n); return 1; }
            ++checked;
        }
    }
    std::mt19937 rng(7);
    for (int i = 0; i < 2000000; ++i) {
        uint32_t d = 1 + rng() % 100000, n = rng() & 0x7FFFFFFFu;
        FastDiv f = make_fastdiv(d);
        if (fastdiv_host(n, f) != n / d) { std::printf("FAIL d=%u n=%u\n", d, n); return 1; }
        ++checked;
    }
    for (uint32_t d : {1u, 2u, 3u, 7u, 1000u}) {
        FastDiv f = make_fastdiv(d);
        uint32_t n = 0x7FFFFFFFu;
        if (fastdiv_host(n, f) != n / d) { std::printf("FAIL edge d=%u\n", d); return 1; }
    }
    // plans for a sweep of shapes must stay internally consistent
    for (int B : {1, 3, 64, 256}) for (int Sq : {1, 2, 77, 128, 129, 2048}) for (int Sk : {1, 63, 64, 65, 2048, 8192})
    for (int G : {1, 2, 3, 4, 8}) for (int causal : {0, 1}) for (int pk : {-1, 0, 1}) for (int ns : {0, 1, 3, 16}) {
        Shape s{B, Sq, Sk, 2 * G, 2, 128, causal};
        Plan p;
        if (make_plan(s, pk, ns, 256, &p) != GQA_OK) { std::printf("plan failed\n"); return 1; }
        if (p.ns < 1 || p.ns > (p.key_tiles > 0 ? p.key_tiles : 1)) { std::printf("bad ns\n"); return 1; }
        if ((long long)p.row_tiles * p.block_m < p.R || (long long)(p.row_tiles - 1) * p.block_m >= p.R) { std::printf("bad row tiles\n"); return 1; }
        if (p.decode != (p.R <= kDecBlockM)) { std::printf("bad kernel choice\n"); return 1; }
        const long long items8 = (long long)B * p.units_per_b * ((p.R + kPPBlockM - 1) / kPPBlockM);
        auto kt = [&](long long r1) -> long long {  // key tiles of a row tile ending at row r1
            long long kv_end = Sk;
            if (causal) kv_end = std::min<long long>(Sk, (r1 - 1) / p.Gp + (Sk - Sq) + 1);
            return kv_end <= 0 ? 0 : (kv_end + kBlockN - 1) / kBlockN;
        };
        const bool long_items = kt(std::min<long long>(p.R, kPPBlockM)) + kt(p.R) >= 2LL * kPPMinKeyTiles;
        const bool want8 = !p.decode && p.ns == 1 && s.d == 128 && (causal || p.key_tiles >= 9) &&
                           (items8 >= 2LL * 256 || (items8 >= 256 && long_items));
        if (p.pingpong != want8) { std::printf("bad 8-wave choice\n"); return 1; }
        if (p.block_m != (p.decode ? kDecBlockM : (p.pingpong ? kPPBlockM : kBlockM))) { std::printf("bad block_m\n"); return 1; }
        if (p.threads != (p.decode ? kDecThreads : (p.pingpong ? kPPThreads : kThreads))) { std::printf("bad threads\n"); return 1; }
        // causal 8-wavefront launches pair mirrored row tiles when the pairs give every unit one
        const long long pairs = (long long)B * p.units_per_b * ((p.row_tiles + 1) / 2);
        const bool paired = p.pingpong && causal && pairs >= 256;
        if (p.pair_rows != (paired ? 1 : 0)) { std::printf("bad pairing\n"); return 1; }
        const long long tiles_per_wg = paired ? (p.row_tiles + 1) / 2 : p.row_tiles;
        if (p.grid != (long long)B * p.units_per_b * tiles_per_wg * p.ns) { std::printf("bad grid\n"); return 1; }
    }
    // fp8 K/V decode splits up to two workgroups per compute unit when each unit has at
    // least 256 key tiles and there are at least 32 head units, else up to four; at most
    // 128 splits, at least two 32-key tiles per split; bf16 decode up to one per compute unit
    {
        int pk = -1, ns = 0;
        Shape k8{1, 1, 131072, 32, 8, 128, 0, 1};
        choose(k8, 256, &pk, &ns);
        if (pk != 1 || ns != 128) { std::printf("bad fp8 decode split %d %d\n", pk, ns); return 1; }
        Shape k8b{8, 1, 65536, 32, 8, 128, 0, 1};
        choose(k8b, 256, &pk, &ns);
        if (ns != 8) { std::printf("bad fp8 decode split B=8 %d\n", ns); return 1; }
        Shape k8d{64, 1, 8192, 32, 8, 128, 0, 1};  // 512 key tiles per compute unit: two workgroups each
        choose(k8d, 256, &pk, &ns);
        if (ns != 1) { std::printf("bad fp8 decode split B=64 %d\n", ns); return 1; }
        Shape k8e{1, 1, 262144, 32, 8, 128, 0, 1};  // 256 tiles per unit but 8 head units: four each
        choose(k8e, 256, &pk, &ns);
        if (ns != 128) { std::printf("bad fp8 decode split 1 x 256K %d\n", ns); return 1; }
        Shape k8c{1, 1, 2048, 32, 8, 128, 0, 1};
        choose(k8c, 256, &pk, &ns);
        if (ns != 32) { std::printf("bad fp8 decode split short %d\n", ns); return 1; }
        Shape b16{1, 1, 131072, 32, 8, 128, 0};
        choose(b16, 256, &pk, &ns);
        if (ns != 32) { std::printf("bad bf16 decode split %d\n", ns); return 1; }
    }
    std::printf("ok %lld\n", checked);
    return 0;
}
"""


def test_fastdiv_and_plan_under_sanitizers(tmp_path):
    """The magic-number divide equals n / d (exhaustive for d <= 64, n < 2^20; random up to 2^31),
    and launch plans stay consistent, in a g++ build with AddressSanitizer and UBSan."""
    csrc = os.path.join(ROOT, "grouped_query_exact_amd", "csrc")
    src = tmp_path / "t.cpp"
    src.write_text(CPP_TEST.replace('"host_logic.h"', f'"{csrc}/host_logic.h"')
                   .replace('"../../include/gqa_attn.h"', f'"{ROOT}/include/gqa_attn.h"'))
    exe = tmp_path / "t"
    cmd = ["g++", "-std=c++17", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           str(src), os.path.join(csrc, "host_logic.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
