"""Exact grouped-query attention forward pass on AMD MI355X (gfx950).

A thin ctypes binding over the C-ABI library ``libgqa_attn.so`` built from
``csrc/`` (declared in ``include/gqa_attn.h``). The functions keep the C
names; they only turn torch tensors into pointers and sizes. Every step of
the computation runs in the library's HIP kernels: there is no fallback, and
a missing library raises at the first call.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = ["GqaAttnError", "gqa_attn_fwd", "gqa_attn_fwd_noalloc", "gqa_attn_func", "gqa_attn_fwd_paged", "gqa_attn_func_paged",
           "gqa_attn_fwd_kv8", "gqa_attn_fwd_paged_kv8", "gqa_attn_fwd_qk8", "gqa_attn_fwd_varlen", "gqa_attn_bwd",
           "gqa_attn_choose", "gqa_attn_plan",
           "gqa_attn_strerror", "library_path", "load_library",
           "GQA_OK", "GQA_ERR_INVALID_ARG", "GQA_ERR_UNSUPPORTED", "GQA_ERR_NOMEM", "GQA_ERR_HIP",
           "GQA_ERR_SCRATCH", "GQA_NOALLOC_SCRATCH_BYTES"]

GQA_OK = 0
GQA_ERR_INVALID_ARG = -1
GQA_ERR_UNSUPPORTED = -2
GQA_ERR_NOMEM = -3
GQA_ERR_HIP = -4
GQA_ERR_SCRATCH = -5
GQA_NOALLOC_SCRATCH_BYTES = 64 << 20  # fixed split-KV workspace of gqa_attn_fwd_noalloc, per GPU

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libgqa_attn.so")


class _Plan(ctypes.Structure):
    _fields_ = [("pack_gqa", ctypes.c_int), ("num_splits", ctypes.c_int), ("block_m", ctypes.c_int),
                ("block_n", ctypes.c_int), ("row_tiles", ctypes.c_int), ("key_tiles", ctypes.c_int),
                ("grid", ctypes.c_longlong), ("combine_grid", ctypes.c_longlong),
                ("workspace_bytes", ctypes.c_longlong), ("threads", ctypes.c_int)]


class GqaAttnError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"gqa_attn: {gqa_attn_strerror(status)} (status {status}){': ' + what if what else ''}")


def load_library():
    """Load libgqa_attn.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m grouped_query_exact_amd.build`")
    lib = ctypes.CDLL(path)
    c_int, c_float, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.gqa_attn_fwd.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 7 + [c_float, c_int, c_int, vp]
    lib.gqa_attn_fwd.restype = c_int
    lib.gqa_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 7 + [c_float, c_int, c_int, vp]
    lib.gqa_attn_fwd_noalloc.restype = c_int
    lib.gqa_attn_fwd_paged.argtypes = [vp] * 7 + [c_int] * 8 + [c_int, c_float, c_int, c_int, vp]
    lib.gqa_attn_fwd_paged.restype = c_int
    lib.gqa_attn_fwd_kv8.argtypes = [vp] * 3 + [c_float, c_float] + [vp, vp] + [c_int] * 7 + [c_float, c_int, c_int, vp]
    lib.gqa_attn_fwd_kv8.restype = c_int
    lib.gqa_attn_fwd_qk8.argtypes = [vp] * 3 + [c_float, c_float] + [vp, vp] + [c_int] * 7 + [c_float, c_int, c_int, vp]
    lib.gqa_attn_fwd_qk8.restype = c_int
    lib.gqa_attn_fwd_paged_kv8.argtypes = [vp] * 3 + [c_float, c_float] + [vp] * 4 + [c_int] * 8 + \
        [c_int, c_float, c_int, c_int, vp]
    lib.gqa_attn_fwd_paged_kv8.restype = c_int
    lib.gqa_attn_fwd_varlen.argtypes = [vp] * 7 + [c_int] * 8 + [c_int, c_float, c_int, c_int, vp]
    lib.gqa_attn_fwd_varlen.restype = c_int
    lib.gqa_attn_bwd.argtypes = [vp] * 9 + [c_int] * 7 + [c_float, vp]
    lib.gqa_attn_bwd.restype = c_int
    lib.gqa_attn_choose.argtypes = [c_int] * 8 + [ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
    lib.gqa_attn_choose.restype = c_int
    lib.gqa_attn_plan.argtypes = [c_int] * 10 + [ctypes.POINTER(_Plan)]
    lib.gqa_attn_plan.restype = c_int
    lib.gqa_attn_strerror.argtypes = [c_int]
    lib.gqa_attn_strerror.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def gqa_attn_strerror(status: int) -> str:
    return load_library().gqa_attn_strerror(int(status)).decode()


def gqa_attn_choose(B: int, Sq: int, Sk: int, Hq: int, Hk: int, d: int, causal: bool,
                    num_cus: int = 0) -> Tuple[int, int]:
    """The library's heuristic: (pack_gqa, num_splits)."""
    pk, ns = ctypes.c_int(), ctypes.c_int()
    st = load_library().gqa_attn_choose(B, Sq, Sk, Hq, Hk, d, int(bool(causal)), num_cus,
                                        ctypes.byref(pk), ctypes.byref(ns))
    if st != GQA_OK:
        raise GqaAttnError(st)
    return pk.value, ns.value


def gqa_attn_plan(B: int, Sq: int, Sk: int, Hq: int, Hk: int, d: int, causal: bool,
                  pack_gqa: int = -1, num_splits: int = 0, num_cus: int = 0) -> dict:
    """The launch plan gqa_attn_fwd would use for these sizes."""
    p = _Plan()
    st = load_library().gqa_attn_plan(B, Sq, Sk, Hq, Hk, d, int(bool(causal)), pack_gqa, num_splits,
                                      num_cus, ctypes.byref(p))
    if st != GQA_OK:
        raise GqaAttnError(st)
    return {name: getattr(p, name) for name, _ in _Plan._fields_}


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def gqa_attn_fwd(q, k, v, out, lse, causal: bool, scale: float, pack_gqa: int = -1,
                 num_splits: int = 0, stream=None) -> None:
    """Run the forward pass into caller-provided ``out`` (and ``lse`` or None).

    q/out: [B, Sq, Hq, d] bf16, k/v: [B, Sk, Hk, d] bf16, lse: [B, Hq, Sq] fp32,
    all contiguous on the same GPU. ``stream`` defaults to torch's current stream.
    """
    _fwd_call("gqa_attn_fwd", q, k, v, out, lse, causal, scale, pack_gqa, num_splits, stream)


def gqa_attn_fwd_noalloc(q, k, v, out, lse, causal: bool, scale: float, pack_gqa: int = -1,
                         num_splits: int = 0, stream=None) -> None:
    """gqa_attn_fwd that never allocates: split calls keep their partials in the
    library's fixed per-GPU scratch array (GQA_NOALLOC_SCRATCH_BYTES); a call that
    needs more raises GqaAttnError(GQA_ERR_SCRATCH). Split calls that overlap in
    time on one GPU share that array and race."""
    _fwd_call("gqa_attn_fwd_noalloc", q, k, v, out, lse, causal, scale, pack_gqa, num_splits, stream)


def _fwd_call(entry, q, k, v, out, lse, causal, scale, pack_gqa, num_splits, stream):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4 or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 4-d bfloat16 GPU tensor")
    B, Sq, Hq, d = q.shape
    _, Sk, Hk, _ = k.shape
    if tuple(k.shape) != (B, Sk, Hk, d) or tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v and out")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_cuda):
        raise ValueError("lse must be a contiguous [B, Hq, Sq] float32 GPU tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    with torch.cuda.device(q.device):
        st = getattr(load_library(), entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                            B, Sq, Sk, Hq, Hk, d, int(bool(causal)), float(scale),
                                            int(pack_gqa), int(num_splits), stream)
    if st != GQA_OK:
        raise GqaAttnError(st)


def gqa_attn_func(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None,
                  pack_gqa: int = -1, num_splits: int = 0, return_lse: bool = False):
    """Allocate the outputs and run gqa_attn_fwd. softmax_scale defaults to 1/sqrt(d)."""
    import torch
    B, Sq, Hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    gqa_attn_fwd(q, k, v, out, lse, causal, softmax_scale, pack_gqa, num_splits)
    return (out, lse) if return_lse else out


def _check_kv8(**tensors):
    import torch
    for name, t in tensors.items():
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or not t.is_contiguous() or t.dim() != 4 or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 4-d GPU tensor of float8_e4m3fn (or uint8) bytes")


def _check_bf16(**tensors):
    import torch
    for name, t in tensors.items():
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4 or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 4-d bfloat16 GPU tensor")


def gqa_attn_fwd_kv8(q, k, v, k_scale: float, v_scale: float, out, lse, causal: bool, scale: float,
                     pack_gqa: int = -1, num_splits: int = 0, stream=None) -> None:
    """Forward pass with fp8 e4m3 K/V ([B, Sk, Hk, d] bytes) and per-tensor factors, into ``out``/``lse``."""
    import torch
    _check_bf16(q=q, out=out)
    _check_kv8(k=k, v=v)
    B, Sq, Hq, d = q.shape
    _, Sk, Hk, _ = k.shape
    if tuple(k.shape) != (B, Sk, Hk, d) or tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v and out")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_cuda):
        raise ValueError("lse must be a contiguous [B, Hq, Sq] float32 GPU tensor")
    stream = _stream(q, stream)
    with torch.cuda.device(q.device):
        st = load_library().gqa_attn_fwd_kv8(_ptr(q), _ptr(k), _ptr(v), float(k_scale), float(v_scale), _ptr(out),
                                             _ptr(lse), B, Sq, Sk, Hq, Hk, d, int(bool(causal)), float(scale),
                                             int(pack_gqa), int(num_splits), stream)
    if st != GQA_OK:
        raise GqaAttnError(st)


def gqa_attn_fwd_qk8(q, k, v, q_scale: float, k_scale: float, out, lse, causal: bool, scale: float,
                     pack_gqa: int = -1, num_splits: int = 0, stream=None) -> None:
    """Forward pass with fp8 e4m3 Q ([B, Sq, Hq, d] bytes) and K ([B, Sk, Hk, d] bytes) with per-tensor
    factors and bf16 V, into ``out``/``lse``: the scores run on the fp8 matrix cores."""
    import torch
    _check_kv8(q=q, k=k)
    _check_bf16(v=v, out=out)
    B, Sq, Hq, d = q.shape
    _, Sk, Hk, _ = k.shape
    if tuple(k.shape) != (B, Sk, Hk, d) or tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v and out")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_cuda):
        raise ValueError("lse must be a contiguous [B, Hq, Sq] float32 GPU tensor")
    stream = _stream(q, stream)
    with torch.cuda.device(q.device):
        st = load_library().gqa_attn_fwd_qk8(_ptr(q), _ptr(k), _ptr(v), float(q_scale), float(k_scale), _ptr(out),
                                             _ptr(lse), B, Sq, Sk, Hq, Hk, d, int(bool(causal)), float(scale),
                                             int(pack_gqa), int(num_splits), stream)
    if st != GQA_OK:
        raise GqaAttnError(st)


def _stream(q, stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream(q.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check_paged(q, k_cache, block_table, seqlens_k, lse):
    import torch
    B, Sq, Hq, d = q.shape
    if (block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B
            or not block_table.is_contiguous() or not block_table.is_cuda):
        raise ValueError("block_table must be a contiguous [B, max_pages] int32 GPU tensor")
    if (seqlens_k.dtype != torch.int32 or tuple(seqlens_k.shape) != (B,) or not seqlens_k.is_contiguous()
            or not seqlens_k.is_cuda):
        raise ValueError("seqlens_k must be a contiguous [B] int32 GPU tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_cuda):
        raise ValueError("lse must be a contiguous [B, Hq, Sq] float32 GPU tensor")


def gqa_attn_fwd_paged_kv8(q, k_cache, v_cache, k_scale: float, v_scale: float, block_table, seqlens_k, out, lse,
                           causal: bool, scale: float, pack_gqa: int = -1, num_splits: int = 0, stream=None) -> None:
    """gqa_attn_fwd_paged over fp8 e4m3 page pools with per-tensor factors."""
    import torch
    _check_bf16(q=q, out=out)
    _check_kv8(k_cache=k_cache, v_cache=v_cache)
    B, Sq, Hq, d = q.shape
    num_pages, page_size, Hk, dk = k_cache.shape
    if dk != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k_cache, v_cache and out")
    _check_paged(q, k_cache, block_table, seqlens_k, lse)
    stream = _stream(q, stream)
    with torch.cuda.device(q.device):
        st = load_library().gqa_attn_fwd_paged_kv8(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale),
                                                   float(v_scale), _ptr(block_table), _ptr(seqlens_k), _ptr(out),
                                                   _ptr(lse), B, Sq, Hq, Hk, d, num_pages, page_size,
                                                   block_table.shape[1], int(bool(causal)), float(scale),
                                                   int(pack_gqa), int(num_splits), stream)
    if st != GQA_OK:
        raise GqaAttnError(st)


def gqa_attn_fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, out, lse, causal: bool, scale: float,
                       pack_gqa: int = -1, num_splits: int = 0, stream=None) -> None:
    """Run the forward pass over a paged KV cache into ``out`` (and ``lse`` or None).

    q/out: [B, Sq, Hq, d] bf16; k_cache/v_cache: [num_pages, page_size, Hk, d] bf16;
    block_table: [B, max_pages] int32; seqlens_k: [B] int32; lse: [B, Hq, Sq] fp32.
    All contiguous on the same GPU.
    """
    import torch
    _check_bf16(q=q, k_cache=k_cache, v_cache=v_cache, out=out)
    B, Sq, Hq, d = q.shape
    num_pages, page_size, Hk, dk = k_cache.shape
    if dk != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k_cache, v_cache and out")
    _check_paged(q, k_cache, block_table, seqlens_k, lse)
    stream = _stream(q, stream)
    with torch.cuda.device(q.device):
        st = load_library().gqa_attn_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                               _ptr(seqlens_k), _ptr(out), _ptr(lse), B, Sq, Hq, Hk, d,
                                               num_pages, page_size, block_table.shape[1], int(bool(causal)),
                                               float(scale), int(pack_gqa), int(num_splits), stream)
    if st != GQA_OK:
        raise GqaAttnError(st)


def gqa_attn_func_paged(q, k_cache, v_cache, block_table, seqlens_k, causal: bool = False,
                        softmax_scale: Optional[float] = None, pack_gqa: int = -1, num_splits: int = 0,
                        return_lse: bool = False):
    """Allocate the outputs and run gqa_attn_fwd_paged. softmax_scale defaults to 1/sqrt(d)."""
    import torch
    B, Sq, Hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    gqa_attn_fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, out, lse, causal, softmax_scale, pack_gqa,
                       num_splits)
    return (out, lse) if return_lse else out


def gqa_attn_fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                        causal: bool, scale: float, pack_gqa: int = -1, num_splits: int = 0, stream=None) -> None:
    """Forward pass over packed variable-length sequences.

    q/out: [total_q, Hq, d] bf16; k/v: [total_k, Hk, d] bf16; lse: [Hq, total_q] fp32 or None;
    cu_seqlens_q / cu_seqlens_k: [B+1] int32 cumulative lengths. All contiguous on the same GPU.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 3 or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 3-d bfloat16 GPU tensor")
    total_q, Hq, d = q.shape
    total_k, Hk, dk = k.shape
    if dk != d or tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v and out")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 1-d int32 GPU tensor")
    if cu_seqlens_k.shape[0] != cu_seqlens_q.shape[0]:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length B+1")
    B = cu_seqlens_q.shape[0] - 1
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (Hq, total_q) or not lse.is_cuda):
        raise ValueError("lse must be a contiguous [Hq, total_q] float32 GPU tensor")
    stream = _stream(q, stream)
    with torch.cuda.device(q.device):
        st = load_library().gqa_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                                _ptr(cu_seqlens_k), B, int(max_seqlen_q), int(max_seqlen_k), total_q,
                                                total_k, Hq, Hk, d, int(bool(causal)), float(scale), int(pack_gqa),
                                                int(num_splits), stream)
    if st != GQA_OK:
        raise GqaAttnError(st)


def gqa_attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, causal: bool, scale: float, stream=None) -> None:
    """Gradients of the forward pass into ``dq``, ``dk``, ``dv`` (caller-allocated).

    q/out/dout/dq: [B, Sq, Hq, d] bf16; k/v/dk/dv: [B, Sk, Hk, d] bf16; lse: [B, Hq, Sq] fp32 from the
    forward call on the same inputs. All contiguous on the same GPU.
    """
    import torch
    _check_bf16(q=q, k=k, v=v, out=out, dout=dout, dq=dq, dk=dk, dv=dv)
    B, Sq, Hq, d = q.shape
    _, Sk, Hk, _ = k.shape
    for name, t, shape in (("out", out, q.shape), ("dout", dout, q.shape), ("dq", dq, q.shape),
                           ("v", v, k.shape), ("dk", dk, k.shape), ("dv", dv, k.shape)):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has the wrong shape")
    if tuple(k.shape) != (B, Sk, Hk, d):
        raise ValueError("k must be [B, Sk, Hk, d]")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_cuda:
        raise ValueError("lse must be a contiguous [B, Hq, Sq] float32 GPU tensor")
    stream = _stream(q, stream)
    with torch.cuda.device(q.device):
        st = load_library().gqa_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                         _ptr(dk), _ptr(dv), B, Sq, Sk, Hq, Hk, d, int(bool(causal)), float(scale),
                                         stream)
    if st != GQA_OK:
        raise GqaAttnError(st)
