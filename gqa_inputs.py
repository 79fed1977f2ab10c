"""Seeded synthetic inputs for the grouped-query attention forward pass.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
smoke check and the benchmark. It draws random numbers and names workload
shapes; it holds none of the attention arithmetic.

Recipe: every tensor (q=0, k=1, v=2) of every batch element b has its own
CPU generator seeded with ``seed * 1_000_000 + tensor * 100_000 + b``. A
draw is ``randn([S, H, d], float32)`` rounded to bfloat16 (round to nearest
even). Any batch element can therefore be regenerated on its own, which is
what the full-size parity checks do.

The workload shapes follow the pages: Hq=6/Hk=2 is the worked head-grouping
example (Stable-Diffusion GQA guide, "core principle" section; batch-sensitivity
article, "technical principle" section), Hq=32/Hk=8/d=128 is the Llama-2 GQA
configuration (Llama-2 GQA article, section 3.1) and the H100 batch sweep
(GQA throughput rise-and-fall article, "symptom" table), length 77 with batch
16384 // 77 = 212 is the text-encoder case of the batch formula
(Stable-Diffusion GQA guide, "dynamic batch scheduling" section).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Iterable, Optional, Sequence

import torch

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Sq: int
    Sk: int
    Hq: int
    Hk: int
    d: int
    causal: bool
    seed: int
    # (pack_gqa, num_splits) variants the parity tests run on this workload
    variants: tuple = field(default=((1, 1), (0, 1)))

    @property
    def scale(self) -> float:
        """Default softmax scale 1/sqrt(d), rounded to fp32 (the ABI passes fp32)."""
        return fp32(1.0 / math.sqrt(self.d))

    @property
    def flops(self) -> float:
        """4*B*Hq*Sq*Sk*d, halved when causal (the metric's formula)."""
        f = 4.0 * self.B * self.Hq * self.Sq * self.Sk * self.d
        return f / 2 if self.causal else f

    @property
    def io_bytes(self) -> int:
        """Q + K + V + O (bf16) + LSE (fp32), each touched once."""
        q = self.B * self.Sq * self.Hq * self.d * 2
        kv = 2 * self.B * self.Sk * self.Hk * self.d * 2
        lse = self.B * self.Hq * self.Sq * 4
        return 2 * q + kv + lse

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def fp32(x: float) -> float:
    """Round a Python float to the nearest fp32 value."""
    return float(torch.tensor(x, dtype=torch.float32).item())


# The five workloads: tiny, Llama-2-7B prefill, the batch sweep, short ragged
# sequences and split-KV decode.
TINY = Workload("tiny_hq6_hk2_d64_s128", 1, 128, 128, 6, 2, 64, True, 1001,
                ((1, 1), (0, 1), (1, 2), (0, 2)))
LLAMA_PREFILL = Workload("llama2_prefill_b4_s2048", 4, 2048, 2048, 32, 8, 128, True, 2001,
                         ((1, 1), (0, 1)))


def sweep(B: int) -> Workload:
    return Workload(f"sweep_b{B}_s2048", B, 2048, 2048, 32, 8, 128, True, 3000 + B,
                    ((1, 1), (0, 4)))


SWEEP_BATCHES = (16, 64, 128, 256)
RAGGED = Workload("ragged_b212_s77", 212, 77, 77, 6, 2, 64, False, 4001, ((1, 1), (0, 1)))
DECODE = Workload("decode_b64_sk8192", 64, 1, 8192, 32, 8, 128, False, 5001,
                  ((1, 1), (1, 4), (1, 8), (0, 4)))

ALL = [TINY, TINY.with_(causal=False, name="tiny_hq6_hk2_d64_s128_noncausal"), LLAMA_PREFILL] + \
      [sweep(b) for b in SWEEP_BATCHES] + [RAGGED, DECODE]


def _gen(seed: int, tensor: int, b: int, shape: Sequence[int], std: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1_000_000 + tensor * 100_000 + b)
    x = torch.randn(list(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def batch_slice(seed: int, b: int, Sq: int, Sk: int, Hq: int, Hk: int, d: int, std: float = 1.0):
    """q [Sq,Hq,d], k [Sk,Hk,d], v [Sk,Hk,d] bf16 CPU tensors of batch element b."""
    q = _gen(seed, TENSOR_Q, b, (Sq, Hq, d), std)
    k = _gen(seed, TENSOR_K, b, (Sk, Hk, d), std)
    v = _gen(seed, TENSOR_V, b, (Sk, Hk, d))
    return q, k, v


def make_qkv(w: Workload, batches: Optional[Iterable[int]] = None, std: float = 1.0):
    """Full bf16 CPU tensors q [B,Sq,Hq,d], k/v [B,Sk,Hk,d] (or only the listed batches)."""
    bs = list(range(w.B)) if batches is None else list(batches)
    q = torch.empty((len(bs), w.Sq, w.Hq, w.d), dtype=torch.bfloat16)
    k = torch.empty((len(bs), w.Sk, w.Hk, w.d), dtype=torch.bfloat16)
    v = torch.empty((len(bs), w.Sk, w.Hk, w.d), dtype=torch.bfloat16)
    for i, b in enumerate(bs):
        q[i], k[i], v[i] = batch_slice(w.seed, b, w.Sq, w.Sk, w.Hq, w.Hk, w.d, std)
    return q, k, v


def make_qkv_device(w: Workload, device, std: float = 1.0):
    """Generate batch by batch on the CPU and copy into device tensors."""
    q = torch.empty((w.B, w.Sq, w.Hq, w.d), dtype=torch.bfloat16, device=device)
    k = torch.empty((w.B, w.Sk, w.Hk, w.d), dtype=torch.bfloat16, device=device)
    v = torch.empty((w.B, w.Sk, w.Hk, w.d), dtype=torch.bfloat16, device=device)
    for b in range(w.B):
        qb, kb, vb = batch_slice(w.seed, b, w.Sq, w.Sk, w.Hq, w.Hk, w.d, std)
        q[b].copy_(qb)
        k[b].copy_(kb)
        v[b].copy_(vb)
    return q, k, v


def random_bf16(seed: int, shape: Sequence[int], std: float = 1.0) -> torch.Tensor:
    """One seeded bf16 tensor of any shape (edge-case tests)."""
    return _gen(seed, 0, 0, shape, std)


@dataclass
class PagedKV:
    """A paged K/V cache: ``k_cache``/``v_cache`` [num_pages, page_size, Hk, d] bf16,
    ``block_table`` [B, max_pages] int32, ``seqlens_k`` [B] int32 (CPU tensors)."""
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seqlens_k: torch.Tensor

    def to(self, device) -> "PagedKV":
        return PagedKV(self.k_cache.to(device), self.v_cache.to(device), self.block_table.to(device),
                       self.seqlens_k.to(device))


def paged_kv(seed: int, seqlens: Sequence[int], page_size: int, Hk: int, d: int, spare_pages: int = 2,
             max_pages: Optional[int] = None, fill: float = float("nan")) -> PagedKV:
    """A seeded paged K/V cache holding sequences of the given key lengths.

    Sequence b owns ceil(seqlens[b] / page_size) pages of the pool, handed out
    in a seeded random order; key j of sequence b is row j % page_size of page
    block_table[b, j // page_size]. Its keys and values are the draws of
    batch_slice for batch element b (tensors 1 and 2, shape [seqlens[b], Hk, d]).
    Page rows that hold no key (the tail of each last page and ``spare_pages``
    unused pages) are set to ``fill`` and table entries past a sequence's last
    page are -1, so a reader that touches anything else shows it.
    """
    lens = [int(n) for n in seqlens]
    need = [-(-n // page_size) for n in lens]
    mp = max(max(need) if need else 1, 1) if max_pages is None else int(max_pages)
    num_pages = sum(need) + spare_pages
    order = torch.randperm(max(num_pages, 1), generator=torch.Generator().manual_seed(seed * 7919 + 13))
    k_cache = torch.full((max(num_pages, 1), page_size, Hk, d), fill, dtype=torch.bfloat16)
    v_cache = torch.full_like(k_cache, fill)
    table = torch.full((len(lens), mp), -1, dtype=torch.int32)
    nxt = 0
    for b, n in enumerate(lens):
        kb = _gen(seed, TENSOR_K, b, (n, Hk, d))
        vb = _gen(seed, TENSOR_V, b, (n, Hk, d))
        for p in range(need[b]):
            page = int(order[nxt])
            nxt += 1
            table[b, p] = page
            rows = min(page_size, n - p * page_size)
            k_cache[page, :rows] = kb[p * page_size:p * page_size + rows]
            v_cache[page, :rows] = vb[p * page_size:p * page_size + rows]
    return PagedKV(k_cache, v_cache, table, torch.tensor(lens, dtype=torch.int32))


def random_fp8(seed: int, shape: Sequence[int], std: float = 1.0) -> torch.Tensor:
    """Seeded fp8 e4m3 bytes (uint8): N(0, std^2) draws rounded to float8_e4m3fn."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1_000_003 + 17)
    x = torch.randn(list(shape), generator=g, dtype=torch.float32) * std
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def to_fp8_bytes(x: torch.Tensor) -> torch.Tensor:
    """Round a tensor to float8_e4m3fn and return its bytes (uint8), e.g. a paged pool (NaN stays NaN)."""
    return x.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


def varlen_batch(seed: int, seqlens_q: Sequence[int], seqlens_k: Sequence[int], Hq: int, Hk: int, d: int):
    """Packed variable-length inputs: q [total_q, Hq, d], k/v [total_k, Hk, d] bf16 and int32
    cu_seqlens_q / cu_seqlens_k [B+1]. Sequence b's tokens are the draws of batch_slice for
    batch element b, so a sequence can be regenerated on its own."""
    qs, ks, vs = [], [], []
    for b, (nq, nk) in enumerate(zip(seqlens_q, seqlens_k)):
        qb, kb, vb = batch_slice(seed, b, int(nq), int(nk), Hq, Hk, d)
        qs.append(qb)
        ks.append(kb)
        vs.append(vb)
    cu = lambda lens: torch.tensor([0] + list(torch.tensor([int(x) for x in lens]).cumsum(0).tolist()), dtype=torch.int32)
    return torch.cat(qs), torch.cat(ks), torch.cat(vs), cu(seqlens_q), cu(seqlens_k)
