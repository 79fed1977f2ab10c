#!/usr/bin/env python3
"""Benchmark of the exact GQA forward pass on one MI355X.

Headline workload: the causal batch-sensitivity sweep shape Hq=32, Hk=8,
d=128, Sq=Sk=2048 at B=128 (the pages' H100 sweep covers B=64..256), one
gqa_attn_fwd call per step with the library's own choice of pack_gqa and
num_splits. Inputs are the seeded bf16 N(0,1) recipe of gqa_inputs, resident
in HBM before the timed region. The metric is TFLOP/s = 4*B*Hq*Sq*Sk*d/2/t
(causal) and tokens/s = B*Sq/t; `value` is the average over exactly --steps
launches between two HIP events on the launch stream.

Also measured in the same run and reported in the same JSON line (unless
--quick), each as the median (and minimum) of >= 20 individually timed calls
after warm-up. Before the headline: split-KV decode (B=64, Sq=1, Sk=8192;
ns = auto, 1, 4, 8 and pack off) as HBM GB/s of Q+K+V+O+LSE bytes, the same
decode over a paged cache and with fp8 K/V; the tiny workload (B=1, Hq=6,
Hk=2, d=64, S=128, causal and not, pack on and off) and the short ragged
workload (B=212, S=77, pack on and off, GB/s and the pack speedup), both
timed with a 512 MiB write between calls so that no input stays in the
caches. After the headline: the Llama-2 prefill shape (B=4); the whole batch sweep (B = 16, 64,
128, 256 with (pack 1, ns 1), (pack 0, ns 4) and auto); the headline shape
with fp8 Q and K (rated against the mixed fp8/bf16 peak); a variable-length
prefill batch next to an equal-token batched call; and the backward pass at
the Llama-2 shape. Those inputs are drawn on the GPU from N(0,1) (timing
does not depend on the values' seeds).

cpu_baseline: the fp64 numpy oracle as it stands, on this host's cores
(BLAS threads = the CPUs this process may run on), on whole batch elements of
the headline workload until >= --cpu-seconds of CPU work, scaled to the same
metric; the tiny, ragged and decode workloads are timed in full, on all cores
and on one core, and the Llama-2 and sweep configurations are extrapolated
from the headline's per-element time (same per-element shape).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
FLUSH_BYTES = 512 << 20    # written between calls of the sub-cache workloads (MALL is 256 MiB)
# the forward kernels' sources: the traffic counters are valid while these are unchanged
KERNEL_SRCS = [os.path.join(ROOT, "grouped_query_exact_amd", "csrc", f)
               for f in ("gqa_attn_kernels.hip", "device_common.h", "kernels.h", "host_logic.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_calls(fn, steps: int, warmup: int, flush=None, warmup_s: float = 0.3):
    """Per-call times of fn (ms): HIP events around each call on torch's current stream.

    Warm-up: at least `warmup` calls and at least `warmup_s` seconds of them
    (at most 400 calls), so short calls are timed at the GPU's steady clock.
    flush (optional) runs before each call, outside the events. Returns
    {"median": ..., "min": ..., "mean": ..., "n": steps}.
    """
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0 < warmup_s and n < 400):
        if flush is not None:
            flush()
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        if flush is not None:
            flush()
        e0.record(st)
        fn()
        e1.record(st)
    torch.cuda.synchronize()
    ts = [e0.elapsed_time(e1) for e0, e1 in ev]
    return {"median": statistics.median(ts), "min": min(ts), "mean": sum(ts) / len(ts), "n": len(ts)}


def gpu_randn(shape, gen, device):
    import torch
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def gpu_randn_inputs(w, device, seed):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return (gpu_randn((w.B, w.Sq, w.Hq, w.d), gen, device), gpu_randn((w.B, w.Sk, w.Hk, w.d), gen, device),
            gpu_randn((w.B, w.Sk, w.Hk, w.d), gen, device))


def fwd_timer(g, w, q, k, v, pack, ns, steps, warmup, flush=None):
    import torch
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], w.Hq, w.Sq), dtype=torch.float32, device=q.device)

    def fn():
        g.gqa_attn_fwd(q, k, v, out, lse, w.causal, w.scale, pack, ns)
    t = time_calls(fn, steps, warmup, flush)
    plan = g.gqa_attn_plan(q.shape[0], w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, pack, ns)
    return t, plan


def rate_entry(t, flops=None, nbytes=None, peak_tflops=PEAK_BF16_TFLOPS, **kw):
    ms = t["median"]
    e = {"ms_median": round(ms, 5), "ms_min": round(t["min"], 5), "calls": t["n"]}
    if flops is not None:
        e["tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        e["frac_peak"] = round(flops / (ms * 1e-3) / 1e12 / peak_tflops, 4)
    if nbytes is not None:
        e["GB_per_s"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        e["frac_hbm_peak"] = round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    e.update(kw)
    return e


# ------------------------------------------------------------------- extras
def extra_decode(g, gi, dev, steps):
    import torch
    wd = gi.DECODE
    qd, kd, vd = gpu_randn_inputs(wd, dev, 9)
    dec = {}
    for pack, ns in ((-1, 0), (1, 1), (1, 4), (1, 8), (0, 4)):
        t, pl = fwd_timer(g, wd, qd, kd, vd, pack, ns, steps, 5)
        name = f"pack{pl['pack_gqa']}_ns{pl['num_splits']}" + ("_auto" if pack < 0 else "")
        dec[name] = rate_entry(t, nbytes=wd.io_bytes,
                               kernel="attn_decode_kernel" + (" + combine_kernel" if pl["num_splits"] > 1 else ""))
        log(f"decode pack={pack} ns={ns}: median {t['median'] * 1e3:.1f} us")
    # the split calls through the entry point that allocates nothing: the
    # partials live in the library's fixed device array, so a call enqueues
    # no stream-ordered allocation and release (each of which leaves the GPU
    # idle for a few microseconds between calls)
    od = torch.empty_like(qd)
    ld = torch.empty((wd.B, wd.Hq, wd.Sq), dtype=torch.float32, device=dev)
    for ns in (4, 8):
        t = time_calls(lambda: g.gqa_attn_fwd_noalloc(qd, kd, vd, od, ld, wd.causal, wd.scale, 1, ns), steps, 5)
        dec[f"pack1_ns{ns}_noalloc"] = rate_entry(t, nbytes=wd.io_bytes,
                                                  kernel="attn_decode_kernel + combine_kernel (gqa_attn_fwd_noalloc)")
        log(f"decode pack=1 ns={ns} no-allocation entry point: median {t['median'] * 1e3:.1f} us")
    del kd, vd
    out = {"decode_b64_sk8192": dec}
    # the same decode over a paged cache: pages of 256 keys in random pool order
    ps = 256
    P = wd.Sk // ps
    gen = torch.Generator(device=dev)
    gen.manual_seed(10)
    kc = gpu_randn((wd.B * P, ps, wd.Hk, wd.d), gen, dev)
    vc = gpu_randn((wd.B * P, ps, wd.Hk, wd.d), gen, dev)
    table = torch.randperm(wd.B * P, generator=gen, device=dev).to(torch.int32).view(wd.B, P).contiguous()
    lens = torch.full((wd.B,), wd.Sk, dtype=torch.int32, device=dev)
    outp = torch.empty_like(qd)
    lsep = torch.empty((wd.B, wd.Hq, wd.Sq), dtype=torch.float32, device=dev)
    t = time_calls(lambda: g.gqa_attn_fwd_paged(qd, kc, vc, table, lens, outp, lsep, wd.causal, wd.scale), steps, 5)
    out["decode_paged_b64_sk8192_ps256"] = rate_entry(t, nbytes=wd.io_bytes, kernel="attn_decode_kernel (paged)")
    log(f"paged decode: median {t['median'] * 1e3:.1f} us")
    del kc, vc, table
    # the same decode with fp8 e4m3 K/V (half the K/V bytes)
    k8 = torch.randn((wd.B, wd.Sk, wd.Hk, wd.d), generator=gen, device=dev).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = torch.randn((wd.B, wd.Sk, wd.Hk, wd.d), generator=gen, device=dev).to(torch.float8_e4m3fn).view(torch.uint8)
    t = time_calls(lambda: g.gqa_attn_fwd_kv8(qd, k8, v8, 1.0, 1.0, outp, lsep, wd.causal, wd.scale), steps, 5)
    bytes8 = wd.io_bytes - (k8.numel() + v8.numel())  # K and V at one byte per element
    out["decode_kv8_b64_sk8192"] = rate_entry(t, nbytes=bytes8, algorithmic_bytes=bytes8,
                                              kernel="attn_decode_kernel (fp8 K/V)")
    log(f"fp8 K/V decode: median {t['median'] * 1e3:.1f} us")
    return out


def extra_small(g, gi, dev, steps):
    """The tiny and short ragged workloads, each call after a 512 MiB write (cold caches)."""
    import torch
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush = lambda: scratch.fill_(1.0)
    out = {}
    tiny = {}
    for causal in (True, False):
        w = gi.TINY.with_(causal=causal)
        q, k, v = (t.to(dev) for t in gi.make_qkv(w))
        for pack in (1, 0):
            t, pl = fwd_timer(g, w, q, k, v, pack, 1, steps, 3, flush)
            tiny[f"{'causal' if causal else 'noncausal'}_pack{pack}"] = rate_entry(
                t, flops=w.flops, nbytes=w.io_bytes, grid=pl["grid"])
            log(f"tiny causal={causal} pack={pack}: median {t['median'] * 1e3:.1f} us")
    out["tiny_b1_hq6_hk2_d64_s128"] = tiny
    w = gi.RAGGED
    q, k, v = (t.to(dev) for t in gi.make_qkv(w))
    rag = {}
    for pack in (1, 0, -1):
        t, pl = fwd_timer(g, w, q, k, v, pack, 0 if pack < 0 else 1, steps, 3, flush)
        rag[f"pack{pl['pack_gqa']}_ns{pl['num_splits']}" + ("_auto" if pack < 0 else "")] = rate_entry(
            t, flops=w.flops, nbytes=w.io_bytes, grid=pl["grid"])
        log(f"ragged pack={pack}: median {t['median'] * 1e3:.1f} us")
    rag["pack_speedup"] = round(rag["pack0_ns1"]["ms_median"] / rag["pack1_ns1"]["ms_median"], 3)
    out["ragged_b212_s77"] = rag
    out["cache_flush"] = f"{FLUSH_BYTES >> 20} MiB device write before every timed call (not timed)"
    return out


def extra_prefill(g, gi, dev, steps):
    import torch
    out = {}
    wl = gi.LLAMA_PREFILL
    ql, kl, vl = gpu_randn_inputs(wl, dev, 8)
    llama = {}
    for pack, ns in ((1, 1), (0, 1), (-1, 0)):
        t, pl = fwd_timer(g, wl, ql, kl, vl, pack, ns, steps, 5)
        llama[f"pack{pl['pack_gqa']}_ns{pl['num_splits']}" + ("_auto" if pack < 0 else "")] = rate_entry(
            t, flops=wl.flops, kernel="attn_fwd_pingpong_kernel" if pl["threads"] == 512 else "attn_fwd_kernel")
    llama["pack_speedup"] = round(llama["pack0_ns1"]["ms_median"] / llama["pack1_ns1"]["ms_median"], 3)
    out["llama_prefill_b4"] = llama
    log(f"llama prefill: {llama['pack1_ns1']['tflops']} TFLOP/s")
    del ql, kl, vl
    # the sweep: both variants and the library's choice at every batch size
    big = gi.sweep(max(gi.SWEEP_BATCHES))
    qb, kb, vb = gpu_randn_inputs(big, dev, 7)
    sweep = {}
    for B in gi.SWEEP_BATCHES:
        wb = gi.sweep(B)
        for pack, ns in tuple(wb.variants) + ((-1, 0),):
            t, pl = fwd_timer(g, wb, qb[:B], kb[:B], vb[:B], pack, ns, steps, 3)
            key = f"B{B}_auto" if pack < 0 else f"B{B}_pack{pack}_ns{ns}"
            sweep[key] = rate_entry(t, flops=wb.flops, tokens_per_s=round(B * wb.Sq / (t["median"] * 1e-3), 1),
                                    pack=pl["pack_gqa"], ns=pl["num_splits"])
            log(f"sweep B={B} pack={pack} ns={ns}: median {t['median']:.4f} ms")
    out["sweep"] = sweep
    # the headline shape with Q and K in fp8 e4m3: the score products on the fp8
    # matrix cores (half the flops at 5.0 PF), P V in bf16 (half at 2.5 PF)
    w128 = gi.sweep(128)
    q8 = qb[:128].to(torch.float8_e4m3fn).view(torch.uint8)
    k8 = kb[:128].to(torch.float8_e4m3fn).view(torch.uint8)
    o8 = torch.empty_like(qb[:128])
    l8 = torch.empty((128, w128.Hq, w128.Sq), dtype=torch.float32, device=dev)
    t = time_calls(lambda: g.gqa_attn_fwd_qk8(q8, k8, vb[:128], 1.0, 1.0, o8, l8, w128.causal, w128.scale), steps, 3)
    mixed_peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
    out["sweep_b128_fp8_qk"] = rate_entry(t, flops=w128.flops, peak_tflops=mixed_peak,
                                          peak_note=f"mixed peak {mixed_peak:.0f} TFLOP/s: QK^T at fp8 5.0 PF, "
                                                    f"P V at bf16 2.5 PF",
                                          kernel="attn_fwd_pingpong_kernel (fp8 Q/K scores, bf16 P V)")
    log(f"fp8 Q/K sweep B=128: median {t['median']:.4f} ms")
    del q8, k8, o8, l8, qb, kb, vb
    torch.cuda.empty_cache()
    # variable-length prefill: 16 packed sequences of 128 .. 2048 tokens (Llama-2 heads,
    # causal), next to a batched call of about the same tokens (8 x 2048)
    lens = [128 * (i + 1) for i in range(16)]
    tot = sum(lens)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    qv = gpu_randn((tot, wl.Hq, wl.d), gen, dev)
    kv_ = gpu_randn((tot, wl.Hk, wl.d), gen, dev)
    vv = gpu_randn((tot, wl.Hk, wl.d), gen, dev)
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int32, device=dev)
    ov = torch.empty_like(qv)
    lv = torch.empty((wl.Hq, tot), dtype=torch.float32, device=dev)
    t = time_calls(lambda: g.gqa_attn_fwd_varlen(qv, kv_, vv, ov, lv, cu, cu, max(lens), max(lens), True, wl.scale),
                   steps, 5)
    fl = sum(4.0 * wl.Hq * L * L * wl.d / 2 for L in lens)
    var = rate_entry(t, flops=fl, tokens=tot)
    wb8 = wl.with_(B=8)
    q8b, k8b, v8b = gpu_randn_inputs(wb8, dev, 13)
    tb, _ = fwd_timer(g, wb8, q8b, k8b, v8b, -1, 0, steps, 5)
    var["batched_8x2048"] = rate_entry(tb, flops=wb8.flops)
    var["ratio_to_batched"] = round(var["tflops"] / var["batched_8x2048"]["tflops"], 3)
    out["varlen_prefill_16seq_128to2048"] = var
    log(f"varlen prefill: {var['tflops']} TFLOP/s ({var['ratio_to_batched']} of batched)")
    del qv, kv_, vv, ov, lv, q8b, k8b, v8b
    # backward at the Llama-2 prefill shape (B=4, causal): dQ, dK, dV from the forward's O and LSE
    ql, kl, vl = gpu_randn_inputs(wl, dev, 12)
    dol = torch.randn_like(ql, dtype=torch.float32).to(torch.bfloat16)
    ol = torch.empty_like(ql)
    ll = torch.empty((wl.B, wl.Hq, wl.Sq), dtype=torch.float32, device=dev)
    g.gqa_attn_fwd(ql, kl, vl, ol, ll, wl.causal, wl.scale)
    dql, dkl, dvl = torch.empty_like(ql), torch.empty_like(kl), torch.empty_like(vl)
    t = time_calls(lambda: g.gqa_attn_bwd(ql, kl, vl, ol, ll, dol, dql, dkl, dvl, wl.causal, wl.scale), steps, 5)
    out["backward_llama_b4"] = rate_entry(t, flops=2.5 * wl.flops,
                                          flops_convention="2.5x forward (5 products of the causal band)")
    log(f"backward llama b4: median {t['median']:.4f} ms")
    return out


# ------------------------------------------------------------- cpu baseline
def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = f"{infos[0].get('internal_api')} {infos[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return model, blas


def _oracle_seconds(w, batches=None):
    """Wall time of the oracle on the workload's seeded inputs (whole, or the listed batch elements)."""
    import gqa_inputs as gi
    import oracle
    q, k, v = gi.make_qkv(w, batches)
    qd, kd, vd = (x.double().numpy() for x in (q, k, v))
    t0 = time.perf_counter()
    oracle.attention_fp64(qd, kd, vd, w.causal, w.scale)
    return time.perf_counter() - t0


def cpu_baseline(w, min_seconds, gpu_ms):
    """The oracle on this host: headline sample (the reported value) and every configuration."""
    import gqa_inputs as gi
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    model, blas = cpu_info()
    per_cfg = {}
    with threadpool_limits(limits=cores, user_api="blas"):
        done, t = 0, 0.0
        while done < w.B and t < min_seconds:
            t += _oracle_seconds(w, [done])
            done += 1
        per_elem = t / done
        for cfg, wc in (("tiny_causal", gi.TINY), ("tiny_noncausal", gi.TINY.with_(causal=False)),
                        ("ragged_b212_s77", gi.RAGGED), ("decode_b64_sk8192", gi.DECODE)):
            per_cfg[cfg] = {"seconds": round(_oracle_seconds(wc), 4), "threads": cores, "timed": "whole workload"}
    with threadpool_limits(limits=1, user_api="blas"):
        for cfg, wc in (("tiny_causal", gi.TINY), ("tiny_noncausal", gi.TINY.with_(causal=False)),
                        ("ragged_b212_s77", gi.RAGGED), ("decode_b64_sk8192", gi.DECODE)):
            per_cfg[cfg]["seconds_1core"] = round(_oracle_seconds(wc), 4)
    for cfg, B in (("llama2_prefill_b4_s2048", 4),) + tuple((f"sweep_b{b}_s2048", b) for b in gi.SWEEP_BATCHES):
        per_cfg[cfg] = {"seconds": round(per_elem * B, 2), "threads": cores,
                        "timed": f"extrapolated: {B} x the headline's {per_elem:.3f} s per batch element "
                                 f"(same per-element shape, {done} elements timed)"}
    for cfg, e in per_cfg.items():
        if cfg in gpu_ms:
            e["gpu_ms"] = gpu_ms[cfg]
            e["speedup_gpu_vs_oracle"] = round(e["seconds"] * 1e3 / gpu_ms[cfg], 1)
    flops = w.flops / w.B * done
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {w.B} batch elements of {w.name} (all {w.Hq} heads, {w.Sq} rows), "
                      f"{t:.1f} s, fp64 numpy, metric flops (causal-halved)",
            "cpu_model": model, "blas": blas, "blas_threads": cores,
            "tokens_per_s": done * w.Sq / t, "seconds": t, "per_config": per_cfg}


# --------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=128)
    ap.add_argument("--pack", type=int, default=-1)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--extra-steps", type=int, default=20, help="timed calls per extra measurement (>= 20)")
    ap.add_argument("--quick", action="store_true", help="headline only (no extras, no cpu baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the attention runs on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_query_exact_amd as g
    import gqa_inputs as gi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    extra = {}
    steps_x = max(20, args.extra_steps)
    if not args.quick:
        # the memory-bound and small workloads first, each after its own warm-up
        # (measured right after the compute-bound prefill they ran ~4% slower)
        extra.update(extra_decode(g, gi, dev, steps_x))
        torch.cuda.empty_cache()
        extra.update(extra_small(g, gi, dev, steps_x))
        torch.cuda.empty_cache()
    w = gi.sweep(args.batch)
    q, k, v = gi.make_qkv_device(w, dev)
    log(f"inputs ready: {w.name}")

    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)

    def step():
        g.gqa_attn_fwd(q, k, v, out, lse, w.causal, w.scale, args.pack, args.splits)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, args.pack, args.splits)
    tflops = w.flops / (ms * 1e-3) / 1e12
    log(f"headline {ms:.4f} ms/step {tflops:.1f} TFLOP/s plan={plan}")

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        # measured by bench_traffic.py for the library's choice on this workload
        if tr.get("kernel_hash") == kernel_hash() and args.pack < 0 and args.splits == 0:
            traffic = tr["entries"][w.name]["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    kernel = ("attn_fwd_pingpong_kernel<128, causal>" if plan["threads"] == 512
              else "attn_fwd_kernel<128, causal, unsplit>") if plan["num_splits"] == 1 \
        else "attn_fwd_kernel<128, causal, split> + combine_kernel"
    result = {
        "metric": "GQA fwd TFLOP/s & tokens/s (Hq32/Hk8,d128,S2K,B64-256); decode HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded bf16 N(0,1) Q/K/V resident in HBM",
        "config": {"workload": w.name, "B": w.B, "Sq": w.Sq, "Sk": w.Sk, "Hq": w.Hq, "Hk": w.Hk,
                   "d": w.d, "causal": w.causal, "pack_gqa": plan["pack_gqa"],
                   "num_splits": plan["num_splits"], "parallelism": "single GPU"},
        "tokens_per_s": round(w.B * w.Sq / (ms * 1e-3), 1),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": kernel, "flops_per_launch": w.flops,
                     "algorithmic_bytes_per_launch": w.io_bytes},
    }
    del q, k, v, out, lse
    torch.cuda.empty_cache()

    gpu_ms = {w.name: ms}
    if not args.quick:
        extra.update(extra_prefill(g, gi, dev, steps_x))
        torch.cuda.empty_cache()
        extra["timing"] = (f"median and minimum of {steps_x} individually event-timed calls after warm-up; "
                           f"decode and the small workloads before the headline, the prefill workloads after it")
        result["extra"] = extra
        gpu_ms.update({
            "tiny_causal": extra["tiny_b1_hq6_hk2_d64_s128"]["causal_pack1"]["ms_median"],
            "tiny_noncausal": extra["tiny_b1_hq6_hk2_d64_s128"]["noncausal_pack1"]["ms_median"],
            "ragged_b212_s77": extra["ragged_b212_s77"]["pack1_ns1"]["ms_median"],
            "decode_b64_sk8192": extra["decode_b64_sk8192"]["pack1_ns1_auto"]["ms_median"],
            "llama2_prefill_b4_s2048": extra["llama_prefill_b4"]["pack1_ns1_auto"]["ms_median"],
        })
        for B in gi.SWEEP_BATCHES:
            gpu_ms[f"sweep_b{B}_s2048"] = extra["sweep"][f"B{B}_auto"]["ms_median"]

    if not args.quick and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, gpu_ms)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.4f} TFLOP/s on {result['cpu_baseline']['cores']} cores")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
