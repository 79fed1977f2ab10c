#!/usr/bin/env python3
"""Benchmark of the exact GQA forward pass on one MI355X.

Headline workload: the causal batch-sensitivity sweep shape Hq=32, Hk=8,
d=128, Sq=Sk=2048 at B=128 (the pages' H100 sweep covers B=64..256), one
gqa_attn_fwd call per step with the library's own choice of pack_gqa and
num_splits. Inputs are the seeded bf16 N(0,1) recipe of gqa_inputs, resident
in HBM before the timed region. The metric is TFLOP/s = 4*B*Hq*Sq*Sk*d/2/t
(causal) and tokens/s = B*Sq/t.

Also measured in the same run and reported in the same JSON line (unless
--quick): the rest of the sweep (B = 16, 64, 128, 256 with (pack 1, ns 1)
and (pack 0, ns 4)), the Llama-2 prefill shape (B=4), and split-KV decode
(B=64, Sq=1, Sk=8192) as HBM GB/s of Q+K+V+O+LSE bytes, the same decode
over a paged cache and with fp8 K/V, the headline shape with fp8 Q and K
(scores on the fp8 matrix cores), a variable-length prefill batch, and the
backward pass at the Llama-2 shape; those inputs are drawn on the GPU
from N(0,1) (the timing does not depend on the values' seeds).

cpu_baseline: the fp64 numpy oracle on a bounded sample (the first batch
elements of the headline workload, all heads, until >= 10 s of CPU time),
on this host, scaled to the same metric.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
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


def time_calls(fn, steps: int, warmup: int):
    """Average milliseconds per call, HIP events on torch's current stream (the launch stream)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def gpu_randn_inputs(w, device, seed):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = torch.randn((w.B, w.Sq, w.Hq, w.d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((w.B, w.Sk, w.Hk, w.d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((w.B, w.Sk, w.Hk, w.d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def measure(g, w, q, k, v, pack, ns, steps, warmup):
    import torch
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=q.device)

    def fn():
        g.gqa_attn_fwd(q, k, v, out, lse, w.causal, w.scale, pack, ns)
    ms, _ = time_calls(fn, steps, warmup)
    plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, pack, ns)
    return ms, plan


def cpu_baseline(w, min_seconds=10.0, max_batches=None):
    """Time the oracle on whole batch elements of the workload until min_seconds have passed."""
    import numpy as np
    import gqa_inputs as gi
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    done, t = 0, 0.0
    nb = max_batches or w.B
    while done < nb and t < min_seconds:
        q, k, v = gi.batch_slice(w.seed, done, w.Sq, w.Sk, w.Hq, w.Hk, w.d)
        qd, kd, vd = (x.double().numpy()[None] for x in (q, k, v))
        t0 = time.perf_counter()
        oracle.attention_fp64(qd, kd, vd, w.causal, w.scale)
        t += time.perf_counter() - t0
        done += 1
    flops = w.flops / w.B * done
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {w.B} batch elements of {w.name} (all {w.Hq} heads, {w.Sq} rows), "
                      f"{t:.1f} s, fp64 numpy, metric flops (causal-halved)",
            "tokens_per_s": done * w.Sq / t, "seconds": t}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=128)
    ap.add_argument("--pack", type=int, default=-1)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--quick", action="store_true", help="headline only (no sweep, decode, cpu baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build runs the attention on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_query_exact_amd as g
    import gqa_inputs as gi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gi.sweep(args.batch)
    q, k, v = gi.make_qkv_device(w, dev)
    print(f"[bench] inputs ready: {w.name}", file=sys.stderr, flush=True)

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
    print(f"[bench] headline {ms:.4f} ms/step {tflops:.1f} TFLOP/s plan={plan}", file=sys.stderr, flush=True)

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        key = f"{w.name}|pack{plan['pack_gqa']}|ns{plan['num_splits']}"
        if tr.get("kernel_hash") == kernel_hash() and key in tr.get("entries", {}):
            traffic = tr["entries"][key]["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

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
                     "kernel": ("attn_fwd_pingpong_kernel<d=128,causal>" if plan["threads"] == 512
                                else "attn_fwd_kernel<d=128,causal,unsplit>") if plan["num_splits"] == 1
                     else "attn_fwd_kernel<d=128,causal,split> + combine_kernel",
                     "flops_per_launch": w.flops},
    }
    del q, k, v, out, lse
    torch.cuda.empty_cache()

    if not args.quick:
        extra = {}
        # sweep: both variants at every batch size
        big = gi.sweep(max(gi.SWEEP_BATCHES))
        qb, kb, vb = gpu_randn_inputs(big, dev, 7)
        sweep = {}
        for B in gi.SWEEP_BATCHES:
            wb = gi.sweep(B)
            for pack, ns in wb.variants:
                msb, pl = measure(g, wb, qb[:B], kb[:B], vb[:B], pack, ns, max(5, args.steps // 5), 3)
                sweep[f"B{B}_pack{pack}_ns{ns}"] = {
                    "ms": round(msb, 4), "tflops": round(wb.flops / (msb * 1e-3) / 1e12, 1),
                    "tokens_per_s": round(B * wb.Sq / (msb * 1e-3), 1)}
                print(f"[bench] sweep B={B} pack={pack} ns={ns}: {msb:.4f} ms", file=sys.stderr, flush=True)
            msb, pl = measure(g, wb, qb[:B], kb[:B], vb[:B], -1, 0, max(5, args.steps // 5), 3)
            sweep[f"B{B}_auto"] = {"ms": round(msb, 4), "tflops": round(wb.flops / (msb * 1e-3) / 1e12, 1),
                                   "pack": pl["pack_gqa"], "ns": pl["num_splits"]}
        extra["sweep"] = sweep
        # the headline shape with Q and K in fp8 e4m3 (scores on the fp8 matrix cores, V and P V bf16)
        q8 = qb[:128].to(torch.float8_e4m3fn).view(torch.uint8)
        k8 = kb[:128].to(torch.float8_e4m3fn).view(torch.uint8)
        o8 = torch.empty_like(qb[:128])
        l8 = torch.empty((128, wb.Hq, wb.Sq), dtype=torch.float32, device=dev)
        w128 = gi.sweep(128)
        ms8, _ = time_calls(lambda: g.gqa_attn_fwd_qk8(q8, k8, vb[:128], 1.0, 1.0, o8, l8, w128.causal, w128.scale),
                            max(5, args.steps // 5), 3)
        extra["sweep_b128_fp8_qk"] = {"ms": round(ms8, 4), "tflops": round(w128.flops / (ms8 * 1e-3) / 1e12, 1),
                                      "kernel": "attn_fwd_kernel (fp8 Q/K scores, bf16 P V)"}
        print(f"[bench] fp8 Q/K sweep B=128: {ms8:.4f} ms", file=sys.stderr, flush=True)
        del q8, k8, o8, l8
        del qb, kb, vb
        torch.cuda.empty_cache()
        # Llama-2 prefill shape
        wl = gi.LLAMA_PREFILL
        ql, kl, vl = gpu_randn_inputs(wl, dev, 8)
        llama = {}
        for pack, ns in ((1, 1), (0, 1), (-1, 0)):
            msl, pl = measure(g, wl, ql, kl, vl, pack, ns, args.steps, 5)
            llama[f"pack{pl['pack_gqa']}_ns{pl['num_splits']}" + ("_auto" if pack < 0 else "")] = {
                "ms": round(msl, 4), "tflops": round(wl.flops / (msl * 1e-3) / 1e12, 1)}
        extra["llama_prefill_b4"] = llama
        del ql, kl, vl
        # variable-length prefill: 16 packed sequences of 128 .. 2048 tokens, Llama-2 heads, causal
        lens = [128 * (i + 1) for i in range(16)]
        tot = sum(lens)
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        qv = torch.randn((tot, wl.Hq, wl.d), generator=gen, device=dev).to(torch.bfloat16)
        kv_ = torch.randn((tot, wl.Hk, wl.d), generator=gen, device=dev).to(torch.bfloat16)
        vv = torch.randn((tot, wl.Hk, wl.d), generator=gen, device=dev).to(torch.bfloat16)
        cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int32, device=dev)
        ov = torch.empty_like(qv)
        lv = torch.empty((wl.Hq, tot), dtype=torch.float32, device=dev)
        msv, _ = time_calls(lambda: g.gqa_attn_fwd_varlen(qv, kv_, vv, ov, lv, cu, cu, max(lens), max(lens), True,
                                                          wl.scale), args.steps, 5)
        fl = sum(4.0 * wl.Hq * L * L * wl.d / 2 for L in lens)
        extra["varlen_prefill_16seq_128to2048"] = {"ms": round(msv, 4), "tflops": round(fl / (msv * 1e-3) / 1e12, 1),
                                                   "tokens": tot}
        print(f"[bench] varlen prefill: {msv:.4f} ms", file=sys.stderr, flush=True)
        del qv, kv_, vv, ov, lv
        # backward at the Llama-2 prefill shape (B=4, causal): dQ, dK, dV from the forward's O and LSE
        ql, kl, vl = gpu_randn_inputs(wl, dev, 12)
        dol = torch.randn_like(ql, dtype=torch.float32).to(torch.bfloat16)
        ol = torch.empty_like(ql)
        ll = torch.empty((wl.B, wl.Hq, wl.Sq), dtype=torch.float32, device=dev)
        g.gqa_attn_fwd(ql, kl, vl, ol, ll, wl.causal, wl.scale)
        dql, dkl, dvl = torch.empty_like(ql), torch.empty_like(kl), torch.empty_like(vl)
        msbw, _ = time_calls(lambda: g.gqa_attn_bwd(ql, kl, vl, ol, ll, dol, dql, dkl, dvl, wl.causal, wl.scale),
                             args.steps, 5)
        extra["backward_llama_b4"] = {"ms": round(msbw, 4), "tflops": round(2.5 * wl.flops / (msbw * 1e-3) / 1e12, 1),
                                      "flops_convention": "2.5x forward (5 products of the causal band)"}
        print(f"[bench] backward llama b4: {msbw:.4f} ms", file=sys.stderr, flush=True)
        del ql, kl, vl, dol, ol, ll, dql, dkl, dvl
        # split-KV decode
        wd = gi.DECODE
        qd, kd, vd = gpu_randn_inputs(wd, dev, 9)
        dec = {}
        for pack, ns in ((-1, 0), (1, 1), (1, 4), (1, 8), (0, 4)):
            msd, pl = measure(g, wd, qd, kd, vd, pack, ns, args.steps, 5)
            dec[f"pack{pl['pack_gqa']}_ns{pl['num_splits']}" + ("_auto" if pack < 0 else "")] = {
                "us": round(msd * 1e3, 2), "GB_per_s": round(wd.io_bytes / (msd * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(wd.io_bytes / (msd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "kernel": "attn_decode_kernel" if pl["block_m"] == 32 else "attn_fwd_kernel"}
            print(f"[bench] decode pack={pack} ns={ns}: {msd*1e3:.1f} us", file=sys.stderr, flush=True)
        extra["decode_b64_sk8192"] = dec
        del kd, vd
        # the same decode over a paged cache: pages of 256 keys in random pool order
        ps = 256
        P = wd.Sk // ps
        gen = torch.Generator(device=dev)
        gen.manual_seed(10)
        kc = torch.randn((wd.B * P, ps, wd.Hk, wd.d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vc = torch.randn((wd.B * P, ps, wd.Hk, wd.d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        table = torch.randperm(wd.B * P, generator=gen, device=dev).to(torch.int32).view(wd.B, P).contiguous()
        lens = torch.full((wd.B,), wd.Sk, dtype=torch.int32, device=dev)
        outp = torch.empty_like(qd)
        lsep = torch.empty((wd.B, wd.Hq, wd.Sq), dtype=torch.float32, device=dev)
        msp, _ = time_calls(lambda: g.gqa_attn_fwd_paged(qd, kc, vc, table, lens, outp, lsep, wd.causal, wd.scale),
                            args.steps, 5)
        extra["decode_paged_b64_sk8192_ps256"] = {
            "us": round(msp * 1e3, 2), "GB_per_s": round(wd.io_bytes / (msp * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(wd.io_bytes / (msp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel": "attn_decode_kernel (paged)"}
        print(f"[bench] paged decode ps={ps}: {msp*1e3:.1f} us", file=sys.stderr, flush=True)
        del kc, vc, table, lens
        # the same decode with fp8 e4m3 K/V (half the K/V bytes)
        k8 = torch.randn((wd.B, wd.Sk, wd.Hk, wd.d), generator=gen, device=dev).to(torch.float8_e4m3fn).view(torch.uint8)
        v8 = torch.randn((wd.B, wd.Sk, wd.Hk, wd.d), generator=gen, device=dev).to(torch.float8_e4m3fn).view(torch.uint8)
        ms8, _ = time_calls(lambda: g.gqa_attn_fwd_kv8(qd, k8, v8, 1.0, 1.0, outp, lsep, wd.causal, wd.scale),
                            args.steps, 5)
        bytes8 = wd.io_bytes - (k8.numel() + v8.numel())  # K and V at one byte per element
        extra["decode_kv8_b64_sk8192"] = {
            "us": round(ms8 * 1e3, 2), "GB_per_s": round(bytes8 / (ms8 * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(bytes8 / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": bytes8, "kernel": "attn_decode_kernel (fp8 K/V)"}
        print(f"[bench] fp8 decode: {ms8*1e3:.1f} us", file=sys.stderr, flush=True)
        del qd, k8, v8, outp, lsep
        torch.cuda.empty_cache()
        result["extra"] = extra

    if not args.quick and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
