#!/usr/bin/env python3
"""Kernel traces, HBM traffic and pipe counters of the GQA kernels (rocprofv3).

    python bench_traffic.py [--out-dir DIR] [--workloads NAME ...]   (DIR defaults to traffic_out/)

For each workload below, a child process of this script (``--child NAME``)
makes WARMUP calls and then MEASURED calls of one entry point on seeded
N(0,1) GPU inputs of the workload's shape; this script runs that child under
rocprofv3 once per pass:

  trace : --kernel-trace --stats; the per-dispatch durations of the MEASURED
          calls (the warm-up dispatches are dropped) give the median, mean,
          minimum and maximum per kernel;
  fetch : --pmc FETCH_SIZE          (HBM bytes read, KiB per dispatch)
  write : --pmc WRITE_SIZE          (HBM bytes written)
  mfma  : --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE
  lds   : --pmc LdsBankConflict SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS GRBM_GUI_ACTIVE
  valu  : --pmc SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU SQ_WAVES

FETCH_SIZE and WRITE_SIZE are calibrated on a plain 1 GiB device copy
(``--child copy``): the bytes the copy moves divided by what each counter
reads for it. Counter values are the medians over the MEASURED dispatches.
MfmaUtil is rocprofv3's own derived metric, 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES)
/ (max(GRBM_GUI_ACTIVE) * SIMDs); LdsBankConflict is its conflicts per LDS
access, sum(SQ_LDS_BANK_CONFLICT) / (sum(SQ_LDS_IDX_ACTIVE) -
sum(SQ_LDS_BANK_CONFLICT)).

Output in <out-dir>/profiles/ (to be copied into profiles/): one
``<kernel family>_<workload>.md`` per workload with the commands, the trace
table, the HBM bytes against the algorithmic bytes and the counters, and
traffic.json (HBM bytes per launch keyed by a hash of the forward kernels'
sources, which bench.py reports as roofline.traffic while the sources are
unchanged). ``--bench-trace`` also traces the headline command itself
(bench.py --quick with its default steps and warm-up).

This script never touches the GPU itself; the profiled children do.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
KERNEL_SRCS = [os.path.join(ROOT, "grouped_query_exact_amd", "csrc", f)
               for f in ("gqa_attn_kernels.hip", "device_common.h", "kernels.h", "host_logic.h")]
BWD_SRCS = [os.path.join(ROOT, "grouped_query_exact_amd", "csrc", "gqa_attn_bwd.hip")]
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30
WARMUP = 5            # warm-up calls at least, and
WARMUP_SECONDS = 0.5  # at least this long (at most WARMUP_MAX calls)
WARMUP_MAX = 400
MEASURED = 20         # calls whose dispatches the statistics use (the last ones of each kernel)
KERNELS = ("attn_fwd_kernel", "attn_fwd_pingpong_kernel", "attn_decode_kernel", "combine_kernel",
           "combine_wide_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "varlen_schedule_kernel")
VARLEN_LENS = [128 * (i + 1) for i in range(16)]  # packed sequences of the variable-length workload
PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "mfma": ["MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"],
    "lds": ["LdsBankConflict", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"],
    "valu": ["SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_SALU", "SQ_WAVES"],
}

# name -> (file prefix, description). The children below build the inputs.
WORKLOADS = {
    "sweep_b128_s2048": ("attn_fwd", "causal B=128, Sq=Sk=2048, Hq=32, Hk=8, d=128, library's choice (headline)"),
    "llama2_prefill_b4_s2048": ("attn_fwd", "causal B=4, Sq=Sk=2048, Hq=32, Hk=8, d=128, library's choice"),
    "decode_b64_sk8192": ("attn_fwd", "B=64, Sq=1, Sk=8192, Hq=32, Hk=8, d=128, library's choice"),
    "decode_b64_sk8192_ns4": ("attn_fwd", "the decode workload at pack_gqa=1, num_splits=4"),
    "decode_b64_sk8192_ns8": ("attn_fwd", "the decode workload at pack_gqa=1, num_splits=8"),
    "ragged_b212_s77": ("attn_fwd", "non-causal B=212, Sq=Sk=77, Hq=6, Hk=2, d=64, library's choice"),
    "llama2_prefill_b4_s2048_bwd": ("attn_bwd", "backward at the Llama-2 prefill shape, causal"),
    "qk8_sweep_b128_s2048": ("attn_fwd", "the headline shape with fp8 e4m3 Q and K (gqa_attn_fwd_qk8)"),
    "kv8_decode_b64_sk8192": ("attn_fwd", "the decode workload with fp8 e4m3 K and V (gqa_attn_fwd_kv8)"),
    "varlen_16seq_128to2048": ("attn_fwd", "16 packed sequences of 128, 256, ..., 2048 tokens, causal, Hq=32, Hk=8, "
                                           "d=128 (gqa_attn_fwd_varlen)"),
}


def src_hash(paths=KERNEL_SRCS) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------- child programs
def _inputs(w, dev, seed):
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    r = lambda shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return r((w.B, w.Sq, w.Hq, w.d)), r((w.B, w.Sk, w.Hk, w.d)), r((w.B, w.Sk, w.Hk, w.d))


def child(name):
    """WARMUP + MEASURED calls of the workload's entry point; returns its description dict."""
    import torch
    import grouped_query_exact_amd as g
    import gqa_inputs as gi
    dev = torch.device("cuda:0")
    base = {"sweep_b128_s2048": gi.sweep(128), "llama2_prefill_b4_s2048": gi.LLAMA_PREFILL,
            "decode_b64_sk8192": gi.DECODE, "decode_b64_sk8192_ns4": gi.DECODE, "decode_b64_sk8192_ns8": gi.DECODE,
            "ragged_b212_s77": gi.RAGGED, "llama2_prefill_b4_s2048_bwd": gi.LLAMA_PREFILL,
            "qk8_sweep_b128_s2048": gi.sweep(128), "kv8_decode_b64_sk8192": gi.DECODE,
            "varlen_16seq_128to2048": gi.LLAMA_PREFILL}[name]
    w = base
    if name.startswith("varlen_"):  # one batch element of len(VARLEN_LENS) * ... tokens, packed
        w = w.with_(B=1, Sq=sum(VARLEN_LENS), Sk=sum(VARLEN_LENS))
    q, k, v = _inputs(w, dev, 1234)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    pack, ns = {"decode_b64_sk8192_ns4": (1, 4), "decode_b64_sk8192_ns8": (1, 8)}.get(name, (-1, 0))
    plan = None
    if name.startswith("varlen_"):
        cu = torch.tensor([0] + torch.tensor(VARLEN_LENS).cumsum(0).tolist(), dtype=torch.int32, device=dev)
        qv, kv_, vv, ov = q[0], k[0], v[0], out[0]
        call = lambda: g.gqa_attn_fwd_varlen(qv, kv_, vv, ov, lse[0], cu, cu, max(VARLEN_LENS), max(VARLEN_LENS),
                                             w.causal, w.scale)
    elif name.endswith("_bwd"):
        do = torch.randn_like(q, dtype=torch.float32).to(torch.bfloat16)
        g.gqa_attn_fwd(q, k, v, out, lse, w.causal, w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        call = lambda: g.gqa_attn_bwd(q, k, v, out, lse, do, dq, dk, dv, w.causal, w.scale)
    elif name.startswith("qk8_"):
        q8 = q.to(torch.float8_e4m3fn).view(torch.uint8)
        k8 = k.to(torch.float8_e4m3fn).view(torch.uint8)
        del q
        call = lambda: g.gqa_attn_fwd_qk8(q8, k8, v, 1.0, 1.0, out, lse, w.causal, w.scale)
    elif name.startswith("kv8_"):
        k8 = k.to(torch.float8_e4m3fn).view(torch.uint8)
        v8 = v.to(torch.float8_e4m3fn).view(torch.uint8)
        del k, v
        call = lambda: g.gqa_attn_fwd_kv8(q, k8, v8, 1.0, 1.0, out, lse, w.causal, w.scale)
    else:
        call = lambda: g.gqa_attn_fwd(q, k, v, out, lse, w.causal, w.scale, pack, ns)
    # warm up by time as well as by count: short calls in a fresh process run
    # well below their steady-state clock for the first few hundred milliseconds
    t0 = time.perf_counter()
    n = 0
    while n < WARMUP or (time.perf_counter() - t0 < WARMUP_SECONDS and n < WARMUP_MAX):
        call()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    for _ in range(MEASURED):
        call()
    torch.cuda.synchronize()
    if not name.startswith("varlen_"):
        plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, pack, ns)
    print(json.dumps({"workload": name, "warmup": n, "measured": MEASURED, "plan": plan}), flush=True)


def child_copy():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied", COPY_BYTES, "bytes x3", flush=True)


# ---------------------------------------------------------------- bookkeeping
def workload_bytes_flops(name):
    """(algorithmic HBM bytes per call, flops per call of the metric) of a workload."""
    import gqa_inputs as gi
    if name.startswith("qk8_"):
        w = gi.sweep(128)
        qe, ke = w.B * w.Sq * w.Hq * w.d, w.B * w.Sk * w.Hk * w.d
        return qe + ke + 2 * ke + 2 * qe + 4 * w.B * w.Hq * w.Sq, w.flops  # Q, K fp8; V, O bf16; LSE fp32
    if name.startswith("kv8_"):
        w = gi.DECODE
        qe, ke = w.B * w.Sq * w.Hq * w.d, w.B * w.Sk * w.Hk * w.d
        return 2 * qe + 2 * ke + 2 * qe + 4 * w.B * w.Hq * w.Sq, w.flops  # Q bf16; K, V fp8; O bf16; LSE
    if name.endswith("_bwd"):
        w = gi.LLAMA_PREFILL
        qb, kb, rb = w.B * w.Sq * w.Hq * w.d * 2, w.B * w.Sk * w.Hk * w.d * 2, w.B * w.Hq * w.Sq * 4
        # Q O dO read, dQ written; K V read, dK dV written; LSE read, D and base-2 LSE written and read
        return 4 * qb + 4 * kb + 5 * rb, 2.5 * w.flops
    if name.startswith("varlen_"):
        w, tot = gi.LLAMA_PREFILL, sum(VARLEN_LENS)
        flops = sum(4.0 * w.Hq * n * n * w.d / 2 for n in VARLEN_LENS)
        # Q, O bf16; K, V bf16; LSE fp32; the offsets and the work list are a few KB
        return 4 * tot * w.Hq * w.d + 4 * tot * w.Hk * w.d + 4 * tot * w.Hq, flops
    w = {"sweep_b128_s2048": gi.sweep(128), "llama2_prefill_b4_s2048": gi.LLAMA_PREFILL,
         "ragged_b212_s77": gi.RAGGED}.get(name, gi.DECODE)
    return w.io_bytes, w.flops


def rocprof(args, out_dir, tag, child_args, script=None, keep_stdout=False):
    cmd = ["rocprofv3"] + args + ["--output-format", "csv", "-d", os.path.join(out_dir, tag), "-o", tag,
                                  "--", sys.executable, script or os.path.abspath(__file__)] + child_args
    env = dict(os.environ, TMPDIR="/tmp")
    t0 = time.time()
    # a counter pass over a short program takes seconds; a refused counter set must not hang
    limit = "120" if "--pmc" in args else "300"
    r = subprocess.run(["timeout", "-s", "KILL", limit] + cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    print(f"[profile] {tag}: rc={r.returncode} {time.time() - t0:.1f}s", flush=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout[-3000:] + r.stderr[-3000:])
        raise SystemExit(f"rocprofv3 pass {tag} failed")
    return (" ".join(cmd), r.stdout) if keep_stdout else " ".join(cmd)


def short_name(kname):
    for n in sorted(KERNELS, key=len, reverse=True):
        if n in kname:
            return n
    return kname[:60]


def read_trace(out_dir, tag):
    """Per kernel: durations (ns) of its dispatches in order."""
    per = collections.defaultdict(list)
    for path in glob.glob(os.path.join(out_dir, tag, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows = list(csv.DictReader(f))
        if rows and not {"Kernel_Name", "Start_Timestamp", "End_Timestamp"} <= set(rows[0]):
            raise SystemExit(f"unexpected kernel trace columns in {path}: {sorted(rows[0])}")
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            if any(n in r["Kernel_Name"] for n in KERNELS):
                per[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return per


def read_counters(out_dir, tag):
    """Per kernel and counter: the per-dispatch values in dispatch order."""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for path in glob.glob(os.path.join(out_dir, tag, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if not any(n in row["Kernel_Name"] for n in KERNELS):
                    continue
                d = per[row["Kernel_Name"]][row["Counter_Name"]]
                did = int(row["Dispatch_Id"])
                d[did] = d.get(did, 0.0) + float(row["Counter_Value"])
    return {k: {c: [v[i] for i in sorted(v)] for c, v in cs.items()} for k, cs in per.items()}


def measured_median(values):
    """Median over the MEASURED calls: a kernel's last MEASURED dispatches (each kernel runs once per call)."""
    tail = values[-MEASURED:]
    return statistics.median(tail) if tail else float("nan")


# --------------------------------------------------------------------- driver
def profile_workload(name, out, prof_out, fscale, wscale, copy_cmds):
    prefix, desc = WORKLOADS[name]
    cmds = {"trace": rocprof(["--kernel-trace", "--stats"], out, f"{name}_trace", ["--child", name])}
    for p, counters in PASSES.items():
        cmds[p] = rocprof(["--pmc"] + counters, out, f"{name}_{p}", ["--child", name])
    trace = read_trace(out, f"{name}_trace")
    ctr = {}
    for p in PASSES:
        for k, cs in read_counters(out, f"{name}_{p}").items():
            ctr.setdefault(k, {}).update(cs)
    alg, flops = workload_bytes_flops(name)
    kernels = {}
    for kname, durs in trace.items():
        tail = durs[-MEASURED:]
        kc = ctr.get(kname, {})
        med = lambda c: measured_median(kc.get(c, []))
        e = {"calls": len(durs), "median_us": statistics.median(tail) / 1e3, "mean_us": sum(tail) / len(tail) / 1e3,
             "min_us": min(tail) / 1e3, "max_us": max(tail) / 1e3,
             "fetch_bytes": med("FETCH_SIZE") * 1024 * fscale, "write_bytes": med("WRITE_SIZE") * 1024 * wscale}
        for c in set(sum(PASSES.values(), [])) - {"FETCH_SIZE", "WRITE_SIZE"}:
            e[c] = med(c)
        kernels[short_name(kname)] = e
    # kernels dispatched fewer times than there are measured calls ran once for
    # the set-up (the backward's forward pass), not in every call
    per_call = {k: e for k, e in kernels.items() if e["calls"] >= MEASURED}
    main = max(per_call, key=lambda k: per_call[k]["median_us"])
    call_us = sum(k["median_us"] for k in per_call.values())
    hbm = sum(k["fetch_bytes"] + k["write_bytes"] for k in per_call.values())
    md = [f"# {name}: {desc}", "",
          f"At least {WARMUP} warm-up calls and {WARMUP_SECONDS} s of them, then {MEASURED} measured calls per "
          f"profiled run, seeded N(0,1) inputs on the GPU. "
          f"Forward kernel source hash {src_hash()}, backward source hash {src_hash(BWD_SRCS)}.", "",
          "Commands (REPO = repository root, run from /tmp with TMPDIR=/tmp):", ""]
    md += ["    " + c.replace(ROOT, "$REPO") for c in list(cmds.values()) + copy_cmds]
    md += ["", f"Kernel trace (rocprofv3 --kernel-trace; statistics over the {MEASURED} measured calls):", "",
           "| kernel | dispatches | median (us) | mean (us) | min (us) | max (us) |", "|---|---|---|---|---|---|"]
    for kn, e in kernels.items():
        md.append(f"| `{kn}`{'' if kn in per_call else ' (set-up, once)'} | {e['calls']} | {e['median_us']:.2f} | "
                  f"{e['mean_us']:.2f} | {e['min_us']:.2f} | {e['max_us']:.2f} |")
    rate_flops = flops / (call_us * 1e-6) / 1e12
    md += ["", f"One call at the medians (the kernels every call runs): {call_us:.2f} us = {rate_flops:.1f} TFLOP/s of the metric's flops "
               f"({flops / 1e9:.1f} GFLOP) and {alg / (call_us * 1e-6) / 1e9:.1f} GB/s of algorithmic bytes "
               f"({alg / 1e9:.4f} GB).", "",
           f"HBM traffic per call (median of the measured dispatches; FETCH_SIZE x{fscale:.3f}, WRITE_SIZE "
           f"x{wscale:.3f} from the 1 GiB copy):", "",
           "| kernel | read (GB) | written (GB) |", "|---|---|---|"]
    for kn, e in kernels.items():
        md.append(f"| `{kn}` | {e['fetch_bytes'] / 1e9:.4f} | {e['write_bytes'] / 1e9:.4f} |")
    md += ["", f"Measured / algorithmic bytes: {hbm / 1e9:.4f} / {alg / 1e9:.4f} GB = {hbm / alg:.3f}.", "",
           "Pipe counters (median over the measured dispatches; MfmaUtil and LdsBankConflict are rocprofv3's "
           "derived metrics, percent of SIMD-cycles with the matrix pipe busy and conflict cycles per LDS access):",
           "", "| kernel | MfmaUtil % | MFMA busy cycles | MFMA instrs | LdsBankConflict | LDS bank-conflict cycles | "
               "LDS active cycles | LDS instrs | VALU instrs | MFMA+VALU co-issue cycles | SALU instrs | waves |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for kn, e in kernels.items():
        f = lambda c, fmt="{:.0f}": fmt.format(e.get(c, float("nan")))
        md.append(f"| `{kn}` | {f('MfmaUtil', '{:.1f}')} | {f('SQ_VALU_MFMA_BUSY_CYCLES')} | {f('SQ_INSTS_MFMA')} | "
                  f"{f('LdsBankConflict', '{:.4f}')} | {f('SQ_LDS_BANK_CONFLICT')} | {f('SQ_LDS_IDX_ACTIVE')} | "
                  f"{f('SQ_INSTS_LDS')} | {f('SQ_INSTS_VALU')} | {f('SQ_VALU_MFMA_COEXEC_CYCLES')} | "
                  f"{f('SQ_INSTS_SALU')} | {f('SQ_WAVES')} |")
    md.append("")
    with open(os.path.join(prof_out, f"{prefix}_{name}.md"), "w") as f:
        f.write("\n".join(md))
    print(f"[profile] {name}: {call_us:.1f} us per call, main kernel {main} "
          f"MfmaUtil {kernels[main].get('MfmaUtil', float('nan')):.1f}%, HBM {hbm / alg:.3f} x algorithmic", flush=True)
    return {"kernels": per_call, "main_kernel": main, "hbm_bytes_per_call": hbm, "algorithmic_bytes": alg,
            "hbm_bytes_per_launch": kernels[main]["fetch_bytes"] + kernels[main]["write_bytes"],
            "call_us_median": call_us, "measured": time.strftime("%Y-%m-%d %H:%M:%S")}


def bench_trace(out, prof_out):
    """Kernel trace of the headline measurement: bench.py --quick with its default steps and warm-up."""
    bench = os.path.join(ROOT, "bench.py")
    cmd, stdout = rocprof(["--kernel-trace", "--stats"], out, "bench_headline_trace", ["--quick"], script=bench,
                          keep_stdout=True)
    res = json.loads([l for l in stdout.splitlines() if l.startswith("{")][-1])
    trace = read_trace(out, "bench_headline_trace")
    md = ["# sweep_b128_s2048: the headline measurement under the kernel trace", "",
          f"The command bench.py times (causal B=128, Sq=Sk=2048, Hq=32, Hk=8, d=128; {res['warmup']} warm-up and "
          f"{res['steps']} timed launches), traced. Forward kernel source hash {src_hash()}.", "",
          "Command (REPO = repository root, run from /tmp with TMPDIR=/tmp):", "",
          "    " + cmd.replace(ROOT, "$REPO"), "",
          "| kernel | dispatches | median of the timed launches (us) | mean of the timed launches (us) | "
          "mean of all (us) |", "|---|---|---|---|---|"]
    for kn, durs in trace.items():
        tail = durs[-res["steps"]:]
        md.append(f"| `{short_name(kn)}` | {len(durs)} | {statistics.median(tail) / 1e3:.1f} | "
                  f"{sum(tail) / len(tail) / 1e3:.1f} | {sum(durs) / len(durs) / 1e3:.1f} |")
    md += ["", f"bench.py in the same run (HIP events around the {res['steps']} timed launches): "
               f"{res['ms_per_step'] * 1e3:.1f} us per launch, {res['value']:.1f} TFLOP/s.", ""]
    with open(os.path.join(prof_out, "attn_fwd_sweep_b128_s2048_bench.md"), "w") as f:
        f.write("\n".join(md))
    print(f"[profile] bench trace: {res['ms_per_step']:.4f} ms per launch in bench.py", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--child", help=argparse.SUPPRESS)
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "traffic_out"))
    ap.add_argument("--workloads", nargs="*", default=list(WORKLOADS))
    ap.add_argument("--bench-trace", action="store_true")
    a = ap.parse_args()
    if a.child == "copy":
        return child_copy()
    if a.child:
        return child(a.child)

    out = os.path.abspath(a.out_dir)
    prof_out = os.path.join(out, "profiles")
    os.makedirs(prof_out, exist_ok=True)
    copy_cmds = [rocprof(["--pmc", "FETCH_SIZE"], out, "copy_fetch", ["--child", "copy"]),
                 rocprof(["--pmc", "WRITE_SIZE"], out, "copy_write", ["--child", "copy"])]
    cf = [x for k, v in read_counters_raw(out, "copy_fetch", "FETCH_SIZE").items() if "copyBuffer" in k for x in v]
    cw = [x for k, v in read_counters_raw(out, "copy_write", "WRITE_SIZE").items() if "copyBuffer" in k for x in v]
    fscale = COPY_BYTES / (statistics.median(cf) * 1024)
    wscale = COPY_BYTES / (statistics.median(cw) * 1024)
    print(f"[profile] copy calibration: FETCH x{fscale:.3f}, WRITE x{wscale:.3f}", flush=True)

    tr_path = os.path.join(PROFILES, "traffic.json")
    try:
        with open(tr_path) as f:
            traffic = json.load(f)
    except (OSError, ValueError):
        traffic = {}
    if traffic.get("kernel_hash") != src_hash():
        traffic = {"kernel_hash": src_hash(), "entries": {}}
    traffic["calibration"] = {"copy_bytes": COPY_BYTES, "fetch_scale": fscale, "write_scale": wscale}
    for name in a.workloads:
        res = profile_workload(name, out, prof_out, fscale, wscale, [c.replace(ROOT, "$REPO") for c in copy_cmds])
        traffic["entries"][name] = res
        with open(os.path.join(prof_out, "traffic.json"), "w") as f:
            json.dump(traffic, f, indent=1, sort_keys=True)
    if a.bench_trace:
        bench_trace(out, prof_out)
    print(f"[profile] wrote {prof_out}", flush=True)


def read_counters_raw(out_dir, tag, counter):
    """Per kernel: one counter's per-dispatch values (any kernel, e.g. the copy)."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for path in glob.glob(os.path.join(out_dir, tag, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    per[row["Kernel_Name"]][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


if __name__ == "__main__":
    main()
