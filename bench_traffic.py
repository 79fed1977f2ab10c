#!/usr/bin/env python3
"""HBM traffic and kernel-trace summaries of the GQA forward kernels (rocprofv3).

    python bench_traffic.py [--out-dir gpurun_out/traffic]

runs, for each benchmark workload, three profiled child processes of this
script (``--run NAME``): one ``--kernel-trace --stats`` pass, one
``--pmc FETCH_SIZE`` pass and one ``--pmc WRITE_SIZE`` pass. It calibrates the
two counters on a plain 1 GiB device copy (``--copy-ref``), then writes

into <out-dir>/profiles/ (to be copied into profiles/):

  * traffic.json: per workload, measured HBM bytes per launch of the
    attention kernel (FETCH + WRITE, each scaled by the copy's bytes/counter
    ratio), keyed by a hash of the kernel source so bench.py drops the figure
    once the kernel changes;
  * attn_fwd_<workload>.md: the trace and counter summary with the
    commands that produced it;
  * attn_fwd_sweep_b128_s2048_bench.md: a ``--kernel-trace --stats`` pass
    over the headline measurement itself (``bench.py --quick`` with its
    default steps and warm-up), whose average kernel time is the one
    bench.py reports;
  * attn_bwd_llama2_prefill_b4_s2048.md: trace and counters of the
    backward kernels at the Llama-2 prefill shape (``--run-bwd``);
  * attn_fwd_kv8_decode_b64_sk8192.md: trace and counters of the fp8 K/V
    decode at the decode workload's shape (``--run-kv8``);
  * attn_fwd_qk8_sweep_b128_s2048.md: trace and counters of the forward
    with fp8 Q and K at the headline shape (``--run-qk8``).

It never touches the GPU itself; the profiled children do.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
# the forward kernels' sources: the traffic counters are valid while these are unchanged
KERNEL_SRCS = [os.path.join(ROOT, "grouped_query_exact_amd", "csrc", f)
               for f in ("gqa_attn_kernels.hip", "device_common.h", "kernels.h", "host_logic.h")]
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30
KERNEL_NAMES = ("attn_fwd_kernel", "attn_fwd_pingpong_kernel", "attn_decode_kernel", "combine_kernel")
BWD_KERNEL_NAMES = ("bwd_dq_kernel", "bwd_dkdv_kernel")
RUN_LAUNCHES = 4
BWD_LAUNCHES = 20  # short kernels: enough calls for the average to be the steady state
QK8_LAUNCHES = 15  # the first launches of a process run slow; these dominate the average
KV8_LAUNCHES = 20

# name -> (workload factory, pack_gqa, num_splits); -1 / 0 = the library's choice
WORKLOADS = {
    "sweep_b128_s2048": ("sweep128", -1, 0),
    "llama2_prefill_b4_s2048": ("llama", -1, 0),
    "decode_b64_sk8192": ("decode", -1, 0),
    "ragged_b212_s77": ("ragged", -1, 0),
}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workload(name):
    import gqa_inputs as gi
    kind = WORKLOADS[name][0]
    return {"sweep128": gi.sweep(128), "llama": gi.LLAMA_PREFILL, "decode": gi.DECODE,
            "ragged": gi.RAGGED}[kind]


# ------------------------------------------------------------- child programs
def run_workload(name):
    import torch
    import grouped_query_exact_amd as g
    import gqa_inputs as gi
    w = workload(name)
    _, pack, ns = WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v = gi.make_qkv_device(w, dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    for _ in range(RUN_LAUNCHES):
        g.gqa_attn_fwd(q, k, v, out, lse, w.causal, w.scale, pack, ns)
    torch.cuda.synchronize()
    plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, pack, ns)
    print(json.dumps({"workload": name, "launches": RUN_LAUNCHES, "plan": plan}), flush=True)


def run_backward():
    """Forward once, then BWD_LAUNCHES backward calls at the Llama-2 prefill shape (B=4, causal)."""
    import torch
    import grouped_query_exact_amd as g
    import gqa_inputs as gi
    w = gi.LLAMA_PREFILL
    dev = torch.device("cuda:0")
    q, k, v = gi.make_qkv_device(w, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 17)
    do = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    g.gqa_attn_fwd(q, k, v, out, lse, w.causal, w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for _ in range(BWD_LAUNCHES):
        g.gqa_attn_bwd(q, k, v, out, lse, do, dq, dk, dv, w.causal, w.scale)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "backward " + w.name, "launches": BWD_LAUNCHES}), flush=True)


def run_qk8():
    """QK8_LAUNCHES fp8 Q/K forward calls at the headline shape (inputs: the bf16 recipe rounded to e4m3)."""
    import torch
    import grouped_query_exact_amd as g
    import gqa_inputs as gi
    w = gi.sweep(128)
    dev = torch.device("cuda:0")
    q, k, v = gi.make_qkv_device(w, dev)
    q8 = q.to(torch.float8_e4m3fn).view(torch.uint8)
    del q
    k8 = k.to(torch.float8_e4m3fn).view(torch.uint8)
    del k
    out = torch.empty((w.B, w.Sq, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    for _ in range(QK8_LAUNCHES):
        g.gqa_attn_fwd_qk8(q8, k8, v, 1.0, 1.0, out, lse, w.causal, w.scale)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "fp8 Q/K " + w.name, "launches": QK8_LAUNCHES}), flush=True)


def qk8_profile(out, prof_out, fetch_scale, write_scale):
    """Kernel trace and HBM counters of the fp8 Q/K forward at the headline shape."""
    import gqa_inputs as gi
    w = gi.sweep(128)
    cmd_t = rocprof(["--kernel-trace", "--stats"], out, "qk8_trace", ["--run-qk8"])
    cmd_f = rocprof(["--pmc", "FETCH_SIZE"], out, "qk8_fetch", ["--run-qk8"])
    cmd_w = rocprof(["--pmc", "WRITE_SIZE"], out, "qk8_write", ["--run-qk8"])
    stats = [r for r in read_trace(out, "qk8_trace") if "attn_fwd_kernel" in r["Name"]]
    fetch = attention_only(read_counter(out, "qk8_fetch", "FETCH_SIZE"))
    write = attention_only(read_counter(out, "qk8_write", "WRITE_SIZE"))
    qe = w.B * w.Sq * w.Hq * w.d
    ke = w.B * w.Sk * w.Hk * w.d
    alg = qe + ke + 2 * ke + 2 * qe + 4 * w.B * w.Hq * w.Sq  # Q, K fp8; V, O bf16; LSE fp32
    md = [f"# {w.name} with fp8 Q and K: B={w.B}, Sq=Sk={w.Sq}, Hq={w.Hq}, Hk={w.Hk}, d={w.d}, causal={w.causal}", "",
          f"{QK8_LAUNCHES} gqa_attn_fwd_qk8 calls (unit factors; the bf16 input recipe rounded to e4m3). "
          f"Kernel source hash {kernel_hash()}.", "",
          "Commands (REPO = repository root on the GPU box, run from /tmp with TMPDIR=/tmp):", "",
          "    " + cmd_t.replace(ROOT, "$REPO"), "    " + cmd_f.replace(ROOT, "$REPO"),
          "    " + cmd_w.replace(ROOT, "$REPO"), "", "Kernel trace (rocprofv3 --stats):", ""] + stats_table(stats)
    for r in stats:
        md += ["", f"Rate at the average time: {w.flops / (float(r['AverageNs']) * 1e-9) / 1e12:.1f} TFLOP/s "
                   f"(the metric's flops, 4*B*Hq*Sq*Sk*d/2)."]
    md += ["", f"HBM counters per dispatch (FETCH x{fetch_scale:.3f}, WRITE x{write_scale:.3f} from a 1 GiB copy):", "",
           "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) |", "|---|---|---|---|"]
    for kname in sorted(set(fetch) | set(write)):
        f_kib = sum(fetch.get(kname, [0])) / max(1, len(fetch.get(kname, [1])))
        w_kib = sum(write.get(kname, [0])) / max(1, len(write.get(kname, [1])))
        md.append(f"| `{kname[:90]}` | {f_kib:.0f} | {w_kib:.0f} | "
                  f"{(f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale) / 1e9:.4f} GB |")
    md += ["", f"Algorithmic bytes (Q and K at one byte, V and O at two, LSE at four, each once): {alg / 1e9:.4f} GB.", ""]
    with open(os.path.join(prof_out, f"attn_fwd_qk8_{w.name}.md"), "w") as f:
        f.write("\n".join(md))
    print("[traffic] fp8 Q/K profile written", flush=True)


def run_kv8():
    """KV8_LAUNCHES fp8 K/V decode calls at the decode workload's shape (K/V: the bf16 recipe rounded to e4m3)."""
    import torch
    import grouped_query_exact_amd as g
    import gqa_inputs as gi
    w = gi.DECODE
    dev = torch.device("cuda:0")
    q, k, v = gi.make_qkv_device(w, dev)
    k8 = k.to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = v.to(torch.float8_e4m3fn).view(torch.uint8)
    del k, v
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    for _ in range(KV8_LAUNCHES):
        g.gqa_attn_fwd_kv8(q, k8, v8, 1.0, 1.0, out, lse, w.causal, w.scale)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "fp8 K/V " + w.name, "launches": KV8_LAUNCHES}), flush=True)


def kv8_profile(out, prof_out, fetch_scale, write_scale):
    """Kernel trace and HBM counters of the fp8 K/V decode at the decode workload's shape."""
    import gqa_inputs as gi
    w = gi.DECODE
    cmd_t = rocprof(["--kernel-trace", "--stats"], out, "kv8_trace", ["--run-kv8"])
    cmd_f = rocprof(["--pmc", "FETCH_SIZE"], out, "kv8_fetch", ["--run-kv8"])
    cmd_w = rocprof(["--pmc", "WRITE_SIZE"], out, "kv8_write", ["--run-kv8"])
    stats = [r for r in read_trace(out, "kv8_trace") if any(n in r["Name"] for n in KERNEL_NAMES)]
    fetch = attention_only(read_counter(out, "kv8_fetch", "FETCH_SIZE"))
    write = attention_only(read_counter(out, "kv8_write", "WRITE_SIZE"))
    qe = w.B * w.Sq * w.Hq * w.d
    ke = w.B * w.Sk * w.Hk * w.d
    alg = 2 * qe + 2 * ke + 2 * qe + 4 * w.B * w.Hq * w.Sq  # Q bf16; K, V fp8; O bf16; LSE fp32
    md = [f"# {w.name} with fp8 K/V: B={w.B}, Sq={w.Sq}, Sk={w.Sk}, Hq={w.Hq}, Hk={w.Hk}, d={w.d}, causal={w.causal}", "",
          f"{KV8_LAUNCHES} gqa_attn_fwd_kv8 calls (unit factors; the bf16 input recipe rounded to e4m3, "
          f"library's choice of packing and splits). Kernel source hash {kernel_hash()}.", "",
          "Commands (REPO = repository root on the GPU box, run from /tmp with TMPDIR=/tmp):", "",
          "    " + cmd_t.replace(ROOT, "$REPO"), "    " + cmd_f.replace(ROOT, "$REPO"),
          "    " + cmd_w.replace(ROOT, "$REPO"), "", "Kernel trace (rocprofv3 --stats):", ""] + stats_table(stats)
    for r in stats:
        if "attn_decode_kernel" in r["Name"]:
            md += ["", f"Rate at the average time: {alg / (float(r['AverageNs']) * 1e-9) / 1e9:.1f} GB/s of "
                       f"algorithmic bytes ({alg / (float(r['AverageNs']) * 1e-9) / 1e9 / 8000:.3f} of 8 TB/s)."]
    md += ["", f"HBM counters per dispatch (FETCH x{fetch_scale:.3f}, WRITE x{write_scale:.3f} from a 1 GiB copy):", "",
           "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) |", "|---|---|---|---|"]
    for kname in sorted(set(fetch) | set(write)):
        f_kib = sum(fetch.get(kname, [0])) / max(1, len(fetch.get(kname, [1])))
        w_kib = sum(write.get(kname, [0])) / max(1, len(write.get(kname, [1])))
        md.append(f"| `{kname[:90]}` | {f_kib:.0f} | {w_kib:.0f} | "
                  f"{(f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale) / 1e9:.4f} GB |")
    md += ["", f"Algorithmic bytes (Q and O at two bytes, K and V at one, LSE at four, each once): {alg / 1e9:.4f} GB.", ""]
    with open(os.path.join(prof_out, f"attn_fwd_kv8_{w.name}.md"), "w") as f:
        f.write("\n".join(md))
    print("[traffic] fp8 K/V decode profile written", flush=True)


def run_copy():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied", COPY_BYTES, "bytes x3", flush=True)


# --------------------------------------------------------------- orchestrator
def rocprof(args, out_dir, tag, child, script=None, keep_stdout=False):
    cmd = ["rocprofv3"] + args + ["--output-format", "csv", "-d", os.path.join(out_dir, tag), "-o", tag,
                                  "--", sys.executable, script or os.path.abspath(__file__)] + child
    env = dict(os.environ, TMPDIR="/tmp")
    t0 = time.time()
    r = subprocess.run(["timeout", "-s", "KILL", "300"] + cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    print(f"[traffic] {tag}: rc={r.returncode} {time.time() - t0:.1f}s", flush=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout[-3000:] + r.stderr[-3000:])
        raise SystemExit(f"rocprofv3 pass {tag} failed")
    return (" ".join(cmd), r.stdout) if keep_stdout else " ".join(cmd)


def read_counter(out_dir, tag, counter):
    """Per-dispatch sums of one counter, grouped by kernel name."""
    files = glob.glob(os.path.join(out_dir, tag, "**", "*counter_collection.csv"), recursive=True)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    per[row["Kernel_Name"]][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def read_trace(out_dir, tag):
    files = glob.glob(os.path.join(out_dir, tag, "**", "*kernel_stats.csv"), recursive=True)
    rows = []
    for path in files:
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def attention_only(d, names=KERNEL_NAMES):
    return {k: v for k, v in d.items() if any(n in k for n in names)}


def stats_table(stats):
    md = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in stats:
        md.append(f"| `{r['Name'][:90]}` | {r.get('Calls')} | {float(r.get('AverageNs', 0)) / 1e3:.2f} | "
                  f"{float(r.get('MinNs', 0)) / 1e3:.2f} | {float(r.get('MaxNs', 0)) / 1e3:.2f} |")
    return md


def bench_trace(out, prof_out):
    """Kernel trace of the headline measurement: bench.py --quick with its default steps and warm-up."""
    bench = os.path.join(ROOT, "bench.py")
    cmd, stdout = rocprof(["--kernel-trace", "--stats"], out, "bench_headline_trace", ["--quick"], script=bench,
                          keep_stdout=True)
    line = [l for l in stdout.splitlines() if l.startswith("{")][-1]
    res = json.loads(line)
    stats = [r for r in read_trace(out, "bench_headline_trace") if any(n in r["Name"] for n in KERNEL_NAMES)]
    md = ["# sweep_b128_s2048: the headline measurement under the kernel trace", "",
          "The command bench.py times (headline workload B=128, Sq=Sk=2048, Hq=32, Hk=8, d=128, causal; "
          f"{res['warmup']} warm-up and {res['steps']} timed launches), traced. Kernel source hash {kernel_hash()}.", "",
          "Command (REPO = repository root on the GPU box, run from /tmp with TMPDIR=/tmp):", "",
          "    " + cmd.replace(ROOT, "$REPO"), "", "Kernel trace (rocprofv3 --stats):", ""] + stats_table(stats) + [
          "", f"bench.py in the same run (HIP events over the {res['steps']} timed launches): "
              f"{res['ms_per_step'] * 1e3:.1f} us per launch, {res['value']:.1f} TFLOP/s.", ""]
    with open(os.path.join(prof_out, "attn_fwd_sweep_b128_s2048_bench.md"), "w") as f:
        f.write("\n".join(md))
    print(f"[traffic] bench trace: {res['ms_per_step']:.4f} ms per launch in bench.py", flush=True)


def backward_profile(out, prof_out, fetch_scale, write_scale):
    """Kernel trace and HBM counters of the backward kernels at the Llama-2 prefill shape."""
    import gqa_inputs as gi
    w = gi.LLAMA_PREFILL
    cmd_t = rocprof(["--kernel-trace", "--stats"], out, "bwd_trace", ["--run-bwd"])
    cmd_f = rocprof(["--pmc", "FETCH_SIZE"], out, "bwd_fetch", ["--run-bwd"])
    cmd_w = rocprof(["--pmc", "WRITE_SIZE"], out, "bwd_write", ["--run-bwd"])
    stats = [r for r in read_trace(out, "bwd_trace") if any(n in r["Name"] for n in BWD_KERNEL_NAMES)]
    fetch = attention_only(read_counter(out, "bwd_fetch", "FETCH_SIZE"), BWD_KERNEL_NAMES)
    write = attention_only(read_counter(out, "bwd_write", "WRITE_SIZE"), BWD_KERNEL_NAMES)
    flops = {"bwd_dq_kernel": 3 * w.flops / 2, "bwd_dkdv_kernel": 4 * w.flops / 2}  # 3 and 4 products of the band
    md = [f"# backward, {w.name}: B={w.B}, Sq=Sk={w.Sq}, Hq={w.Hq}, Hk={w.Hk}, d={w.d}, causal={w.causal}", "",
          f"One forward call, then {BWD_LAUNCHES} gqa_attn_bwd calls on seeded bf16 N(0,1) inputs. "
          f"Kernel source hash (forward files) {kernel_hash()}.", "",
          "Commands (REPO = repository root on the GPU box, run from /tmp with TMPDIR=/tmp):", "",
          "    " + cmd_t.replace(ROOT, "$REPO"), "    " + cmd_f.replace(ROOT, "$REPO"),
          "    " + cmd_w.replace(ROOT, "$REPO"), "", "Kernel trace (rocprofv3 --stats):", ""] + stats_table(stats)
    md += ["", "Matrix-product rate of each kernel (its products over the causal band, 2*d flops per (row, key) pair "
               "and product):", "", "| kernel | products | TFLOP/s at the average time |", "|---|---|---|"]
    for r in stats:
        for kn, fl in flops.items():
            if kn in r["Name"]:
                md.append(f"| `{kn}` | {int(round(fl / (w.flops / 2)))} | {fl / (float(r['AverageNs']) * 1e-9) / 1e12:.1f} |")
    md += ["", f"HBM counters per dispatch (FETCH x{fetch_scale:.3f}, WRITE x{write_scale:.3f} from a 1 GiB copy):", "",
           "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) |", "|---|---|---|---|"]
    for kname in sorted(set(fetch) | set(write)):
        f_kib = sum(fetch.get(kname, [0])) / max(1, len(fetch.get(kname, [1])))
        w_kib = sum(write.get(kname, [0])) / max(1, len(write.get(kname, [1])))
        md.append(f"| `{kname[:90]}` | {f_kib:.0f} | {w_kib:.0f} | "
                  f"{(f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale) / 1e9:.4f} GB |")
    qb = w.B * w.Sq * w.Hq * w.d * 2   # Q, O, dO, dQ
    kb = w.B * w.Sk * w.Hk * w.d * 2   # K, V, dK, dV
    rb = w.B * w.Hq * w.Sq * 4         # LSE, D, base-2 LSE
    alg = 4 * qb + 4 * kb + 5 * rb     # Q O dO read, dQ written; K V read, dK dV written; LSE read, D and L2 written + read
    md += ["", f"Algorithmic bytes of the whole backward (Q, O, dO, K, V and LSE read once, dQ, dK, dV written once, "
               f"D and the base-2 LSE written and read once): {alg / 1e9:.4f} GB.", ""]
    with open(os.path.join(prof_out, f"attn_bwd_{w.name}.md"), "w") as f:
        f.write("\n".join(md))
    print("[traffic] backward profile written", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--run", help=argparse.SUPPRESS)
    ap.add_argument("--copy-ref", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--run-bwd", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--run-qk8", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--run-kv8", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--skip-kv8", action="store_true")
    ap.add_argument("--skip-qk8", action="store_true")
    ap.add_argument("--skip-bench-trace", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "gpurun_out", "traffic"))
    ap.add_argument("--workloads", nargs="*", default=list(WORKLOADS))
    a = ap.parse_args()
    if a.run:
        return run_workload(a.run)
    if a.copy_ref:
        return run_copy()
    if a.run_bwd:
        return run_backward()
    if a.run_qk8:
        return run_qk8()
    if a.run_kv8:
        return run_kv8()

    out = os.path.abspath(a.out_dir)
    os.makedirs(out, exist_ok=True)
    cmd_cf = rocprof(["--pmc", "FETCH_SIZE"], out, "copy_fetch", ["--copy-ref"])
    cmd_cw = rocprof(["--pmc", "WRITE_SIZE"], out, "copy_write", ["--copy-ref"])
    copy_f = [x for k, v in read_counter(out, "copy_fetch", "FETCH_SIZE").items() if "copyBuffer" in k for x in v]
    copy_w = [x for k, v in read_counter(out, "copy_write", "WRITE_SIZE").items() if "copyBuffer" in k for x in v]
    fetch_scale = COPY_BYTES / (sum(copy_f) / len(copy_f) * 1024)
    write_scale = COPY_BYTES / (sum(copy_w) / len(copy_w) * 1024)
    print(f"[traffic] copy calibration: FETCH x{fetch_scale:.3f}, WRITE x{write_scale:.3f}", flush=True)

    prof_out = os.path.join(out, "profiles")  # copied into profiles/ once reviewed
    os.makedirs(prof_out, exist_ok=True)
    tr_path = os.path.join(PROFILES, "traffic.json")
    try:
        with open(tr_path) as f:
            traffic = json.load(f)
    except (OSError, ValueError):
        traffic = {}
    if traffic.get("kernel_hash") != kernel_hash():
        traffic = {"kernel_hash": kernel_hash(), "entries": {}}
    traffic["calibration"] = {"copy_bytes": COPY_BYTES, "fetch_scale": fetch_scale, "write_scale": write_scale}

    for name in a.workloads:
        w = workload(name)
        cmd_t = rocprof(["--kernel-trace", "--stats"], out, f"{name}_trace", ["--run", name])
        cmd_f = rocprof(["--pmc", "FETCH_SIZE"], out, f"{name}_fetch", ["--run", name])
        cmd_w = rocprof(["--pmc", "WRITE_SIZE"], out, f"{name}_write", ["--run", name])
        fetch = attention_only(read_counter(out, f"{name}_fetch", "FETCH_SIZE"))
        write = attention_only(read_counter(out, f"{name}_write", "WRITE_SIZE"))
        stats = [r for r in read_trace(out, f"{name}_trace") if any(n in r["Name"] for n in KERNEL_NAMES)]
        import grouped_query_exact_amd as g  # host-only calls
        _, pack, ns = WORKLOADS[name]
        plan = g.gqa_attn_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hk, w.d, w.causal, pack, ns, 256)
        lines = []
        total_bytes = 0.0
        kernels = {}
        for kname in sorted(set(fetch) | set(write)):
            f_kib = sum(fetch.get(kname, [0])) / max(1, len(fetch.get(kname, [1])))
            w_kib = sum(write.get(kname, [0])) / max(1, len(write.get(kname, [1])))
            bytes_ = f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale
            total_bytes += bytes_
            kernels[kname] = {"fetch_kib": f_kib, "write_kib": w_kib, "hbm_bytes": bytes_}
        key = f"{name}|pack{plan['pack_gqa']}|ns{plan['num_splits']}"
        main_kernel = max(kernels, key=lambda k: kernels[k]["hbm_bytes"]) if kernels else None
        traffic["entries"][key] = {
            "hbm_bytes_per_launch": kernels[main_kernel]["hbm_bytes"] if main_kernel else None,
            "hbm_bytes_per_call": total_bytes, "algorithmic_bytes": w.io_bytes, "kernels": kernels,
            "measured": time.strftime("%Y-%m-%d %H:%M:%S"),
        }
        md = [f"# {name}: attention kernels, pack_gqa={plan['pack_gqa']}, num_splits={plan['num_splits']}", "",
              f"Workload: B={w.B}, Sq={w.Sq}, Sk={w.Sk}, Hq={w.Hq}, Hk={w.Hk}, d={w.d}, causal={w.causal}, "
              f"seeded bf16 N(0,1) inputs; {RUN_LAUNCHES} launches per profiled run. Kernel source hash {kernel_hash()}.", "",
              "Commands (REPO = repository root on the GPU box, run from /tmp with TMPDIR=/tmp):", "",
              "    " + cmd_t.replace(ROOT, "$REPO"), "    " + cmd_f.replace(ROOT, "$REPO"),
              "    " + cmd_w.replace(ROOT, "$REPO"), "    " + cmd_cf.replace(ROOT, "$REPO"),
              "    " + cmd_cw.replace(ROOT, "$REPO"), "",
              "Kernel trace (rocprofv3 --stats):", "", "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
        for r in stats:
            md.append(f"| `{r['Name'][:90]}` | {r.get('Calls')} | {float(r.get('AverageNs', 0)) / 1e3:.2f} | "
                      f"{float(r.get('MinNs', 0)) / 1e3:.2f} | {float(r.get('MaxNs', 0)) / 1e3:.2f} |")
        md += ["", f"HBM counters per dispatch (FETCH x{fetch_scale:.3f}, WRITE x{write_scale:.3f} from a 1 GiB copy):", "",
               "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) |", "|---|---|---|---|"]
        for kname, kv in kernels.items():
            md.append(f"| `{kname[:90]}` | {kv['fetch_kib']:.0f} | {kv['write_kib']:.0f} | {kv['hbm_bytes'] / 1e9:.4f} GB |")
        md += ["", f"Algorithmic bytes (Q + K + V + O + LSE once): {w.io_bytes / 1e9:.4f} GB; "
                   f"measured / algorithmic = {total_bytes / w.io_bytes:.3f}.", ""]
        fname = f"attn_fwd_{name}.md"
        with open(os.path.join(prof_out, fname), "w") as f:
            f.write("\n".join(md))
        print(f"[traffic] {name}: {total_bytes / 1e9:.4f} GB per call (algorithmic {w.io_bytes / 1e9:.4f})", flush=True)

    with open(os.path.join(prof_out, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
    if not a.skip_backward:
        backward_profile(out, prof_out, fetch_scale, write_scale)
    if not a.skip_qk8:
        qk8_profile(out, prof_out, fetch_scale, write_scale)
    if not a.skip_kv8:
        kv8_profile(out, prof_out, fetch_scale, write_scale)
    if not a.skip_bench_trace:
        bench_trace(out, prof_out)
    print(f"[traffic] wrote {prof_out}", flush=True)


if __name__ == "__main__":
    main()
