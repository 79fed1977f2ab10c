"""Build libgqa_attn.so (HIP kernels for gfx950 + the C-ABI) in-tree with hipcc.

Usage: python -m grouped_query_exact_amd.build [--jobs N]
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqa_attn.so")
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
# Packed-fp32 VALU instructions are disabled for all device code. MFMA results
# stay in ordinary VGPRs (no accumulator-register copies around the online
# softmax rescale of the output accumulators).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result"]

SOURCES = [
    ("gqa_attn_kernels.hip", True),
    ("gqa_attn_bwd.hip", True),
    ("gqa_attn_sched.hip", True),
    ("gqa_attn_scratch.hip", True),
    ("gqa_attn_api.cpp", False),
    ("host_logic.cpp", False),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the GQA library)")


def _compile(src: str, is_hip: bool) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + (["-x", "hip"] + DEVICE_FLAGS if is_hip else []) + \
          ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda a: _compile(*a), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    sys.exit(0)
