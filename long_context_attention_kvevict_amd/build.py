"""Builds libkvevict.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m long_context_attention_kvevict_amd.build

Every HIP source is compiled for --offload-arch=gfx950 with packed-fp32
instructions disabled; the host-only planner is compiled by the same
driver.  Objects go to _build/, the shared library to lib/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libkvevict.so")
PROBE_LIB = os.path.join(LIBDIR, "libkveprobe.so")   # memory-system probes of the benchmark

PROBE_SOURCES = ["probe.hip"]
SOURCES = ["api.cpp", "plan.cpp", "timing.cpp", "score_bf16.hip", "score_f32.hip", "pool.hip", "knorm.hip", "merge.hip", "select.hip",
           "compact.hip", "decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=fast", "-munsafe-fp-atomics"]


# The bf16 scorer never sees NaN (finite inputs; masking uses -inf): without
# IEEE mode its max/min reductions need no NaN-quieting instructions.
PER_FILE = {"score_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *PER_FILE.get(src, []), "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # surface real warnings, skip the host pass's unknown-feature notice
    noise = "is not a recognized feature for this target"
    warn = [ln for ln in r.stderr.splitlines() if ln.strip() and noise not in ln]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
