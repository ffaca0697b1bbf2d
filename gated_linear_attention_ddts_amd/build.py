"""Build librodimus.so (gfx950) from csrc/*.hip with hipcc, in-tree.

    python -m gated_linear_attention_ddts_amd.build

Each translation unit is compiled in parallel into ``_build/`` at the repo root,
then linked into ``gated_linear_attention_ddts_amd/librodimus.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "librodimus.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


# Extra flags per translation unit.  The prefill kernels never see NaN (inputs
# are finite; tau = -inf only produces infinities), so they run with the IEEE
# mode off, which drops the NaN-canonicalising moves in front of every min/max.
FILE_FLAGS = {
    "scan_mfma.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
    # The prefill's state pass and the backward's kernels are scheduled for
    # instruction-level parallelism (measured: state pass 51.9 -> 50.7 us,
    # backward gradient kernel 360.2 -> 354.7 us per call, bit-identical
    # results); the output pass and SW-SKA keep the default scheduler, under
    # which they are faster.
    "scan_state.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "scan_bwd_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of librodimus.so failed")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
