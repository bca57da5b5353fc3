"""Build libsvq.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsvq.so")
BUILD_DIR = os.path.join(HERE, "_build")

COMMON_FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per translation unit: the exact-path kernels keep MFMA results in ordinary
# VGPRs (no accvgpr copies in the decode loops); the prefill GEMM keeps its
# 256 accumulators in accumulation registers.
SOURCES = [
    ("csrc/svq_host.cpp", []),
    ("csrc/svq_plan.cpp", []),
    ("csrc/svq_kernels.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("csrc/svq_prefill.hip", []),
    ("csrc/svq_small.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("csrc/svq_moe.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("csrc/svq_encode.hip", []),
    ("csrc/svq_calib.hip", []),
    ("csrc/svq_scratch.hip", []),
]
# kept for callers that list the flags of the exact-path kernels
HIPCC_FLAGS = COMMON_FLAGS + ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        _run([hipcc, *COMMON_FLAGS, *extra, "-c", "-o", obj, os.path.join(HERE, src)], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
