"""Build libmxfp4.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m mxfp4_precision_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxfp4.so")
SOURCES = ["api.cpp", "layout.cpp", "quantize.hip", "quantize_fp8.hip", "gemm.hip", "convert.hip",
           "dequantize.hip", "measure.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmxfp4)")


def common_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # packed fp32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # fp32 denormals are needed by the E2M1 encoder's subnormal range
        "-fno-gpu-flush-denormals-to-zero",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmxfp4.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
