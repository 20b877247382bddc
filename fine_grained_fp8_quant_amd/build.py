"""Build libfgq.so (gfx950) in-tree with hipcc.

    python -m fine_grained_fp8_quant_amd.build

Every translation unit is compiled for gfx950 only.  The quantisation kernels
are compiled with -ffp-contract=off because their binary32 results must be
bit-identical to the written definition; packed FP32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfgq.so")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "dispatch.hip": ["-ffp-contract=off"],
    # MFMA results straight into VGPRs: the per-chunk promotion FMA reads them
    # on the vector ALU, which cannot read AGPRs without an extra move.
    # -ffp-contract=off as well: the fused A-load quantisation must match
    # quant.hip bit for bit.
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-ffp-contract=off"],
    "fgq_api.cpp": [],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfgq)")


def build(verbose: bool = False) -> str:
    """Compile every source and link libfgq.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        cmd = [cc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
