"""Build the fp8blk HIP library (gfx950 only) into _build/libfp8blk.so.

    python -m fp8_fine_grained_token_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Flags: -O3, C++17, no fast
math, explicit FMAs only (-ffp-contract=off), packed-FP32 instructions off.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libfp8blk.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libfp8blk.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [
        hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-gpu-rdc", "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I" + os.path.join(os.path.dirname(HERE), "include"),
        "-o", tmp,
    ] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
