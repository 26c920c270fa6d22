"""Build the fp8blk HIP library (gfx950 only) into _build/libfp8blk.so.

    python -m fp8_fine_grained_token_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Flags: -O3, C++17, no fast
math, explicit FMAs only (-ffp-contract=off), packed-FP32 instructions off.

It also builds _build/libfp8blk_poison.so, the same sources with
FP8BLK_POISON_LDS defined (every LDS-DMA copy first poisons its destination):
a race-check build that tests load through FP8BLK_LIB; the product path loads
libfp8blk.so.

And _build/libfp8probe.so from csrc/probe/clock.hip: the benchmark's
shader-clock probe, kept out of the library.
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
POISON_LIB_PATH = os.path.join(BUILD_DIR, "libfp8blk_poison.so")
PROBE_LIB_PATH = os.path.join(BUILD_DIR, "libfp8probe.so")
PROBE_SRC = os.path.join(CSRC, "probe", "clock.hip")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _command(out: str, defines, srcs=None) -> list:
    return [
        hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-gpu-rdc", "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I" + os.path.join(os.path.dirname(HERE), "include"),
    ] + ["-D" + d for d in defines] + ["-o", out] + (srcs or sources())


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libfp8blk.so, the race-check
    libfp8blk_poison.so and the clock probe libfp8probe.so (always rebuilds;
    they compile in parallel)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for path, defines, srcs in ((LIB_PATH, [], None),
                                (POISON_LIB_PATH, ["FP8BLK_POISON_LDS"], None),
                                (PROBE_LIB_PATH, [], [PROBE_SRC])):
        tmp = path + ".tmp%d" % os.getpid()
        cmd = _command(tmp, defines, srcs)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((subprocess.Popen(cmd), tmp, path, cmd))
    failed = None
    for proc, tmp, path, cmd in jobs:
        if proc.wait() != 0 and failed is None:
            failed = subprocess.CalledProcessError(proc.returncode, cmd)
    if failed is not None:
        raise failed
    for proc, tmp, path, cmd in jobs:
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
