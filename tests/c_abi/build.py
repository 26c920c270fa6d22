"""Builds tests/c_abi/c_abi_check (plain C99, gcc) against the HIP library's C
ABI (include/fp8blk.h, fp8_fine_grained_token_amd/_build/libfp8blk.so) and
the CPU oracle (oracle/_build/liboracle.so), both found at run time through
$ORIGIN-relative rpaths.  Test infrastructure: only the tests and build()
use it."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
SRC = os.path.join(HERE, "c_abi_check.c")
OUT_DIR = os.path.join(HERE, "_build")
EXE = os.path.join(OUT_DIR, "c_abi_check")


def build(force: bool = False) -> str:
    from fp8_fine_grained_token_amd import build as hip_build
    import oracle

    hip_lib = os.path.join(ROOT, "fp8_fine_grained_token_amd", "_build", "libfp8blk.so")
    if not os.path.exists(hip_lib):
        hip_build.build()
    oracle.build()
    if not force and os.path.exists(EXE) and os.path.getmtime(EXE) >= max(
            os.path.getmtime(SRC), os.path.getmtime(hip_lib)):
        return EXE
    os.makedirs(OUT_DIR, exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [
        "gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
        "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(rocm, "include"),
        "-o", EXE, SRC,
        "-L" + os.path.join(ROOT, "fp8_fine_grained_token_amd", "_build"), "-lfp8blk",
        "-L" + os.path.join(ROOT, "oracle", "_build"), "-l:liboracle.so",
        "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
        "-Wl,-rpath,$ORIGIN/../../../fp8_fine_grained_token_amd/_build",
        "-Wl,-rpath,$ORIGIN/../../../oracle/_build",
        "-Wl,-rpath," + os.path.join(rocm, "lib"),
    ]
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build(force=True))
