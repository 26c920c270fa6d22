"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_sanitize_driver.c calls every exported routine of
oracle/oracle.c on small ragged shapes (partial 128-groups and blocks, an
empty expert, special bf16 values) with exact-size heap buffers.  Built with
gcc -fsanitize=address,undefined and no recovery, any out-of-bounds access,
use after free or undefined operation in the oracle ends the run with an
error report.  (The sanitizer build leaves out the oracle's OpenMP
pragmas, so it runs the same loops on one thread.)
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "sanitize", "oracle_sanitize_driver.c")
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
FLAGS = ["-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-Wall", "-Wextra", "-Wno-unknown-pragmas"]


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    build = subprocess.run(["gcc", *FLAGS, DRIVER, ORACLE_C, "-o", exe, "-lm"],
                           capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-2000:]
    # verify_asan_link_order=0: the process environment may preload other
    # libraries ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert "oracle sanitize driver ok" in run.stdout
