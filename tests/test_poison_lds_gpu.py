"""Race check of the LDS pipelines: the poison build against the released one.

In _build/libfp8blk_poison.so every LDS-DMA copy first fills its destination
with 0x7F (an E4M3 NaN, a huge fp32 scale) and waits for that before it
issues the copy.  If any wave of a workgroup still read a stage (or a scale
buffer) that another wave had begun to refill, it would see poison at once
and its outputs would change.  The arithmetic is otherwise the same, so every
GEMM case of tests/poison_cases.py (each tile kind and pipeline: dense two
widths, one 256 x 256 round, small tiles with and without split-K, the
no-allocation GEMM, grouped with partial scale chunks, power-of-two scales,
the fused quantization with and without split-K, Dgrad reading W
transposed (also with power-of-two scales), Wgrad in both plans (also with
power-of-two scales))
must give bitwise the same bytes with either library.  The poison build runs
in a child process (the library is chosen when the process first loads it).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from .gpu_util import log, torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
POISON_LIB = os.path.join(ROOT, "fp8_fine_grained_token_amd", "_build", "libfp8blk_poison.so")


def test_poison_build_matches_released_build(tmp_path):
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(POISON_LIB), "race-check build missing: run __graft_entry__.build()"
    from . import poison_cases
    ref = poison_cases.run_cases()
    out = str(tmp_path / "poison.npz")
    env = dict(os.environ, FP8BLK_LIB=POISON_LIB)
    r = subprocess.run([sys.executable, os.path.join(HERE, "poison_cases.py"), out],
                       capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    got = np.load(out)
    assert sorted(got.files) == sorted(ref), (sorted(got.files), sorted(ref))
    for name in sorted(ref):
        nbad = int((got[name] != ref[name]).sum())
        log(f"  {name}: {ref[name].size} bytes, {nbad} differ")
        assert nbad == 0, name
