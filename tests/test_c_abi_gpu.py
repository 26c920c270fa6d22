"""The C ABI from a plain C99 program with no Python in its process
(tests/c_abi/c_abi_check.c, built by tests/c_abi/build.py and by
__graft_entry__.build()): quantization and the block GEMM through
include/fp8blk.h on its own HIP stream, then the grouped GEMM, the 128x1
transposed quantizer, the weight transpose, Wgrad, the GEMM with the
quantization fused in, the no-allocation GEMM and Dgrad on the forward
weights, each checked inside the program against the oracle's C functions
(bytes and scale bits equal; rel. Frobenius error <= 1e-3 for FP32 output,
<= 8e-3 for BF16; the no-allocation GEMM bitwise equal to fp8_block_gemm),
plus the documented error codes."""
import subprocess

import pytest

from .c_abi import build as cbuild
from .gpu_util import log, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("args", [(), ("1", "128", "128"), ("300", "256", "8192")])
def test_c_program_against_oracle(args):
    # (): 200 x 384 x 2688, K split four ways through the workspace, Wgrad
    # over 128 tokens; 1 x 128 x 128: one ragged token (no whole 128-token
    # block, so no Wgrad); 300 x 256 x 8192: three M tiles, Wgrad over 256
    # tokens
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    exe = cbuild.build()
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300)
    log("  " + r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("c-abi ok")
