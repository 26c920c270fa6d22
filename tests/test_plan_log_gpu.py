"""FP8BLK_LOG: with it set, every GEMM call prints the plan it launches.

The flag is read once per process, so the calls run in a child Python
process started with FP8BLK_LOG=1; its stderr must name the expected plan
for each entry point (two tile widths for 4096 x 7168, split-K for a small
M with a workspace, the unsplit small-tile plan without one, the grouped,
fused, Dgrad and Wgrad kernels, the fused entry point's staged plan with its
workspace, and the pow2 Wgrad's 256-row tiles).
"""
import os
import subprocess
import sys

import pytest

from .gpu_util import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, %r)
import numpy as np, torch
import fp8_fine_grained_token_amd as F
def q8(r, c):
    x = torch.randn(r, c, device="cuda").to(torch.bfloat16)
    return F.fp8_quant_act_1x128(x)
def w8(r, c):
    w = (0.02 * torch.randn(r, c, device="cuda")).to(torch.bfloat16)
    return F.fp8_quant_weight_128x128(w)
qa, sa = q8(4096, 1024); qw, sw = w8(7168, 1024)
F.fp8_block_gemm(qa, sa, qw, sw)
qa2, sa2 = q8(64, 2048); qw2, sw2 = w8(1024, 2048)
ws = torch.empty(F.fp8_gemm_workspace_bytes(64, 1024, 2048), dtype=torch.uint8, device="cuda")
F.fp8_block_gemm(qa2, sa2, qw2, sw2, workspace=ws)
F.fp8_block_gemm(qa2, sa2, qw2, sw2)
x = torch.randn(64, 2048, device="cuda").to(torch.bfloat16)
F.fp8_block_gemm_fused_quant(x, qw2, sw2)
wsf = torch.empty(F.fp8_fused_quant_workspace_bytes(64, 1024, 2048), dtype=torch.uint8,
                  device="cuda")
F.fp8_block_gemm_fused_quant(x, qw2, sw2, workspace=wsf)
qg, sg = q8(300, 256); wg, swg = w8(2 * 256, 256)
off = torch.tensor([0, 100, 300], dtype=torch.int32, device="cuda")
F.fp8_block_grouped_gemm(qg, sg, wg.view(2, 256, 256), swg.view(2, 2, 2), off)
qd, sd = q8(64, 1024)
F.fp8_block_gemm_dgrad(qd, sd, qw2, sw2, out_dtype="f32")
xt = torch.randn(256, 384, device="cuda").to(torch.bfloat16)
dyt = torch.randn(256, 512, device="cuda").to(torch.bfloat16)
qx, sx = F.fp8_quant_act_128x1_t(xt)
qy, sy = F.fp8_quant_act_128x1_t(dyt)
F.fp8_block_gemm_wgrad(qy, sy, qx, sx)
qy2, sy2 = F.fp8_quant_act_128x1_t_pow2(dyt)
qx2, sx2 = F.fp8_quant_act_128x1_t_pow2(xt)
F.fp8_block_gemm_wgrad_pow2(qy2, sy2, qx2, sx2)
torch.cuda.synchronize()
print("child done", flush=True)
""" % ROOT


def test_plan_log_lines():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, FP8BLK_LOG="1")
    r = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "child done" in r.stdout
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("fp8blk: ")]
    print("\n".join(lines))
    expect = [
        "block_gemm M=4096 N=7168 K=1024 tiles=256x256+256x192",
        "block_gemm M=64 N=1024 K=2048 tiles=128x64 split-K + reduction",
        "block_gemm M=64 N=1024 K=2048 tiles=128x64 ksplit=1",
        "block_gemm_fused_quant M=64 N=1024 K=2048 tiles=64x256",
        "block_gemm_fused_quant M=64 N=1024 K=2048 plan=staged",
        "block_gemm M=64 N=1024 K=2048 tiles=128x64 split-K + reduction",
        "block_grouped_gemm M=300 N=256 K=256 tiles=128x256",
        "block_gemm_dgrad (W read transposed) M=64 N=2048 K=1024",
        "block_gemm_wgrad M=512 N=384 K=256",
        "block_gemm_wgrad_pow2 M=512 N=384 K=256 tiles=256x256",
    ]
    assert len(lines) == len(expect), lines
    for ln, e in zip(lines, expect):
        assert e in ln, (ln, e)


def test_no_plan_log_by_default():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ)
    env.pop("FP8BLK_LOG", None)
    r = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    assert not [ln for ln in r.stderr.splitlines() if ln.startswith("fp8blk: ")]
