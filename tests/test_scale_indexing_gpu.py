"""GPU parity with scales that differ by up to 2^10 from one group to the
next: 128x128 weight blocks, 1x128 activation groups and the 128x1 groups of
the Wgrad operands.

Each block (nb, kb) of the bf16 weights is multiplied by 2^e(nb, kb) with
e = (3 nb + 5 kb) mod 11 - 5.  A power of two leaves the E4M3 bytes of the
block unchanged and multiplies its scale exactly, so a kernel that applied
a neighbouring block's weight scale (a wrong column block, K block, chunk
buffer or chunk offset) would be off by a factor of 2 or more on the
affected outputs, far outside the per-output bound.  Shapes put tiles
across column-block boundaries (256 x 192 tiles), K-block counts that are
not a multiple of the eight-block scale chunk, and split-K ranges that start
inside a chunk.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_token_amd import binding as B
from fp8_fine_grained_token_amd import inputs as I

from .gpu_util import (check_gemm, dev, dev_bf16, gemm_error_bound, grouped_error_bound, log,
                       tile_rows, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    t.cuda.synchronize()


def block_exponent(nb, kb):
    return (3 * nb + 5 * kb) % 11 - 5


def scale_blocks(w_bits):
    """bf16 weights [..., N, K] with block (nb, kb) multiplied by 2^e(nb, kb)
    (exact: bf16 -> fp32, times a power of two, back to bf16)."""
    x = (w_bits.astype(np.uint32) << 16).view(np.float32).copy()
    N, K = x.shape[-2:]
    nb = np.arange(N)[:, None] // 128
    kb = np.arange(K)[None, :] // 128
    x *= np.exp2(block_exponent(nb, kb)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_block_exponents_reach_the_scales():
    # the construction does what the test relies on: bytes as without the
    # factors, scales multiplied by exactly 2^e(nb, kb)
    w = I.weights(np.random.default_rng(5), (384, 1280))
    q0, s0 = oracle.quant_weight_128x128(w)
    q1, s1 = oracle.quant_weight_128x128(scale_blocks(w))
    e = block_exponent(np.arange(3)[:, None], np.arange(10)[None, :])
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.exp2(e).astype(np.float32))
    assert e.max() - e.min() == 10


def inputs(M, N, K, seed):
    g = I.gemm_inputs(M, N, K, seed=seed, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa = oracle.quant_act_1x128(g.a_bf16)
    w = scale_blocks(g.w_bf16)
    qw, sw = oracle.quant_weight_128x128(w)
    return g.a_bf16, w, qa, sa, qw, sw


def rows_for(M, tile):
    return np.arange(M) if M <= 300 else tile_rows(M, tile, per_tile=2)


@pytest.mark.parametrize("M,N,K", [
    (4096, 7168, 1280),  # 256 x 256 and 256 x 192 tiles; G = 10 (a partial chunk)
    (256, 2048, 2304),   # split-K (4 splits of 5 blocks: three start inside a chunk)
    (300, 384, 1280),    # 128 x 64 tiles, ragged M, split-K
])
def test_gemm_block_varying_weight_scales(M, N, K):
    _, _, qa, sa, qw, sw = inputs(M, N, K, seed=M + N + K)
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(M, N, K, "f32")
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda") if nbytes else None
    c = B.fp8_block_gemm(dev(qa), dev(sa), dev(qw), dev(sw), out_dtype="f32", workspace=ws)
    rows = rows_for(M, 256)
    log(f"  {M}x{N}x{K} (workspace {nbytes} B): oracle on {rows.size} rows")
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    splits = max(1, nbytes // (M * N * 4))
    check_gemm(c[t.from_numpy(rows).cuda()], R, "f32", f"varying W scales {M}x{N}x{K}",
               gemm_error_bound(qa, sa, qw, sw, rows, splits=splits))


@pytest.mark.parametrize("M,N,K", [
    (4096, 1280, 7168),  # both tile widths (dX 4096 x 7168), 10 inner K blocks
    (300, 2304, 1280),   # small tiles with split-K (4 splits of 5 inner blocks)
])
def test_dgrad_transposed_reads_block_varying_weight_scales(M, N, K):
    # dX = dY W with W in its forward layout [N][K]: the weight scales are
    # read as sw[kb][n / 128] of the transposed view, per K block
    rng = np.random.default_rng(M + N + K)
    dy, _ = I.activations(rng, M, N, 0.01, 20.0)
    w = scale_blocks(I.weights(rng, (N, K)))
    qw, sw = oracle.quant_weight_128x128(w)
    qdy, sdy = oracle.quant_act_1x128(dy)
    qwt, swt = oracle.transpose_weight(qw, sw)
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(M, K, N, "f32")
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda") if nbytes else None
    c = B.fp8_block_gemm_dgrad(dev(qdy), dev(sdy), dev(qw), dev(sw), out_dtype="f32",
                               workspace=ws)
    rows = rows_for(M, 256)
    R = oracle.block_gemm(qdy, sdy, qwt, swt, rows)
    splits = max(1, nbytes // (M * K * 4))
    check_gemm(c[t.from_numpy(rows).cuda()], R, "f32", f"dgrad varying W scales {M}x{N}x{K}",
               gemm_error_bound(qdy, sdy, qwt, swt, rows, splits=splits))


@pytest.mark.parametrize("M,N,K,split", [
    (4096, 256, 2304, True),   # 64-row tiles with split-K (ranges start inside chunks)
    (130, 384, 1280, False),   # a half-filled second column tile, G = 10
])
def test_fused_block_varying_weight_scales(M, N, K, split):
    a, _, qa, sa, qw, sw = inputs(M, N, K, seed=M + 2 * N + K)
    t = torch()
    ws = None
    if split:
        nbytes = B.fp8_fused_quant_kernel_workspace_bytes(M, N, K, "f32")
        assert nbytes > 0, "shape has no split-K plan"
        ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    c = B.fp8_block_gemm_fused_quant(dev_bf16(a), dev(qw), dev(sw), out_dtype="f32",
                                     workspace=ws)
    rows = rows_for(M, 64)
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    splits = max(1, (ws.numel() if ws is not None else 0) // (M * N * 4))
    check_gemm(c[t.from_numpy(rows).cuda()], R, "f32", f"fused varying W scales {M}x{N}x{K}",
               gemm_error_bound(qa, sa, qw, sw, rows, splits=splits))


def test_grouped_block_varying_weight_scales():
    # per-expert weights with the same block pattern; G = 18 (a partial
    # chunk), two column tiles, an empty expert and a one-row expert
    counts = [0, 1, 129, 300]
    E, N, K = 4, 512, 2304
    T = sum(counts)
    gi = I.grouped_inputs(E, T, N, K, seed=77, counts=counts)
    qa, sa = oracle.quant_act_1x128(gi.a_bf16)
    w = scale_blocks(gi.w_bf16)
    qw, sw = oracle.quant_weight_128x128(w.reshape(E * N, K))
    qw, sw = qw.reshape(E, N, K), sw.reshape(E, N // 128, K // 128)
    R, _ = oracle.grouped_gemm(qa, sa, qw, sw, gi.offsets)
    c = B.fp8_block_grouped_gemm(dev(qa), dev(sa), dev(qw), dev(sw),
                                 dev(gi.offsets.astype(np.int32)), out_dtype="f32")
    check_gemm(c, R, "f32", "grouped varying W scales",
               grouped_error_bound(qa, sa, qw, sw, gi.offsets, np.arange(T)))


# ---- activation scales and Wgrad row scales ---------------------------------

def group_exponent(r, kb):
    return (7 * r + 3 * kb) % 11 - 5


def scale_groups(a_bits, along_rows=False):
    """bf16 [R][C] with each 1x128 group (row r, column block kb) multiplied
    by 2^group_exponent(r, kb); with along_rows, each 128x1 group (row block
    r // 128, column c) by 2^group_exponent(c, r // 128) instead."""
    x = (a_bits.astype(np.uint32) << 16).view(np.float32).copy()
    R, C = x.shape
    r = np.arange(R)[:, None]
    c = np.arange(C)[None, :]
    e = group_exponent(c, r // 128) if along_rows else group_exponent(r, c // 128)
    x *= np.exp2(e).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_group_exponents_reach_the_scales():
    a, _ = I.activations(np.random.default_rng(9), 37, 1280, 0.01, 20.0)
    q0, s0 = oracle.quant_act_1x128(a)
    q1, s1 = oracle.quant_act_1x128(scale_groups(a))
    e = group_exponent(np.arange(37)[:, None], np.arange(10)[None, :])
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.exp2(e).astype(np.float32))
    t0, u0 = oracle.quant_act_128x1_t(a)
    t1, u1 = oracle.quant_act_128x1_t(scale_groups(a, along_rows=True))
    assert np.array_equal(t0, t1)
    e_t = group_exponent(np.arange(1280)[:, None], np.arange(1)[None, :])
    assert np.array_equal(u1, u0 * np.exp2(e_t).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [
    (4096, 7168, 1280),  # both tile widths; a partial activation-scale chunk
    (300, 384, 2304),    # small tiles with split-K inside chunks; G = 18
])
def test_gemm_group_varying_activation_scales(M, N, K):
    # activation scales 2^10 apart from group to group and row to row, with
    # the weight-block pattern as well: a wrong row, K block, piece or chunk
    # of the activation scales lands far outside the bound
    g = I.gemm_inputs(M, N, K, seed=M + N + K + 1, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa = oracle.quant_act_1x128(scale_groups(g.a_bf16))
    qw, sw = oracle.quant_weight_128x128(scale_blocks(g.w_bf16))
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(M, N, K, "f32")
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda") if nbytes else None
    c = B.fp8_block_gemm(dev(qa), dev(sa), dev(qw), dev(sw), out_dtype="f32", workspace=ws)
    rows = rows_for(M, 256)
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    splits = max(1, nbytes // (M * N * 4))
    check_gemm(c[t.from_numpy(rows).cuda()], R, "f32", f"varying A scales {M}x{N}x{K}",
               gemm_error_bound(qa, sa, qw, sw, rows, splits=splits))


@pytest.mark.parametrize("T,N,K", [(384, 300, 640), (1152, 1100, 2304)])
def test_wgrad_group_varying_row_scales(T, N, K):
    # dW = dY^T X from 128x1 groups whose scales are 2^10 apart (row chunks
    # of both operands, T / 128 = 3 or 9 K blocks: partial chunks of 4)
    rng = np.random.default_rng(T + N + K)
    dy, _ = I.activations(rng, T, N, 0.0, 1.0)
    x, _ = I.activations(rng, T, K, 0.01, 50.0)
    qdy, sdy = oracle.quant_act_128x1_t(scale_groups(dy, along_rows=True))   # [N][T]
    qx, sx = oracle.quant_act_128x1_t(scale_groups(x, along_rows=True))      # [K][T]
    rows = np.arange(N) if N <= 300 else tile_rows(N, 128, per_tile=2)
    R = oracle.rowscaled_gemm(qdy, sdy, qx, sx, rows)
    c = B.fp8_block_gemm_wgrad(dev(qdy), dev(sdy), dev(qx), dev(sx), out_dtype="f32")
    check_gemm(c[torch().from_numpy(rows).cuda()], R, "f32", f"wgrad varying scales {N}x{K}",
               gemm_error_bound(qdy, sdy, qx, sx, rows, row_scaled_w=True))
