"""GPU parity of the backward-pass pieces (Dgrad and Wgrad).

Page "dssusan.co.kr qna 93378": E4M3 in Fprop, Dgrad and Wgrad; FP8 Wgrad
keeps activations in FP8; per-group scales along each GEMM's inner
dimension.  Reading for the transposed axis: Dgrad = forward GEMM of dY
(1x128 tiles) with the transposed 128x128-quantized weights; Wgrad = GEMM of
128x1-grouped dY and X, written transposed, with one scale per row on both
operands.  The 128x1 quantizer and the weight transpose must match the
oracle bit for bit; the GEMMs must meet the same tolerances as the forward.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_token_amd import binding as B
from fp8_fine_grained_token_amd import inputs as I

from .gpu_util import check_gemm, dev, dev_bf16, gemm_error_bound, host, log, tile_rows, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    t.cuda.synchronize()


def assert_bytes_and_scales(qg, sg, qo, so, what):
    nbad = int((qg != qo).sum())
    sbad = int((sg.view(np.uint32) != so.view(np.uint32)).sum())
    log(f"  {what}: byte mismatches={nbad} scale mismatches={sbad}")
    assert nbad == 0 and sbad == 0


@pytest.mark.parametrize("M,K", [(128, 64), (300, 200), (129, 130), (1, 5), (4096, 7168),
                                 (200, 72)])
def test_quant_128x1_transposed(M, K):
    # (300, 200): partial token group and partial column tile; (129, 130)
    # and (1, 5): the scalar load and byte store paths; (200, 72): vector
    # loads with byte stores (M % 16 != 0)
    x, _ = I.activations(np.random.default_rng(M + 3 * K), M, K, 0.01, 50.0)
    qo, so = oracle.quant_act_128x1_t(x)
    q, s = B.fp8_quant_act_128x1_t(dev_bf16(x))
    assert_bytes_and_scales(host(q), host(s), qo, so, f"128x1 transposed {M}x{K}")


def test_quant_128x1_transposed_zero_and_tiny_groups():
    x, _ = I.activations(np.random.default_rng(41), 256, 128, 0.0, 1.0)
    x = x.copy()
    x[:128, 3] = 0                 # all-zero group: zero scale and bytes
    x[128:, 5] = 0x8000            # all -0 group
    x[:128, 7] = 0x0001            # subnormal amax
    x[128:, 9] = 0x7F7F            # largest bf16
    qo, so = oracle.quant_act_128x1_t(x)
    q, s = B.fp8_quant_act_128x1_t(dev_bf16(x))
    assert_bytes_and_scales(host(q), host(s), qo, so, "128x1 special groups")


@pytest.mark.parametrize("N,K", [(256, 512), (200, 130), (7168, 7168), (3, 5), (384, 256),
                                 (208, 336), (1040, 144)])
def test_transpose_weight(N, K):
    # (200, 130), (3, 5): the byte-wise kernel; the rest the vector kernel,
    # (208, 336) and (1040, 144) with partial edge tiles
    w = I.weights(np.random.default_rng(N + K + 7), (N, K))
    qw, sw = oracle.quant_weight_128x128(w)
    qo, so = oracle.transpose_weight(qw, sw)
    q, s = B.fp8_transpose_weight_128x128(dev(qw), dev(sw))
    assert_bytes_and_scales(host(q), host(s), qo, so, f"weight transpose {N}x{K}")


# ---- Dgrad ----------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(64, 256, 384), (4096, 7168, 7168)])
def test_dgrad_chain(M, N, K):
    # dX [M][K] = dY [M][N] W [N][K]: GPU quantizer, GPU transpose and the
    # forward GEMM, against the oracle's chain (bytes compared on the way)
    rng = np.random.default_rng(M + N + K)
    dy, _ = I.activations(rng, M, N, 0.0, 1.0)
    w = I.weights(rng, (N, K))
    qw, sw = oracle.quant_weight_128x128(w)
    qdy_o, sdy_o = oracle.quant_act_1x128(dy)
    qwt_o, swt_o = oracle.transpose_weight(qw, sw)
    qdy, sdy = B.fp8_quant_act_1x128(dev_bf16(dy))
    qwt, swt = B.fp8_transpose_weight_128x128(dev(qw), dev(sw))
    assert_bytes_and_scales(host(qdy), host(sdy), qdy_o, sdy_o, "dY 1x128")
    assert_bytes_and_scales(host(qwt), host(swt), qwt_o, swt_o, "W^T")
    rows = np.arange(M) if M <= 256 else tile_rows(M, 256, per_tile=1)
    R = oracle.block_gemm(qdy_o, sdy_o, qwt_o, swt_o, rows)
    b = gemm_error_bound(qdy_o, sdy_o, qwt_o, swt_o, rows)
    for out in ("f32", "bf16"):
        c = B.fp8_block_gemm(qdy, sdy, qwt, swt, out_dtype=out)
        check_gemm(c[torch().from_numpy(rows).cuda()], R, out, f"dgrad {M}x{K}x{N} {out}", b)


# ---- Wgrad ----------------------------------------------------------------------

def wgrad_operands(T, N, K, seed):
    rng = np.random.default_rng(seed)
    dy, _ = I.activations(rng, T, N, 0.0, 1.0)
    x, _ = I.activations(rng, T, K, 0.01, 50.0)
    return dy, x


@pytest.mark.parametrize("T,N,K", [(128, 128, 128), (512, 300, 256), (384, 64, 640)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_wgrad_small(T, N, K, out):
    dy, x = wgrad_operands(T, N, K, T + N + K)
    qdy, sdy = oracle.quant_act_128x1_t(dy)     # [N][T]
    qx, sx = oracle.quant_act_128x1_t(x)        # [K][T]
    R = oracle.rowscaled_gemm(qdy, sdy, qx, sx)
    c = B.fp8_block_gemm_wgrad(dev(qdy), dev(sdy), dev(qx), dev(sx), out_dtype=out)
    check_gemm(c, R, out, f"wgrad {N}x{K} over {T} tokens {out}",
               gemm_error_bound(qdy, sdy, qx, sx, row_scaled_w=True))


@pytest.mark.parametrize("T,N,K,rows", [
    # 9 row tiles x 39 columns of 192-wide tiles (351 tiles, more than one
    # round; the last column tile covers 128 of its 192 columns, the last row
    # tile 76 rows)
    (256, 1100, 7424, [0, 1, 127, 128, 555, 1023, 1024, 1099]),
    # 16 row tiles: 10 columns of 256-wide tiles, then 22 of 192-wide tiles
    # from column 2560 (the last row tile 80 rows)
    (256, 2000, 6784, [0, 127, 128, 1023, 1024, 1919, 1920, 1999]),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_wgrad_two_tile_widths_sampled_rows(T, N, K, rows, out):
    dy, x = wgrad_operands(T, N, K, T + N + K)
    qdy, sdy = oracle.quant_act_128x1_t(dy)     # [N][T]
    qx, sx = oracle.quant_act_128x1_t(x)        # [K][T]
    rows = np.array(rows)
    R = oracle.rowscaled_gemm(qdy, sdy, qx, sx, rows)
    c = B.fp8_block_gemm_wgrad(dev(qdy), dev(sdy), dev(qx), dev(sx), out_dtype=out)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, out,
               f"wgrad {N}x{K} over {T} tokens {out}, sampled rows",
               gemm_error_bound(qdy, sdy, qx, sx, rows, row_scaled_w=True))


def test_wgrad_workload_chain_sampled_rows_and_deterministic():
    # dW [7168][7168] over 4096 tokens: GPU 128x1 quantizers feed the GPU
    # GEMM; sampled rows against the oracle chain; repeated calls bitwise
    # equal
    T, N, K = 4096, 7168, 7168
    dy, x = wgrad_operands(T, N, K, 42)
    qdy, sdy = B.fp8_quant_act_128x1_t(dev_bf16(dy))
    qx, sx = B.fp8_quant_act_128x1_t(dev_bf16(x))
    log("  oracle 128x1 quantization of dY and X ...")
    qdy_o, sdy_o = oracle.quant_act_128x1_t(dy)
    qx_o, sx_o = oracle.quant_act_128x1_t(x)
    assert_bytes_and_scales(host(qdy), host(sdy), qdy_o, sdy_o, "dY^T 128x1")
    assert_bytes_and_scales(host(qx), host(sx), qx_o, sx_o, "X^T 128x1")
    c0 = B.fp8_block_gemm_wgrad(qdy, sdy, qx, sx, out_dtype="f32")
    c1 = B.fp8_block_gemm_wgrad(qdy, sdy, qx, sx, out_dtype="f32")
    assert torch().equal(c0, c1)
    rows = tile_rows(N, 128, per_tile=1)
    log(f"  oracle Wgrad on {rows.size} rows of 7168x7168 over 4096 tokens ...")
    R = oracle.rowscaled_gemm(qdy_o, sdy_o, qx_o, sx_o, rows)
    check_gemm(c0[torch().from_numpy(rows).cuda()], R, "f32", "wgrad workload rows",
               gemm_error_bound(qdy_o, sdy_o, qx_o, sx_o, rows, row_scaled_w=True))


# ---- Dgrad with W read transposed inside the GEMM -------------------------------

@pytest.mark.parametrize("M,N,K", [
    (64, 256, 384),      # small tiles, one output tile row
    (300, 384, 640),     # small tiles, ragged M
    (256, 7168, 2048),   # small tiles with split-K through a workspace
    (4000, 1280, 7040),  # 256 x 256 tiles, ragged M, the last 128 output columns
                         # of a 256-wide tile past K (read, never stored)
    (4096, 512, 6144),   # 256 x 192 tiles only (12 chunks per LDS row, rotated)
    (4096, 384, 7168),   # both tile widths (256 x 256 and 256 x 192)
])
def test_dgrad_transposed_reads(M, N, K):
    # dX [M][K] = dY [M][N] W [N][K] with W in its forward layout: against
    # the oracle (every row up to 300, else rows of every tile) within the
    # per-output bound, and FP32 bitwise equal to the forward GEMM on the
    # transposed copy of W (the same bytes and block products per output)
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    dy, _ = I.activations(rng, M, N, 0.01, 20.0)
    w = I.weights(rng, (N, K))
    qw, sw = oracle.quant_weight_128x128(w)
    qdy, sdy = oracle.quant_act_1x128(dy)
    qwt, swt = oracle.transpose_weight(qw, sw)
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(M, K, N, "f32")
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda") if nbytes else None
    d = [dev(qdy), dev(sdy), dev(qw), dev(sw)]
    c32 = B.fp8_block_gemm_dgrad(*d, out_dtype="f32", workspace=ws)
    c16 = B.fp8_block_gemm_dgrad(*d, out_dtype="bf16", workspace=ws)
    ref = B.fp8_block_gemm(dev(qdy), dev(sdy), dev(qwt), dev(swt), out_dtype="f32", workspace=ws)
    rows = np.arange(M) if M <= 300 else tile_rows(M, 256, per_tile=2)
    log(f"  dgrad {M}x{N}x{K} (split-K workspace {nbytes} B): oracle on {rows.size} rows ...")
    R = oracle.block_gemm(qdy, sdy, qwt, swt, rows)
    splits = max(1, nbytes // (M * K * 4))
    b = gemm_error_bound(qdy, sdy, qwt, swt, rows, splits=splits)
    ri = t.from_numpy(rows).cuda()
    check_gemm(c32[ri], R, "f32", f"dgrad transposed reads {M}x{N}x{K} f32", b)
    check_gemm(c16[ri], R, "bf16", f"dgrad transposed reads {M}x{N}x{K} bf16", b)
    assert t.equal(c32, ref), "transposed-read Dgrad differs from the GEMM on W^T"


def test_dgrad_transposed_reads_workload():
    # the 4096 x 7168 x 7168 layer: GPU chain (1x128 quantizer on dY, Dgrad
    # on the forward weights), rows of every 256-row tile against the oracle
    M, N, K = 4096, 7168, 7168
    rng = np.random.default_rng(17)
    dy, _ = I.activations(rng, M, N, 0.0, 1.0)
    w = I.weights(rng, (N, K))
    qw, sw = oracle.quant_weight_128x128(w)
    qdy_o, sdy_o = oracle.quant_act_1x128(dy)
    qdy, sdy = B.fp8_quant_act_1x128(dev_bf16(dy))
    assert_bytes_and_scales(host(qdy), host(sdy), qdy_o, sdy_o, "dY 1x128")
    c = B.fp8_block_gemm_dgrad(qdy, sdy, dev(qw), dev(sw), out_dtype="bf16")
    qwt, swt = oracle.transpose_weight(qw, sw)
    rows = tile_rows(M, 256, per_tile=1)
    log(f"  oracle Dgrad on {rows.size} rows of {M}x{K} over {N} ...")
    R = oracle.block_gemm(qdy_o, sdy_o, qwt, swt, rows)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, "bf16", "dgrad workload rows",
               gemm_error_bound(qdy_o, sdy_o, qwt, swt, rows))
