"""GPU parity of the backward pair with power-of-two scales, through the C ABI.

fp8_quant_act_128x1_t_pow2 must equal the oracle's pow2 128x1 quantizer bit
for bit (bytes and scales).  fp8_block_gemm_wgrad_pow2 must meet the
per-output bound against the oracle's binary64 row-scaled GEMM of the
oracle's own pow2-quantized operands.  The bound is the one of the FP32-scale
path: every scale is a power of two, so applying it is exact, and the matrix
core adds each scaled K block into its FP32 accumulator with one rounding.
The GEMM's tiles (256 x 256 and 256 x 192, two LDS stages) are checked on
ragged shapes and on both plans (one tile width, two widths).
fp8_block_gemm_dgrad_pow2 (the forward weights read transposed) is checked
against the oracle within the same bound, and FP32 bitwise against
fp8_block_gemm_pow2 on the transposed copy of W, on every plan.
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


@pytest.mark.parametrize("M,K", [(128, 64), (300, 200), (129, 130), (1, 5), (200, 72)])
def test_pow2_quant_128x1_transposed(M, K):
    # partial token groups and column tiles; the scalar and vector load and
    # store paths (as for the FP32-scale quantizer)
    x, _ = I.activations(np.random.default_rng(M + 5 * K), M, K, 0.01, 50.0)
    qo, so = oracle.quant_act_128x1_t_pow2(x)
    q, s = B.fp8_quant_act_128x1_t_pow2(dev_bf16(x))
    assert_bytes_and_scales(host(q), host(s), qo, so, f"pow2 128x1 transposed {M}x{K}")


def test_pow2_quant_128x1_transposed_zero_and_tiny_groups():
    x, _ = I.activations(np.random.default_rng(43), 256, 128, 0.0, 1.0)
    x = x.copy()
    x[:128, 3] = 0                 # all-zero group: scale 2^-126, zero bytes
    x[128:, 5] = 0x8000            # all -0 group
    x[:128, 7] = 0x0001            # subnormal amax: the smallest scale
    x[128:, 9] = 0x7F7F            # largest bf16
    qo, so = oracle.quant_act_128x1_t_pow2(x)
    q, s = B.fp8_quant_act_128x1_t_pow2(dev_bf16(x))
    assert_bytes_and_scales(host(q), host(s), qo, so, "pow2 128x1 zero and tiny groups")


def wgrad_operands(T, N, K, seed):
    rng = np.random.default_rng(seed)
    dy, _ = I.activations(rng, T, N, 0.0, 1.0)
    x, _ = I.activations(rng, T, K, 0.01, 50.0)
    return dy, x


def run_wgrad(T, N, K, out, rows=None, seed=None):
    dy, x = wgrad_operands(T, N, K, T + N + K if seed is None else seed)
    qdy, sdy = oracle.quant_act_128x1_t_pow2(dy)     # [N][T]
    qx, sx = oracle.quant_act_128x1_t_pow2(x)        # [K][T]
    c = B.fp8_block_gemm_wgrad_pow2(dev(qdy), dev(sdy), dev(qx), dev(sx), out_dtype=out)
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    R = oracle.rowscaled_gemm(qdy, sdy, qx, sx, rows)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, out,
               f"pow2 wgrad {N}x{K} over {T} tokens {out}",
               gemm_error_bound(qdy, sdy, qx, sx, rows, row_scaled_w=True))


@pytest.mark.parametrize("T,N,K", [(128, 128, 128), (512, 300, 256), (384, 64, 640),
                                   (256, 520, 896)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_pow2_wgrad_small(T, N, K, out):
    # one tile width: ragged rows (300, 64, 520: a last tile of 8 rows) and
    # columns (640, 896: the last 256-wide tile half filled); K blocks 1 to
    # 4, so the scale chunks of 4 blocks are partial or whole
    run_wgrad(T, N, K, out)


@pytest.mark.parametrize("T,N,K,rows", [
    # 17 row tiles (the last holds 4 rows) x 6 columns of 256-wide tiles,
    # then 24 of 192-wide tiles from column 1536 (the last covers 64 of its
    # columns)
    (256, 4100, 6016, [0, 1, 255, 256, 2047, 4095, 4096, 4099]),
    # 192-wide tiles only: 9 row tiles (the last 152 rows), 39 column tiles
    # (the last covers 128 columns); 5 K blocks (a partial scale chunk)
    (640, 2200, 7424, [0, 255, 256, 1024, 2047, 2048, 2199]),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_pow2_wgrad_two_tile_widths_sampled_rows(T, N, K, rows, out):
    run_wgrad(T, N, K, out, rows)


def test_pow2_wgrad_workload_chain_sampled_rows_and_deterministic():
    # dW [7168][7168] over 4096 tokens: the GPU pow2 128x1 quantizers feed
    # the GPU GEMM (256 x 256 tiles on columns [0, 1024), 256 x 192 on the
    # rest); bytes and scales against the oracle; rows of every 128-row half
    # tile against the oracle chain; repeated calls bitwise equal
    T, N, K = 4096, 7168, 7168
    dy, x = wgrad_operands(T, N, K, 44)
    qdy, sdy = B.fp8_quant_act_128x1_t_pow2(dev_bf16(dy))
    qx, sx = B.fp8_quant_act_128x1_t_pow2(dev_bf16(x))
    log("  oracle pow2 128x1 quantization of dY and X ...")
    qdy_o, sdy_o = oracle.quant_act_128x1_t_pow2(dy)
    qx_o, sx_o = oracle.quant_act_128x1_t_pow2(x)
    assert_bytes_and_scales(host(qdy), host(sdy), qdy_o, sdy_o, "dY^T pow2 128x1")
    assert_bytes_and_scales(host(qx), host(sx), qx_o, sx_o, "X^T pow2 128x1")
    c0 = B.fp8_block_gemm_wgrad_pow2(qdy, sdy, qx, sx, out_dtype="f32")
    c1 = B.fp8_block_gemm_wgrad_pow2(qdy, sdy, qx, sx, out_dtype="f32")
    assert torch().equal(c0, c1)
    rows = tile_rows(N, 128, per_tile=1)
    log(f"  oracle Wgrad on {rows.size} rows of 7168x7168 over 4096 tokens ...")
    R = oracle.rowscaled_gemm(qdy_o, sdy_o, qx_o, sx_o, rows)
    check_gemm(c0[torch().from_numpy(rows).cuda()], R, "f32", "pow2 wgrad workload rows",
               gemm_error_bound(qdy_o, sdy_o, qx_o, sx_o, rows, row_scaled_w=True))


# ---- Dgrad on the forward weights, read transposed, power-of-two scales ---------

@pytest.mark.parametrize("M,N,K", [
    (64, 256, 384),      # small tiles, one output tile row
    (300, 384, 640),     # small tiles, ragged M
    (256, 7168, 2048),   # small tiles with split-K through a workspace
    (4000, 1280, 7040),  # 256 x 256 tiles, ragged M, a half-used last tile
    (4096, 512, 6144),   # 256 x 192 tiles only
    (4096, 384, 7168),   # both tile widths
])
def test_pow2_dgrad_transposed_reads(M, N, K):
    # against the oracle (every row up to 300, else rows of every tile)
    # within the per-output bound, and FP32 bitwise equal to the pow2 GEMM
    # on the transposed copy of W
    rng = np.random.default_rng(M + 5 * N + 3 * K)
    dy, _ = I.activations(rng, M, N, 0.01, 20.0)
    w = I.weights(rng, (N, K))
    qw, sw = oracle.quant_weight_128x128_pow2(w)
    qdy, sdy = oracle.quant_act_1x128_pow2(dy)
    qwt, swt = oracle.transpose_weight(qw, sw)
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(M, K, N, "f32")
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda") if nbytes else None
    d = [dev(qdy), dev(sdy), dev(qw), dev(sw)]
    c32 = B.fp8_block_gemm_dgrad_pow2(*d, out_dtype="f32", workspace=ws)
    c16 = B.fp8_block_gemm_dgrad_pow2(*d, out_dtype="bf16", workspace=ws)
    ref = B.fp8_block_gemm_pow2(dev(qdy), dev(sdy), dev(qwt), dev(swt), out_dtype="f32",
                                workspace=ws)
    rows = np.arange(M) if M <= 300 else tile_rows(M, 256, per_tile=2)
    log(f"  pow2 dgrad {M}x{N}x{K} (split-K workspace {nbytes} B): oracle on {rows.size} rows")
    R = oracle.block_gemm(qdy, sdy, qwt, swt, rows)
    b = gemm_error_bound(qdy, sdy, qwt, swt, rows, splits=max(1, nbytes // (M * K * 4)))
    ri = t.from_numpy(rows).cuda()
    check_gemm(c32[ri], R, "f32", f"pow2 dgrad {M}x{N}x{K} f32", b)
    check_gemm(c16[ri], R, "bf16", f"pow2 dgrad {M}x{N}x{K} bf16", b)
    assert t.equal(c32, ref), "transposed-read pow2 Dgrad differs from the pow2 GEMM on W^T"
