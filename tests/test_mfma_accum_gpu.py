"""How the gfx950 FP8 matrix core sums one 128-deep K block.

Page "dssusan.co.kr qna 93378", passage on accumulation precision: FP8 GEMM
on H800 Tensor Cores keeps only about 14 bits of the sum, which is why the
method promotes partial sums to FP32 at a fixed K interval.  These tests
measure the matching property of V_MFMA_F32_16X16X128_F8F6F4 on gfx950,
through the library's own product path.

With K = 128, unit scales and FP32 output, fp8_block_gemm returns the matrix
core's sum itself: the one promotion FMA multiplies it by 1.0 into a zero
accumulator, which is exact.  The exact sum of the FP8 products is the
oracle's binary64 GEMM; it is exact here, since every product is a multiple
of 2^-18 below 2^18 and 128 of them fit in binary64's 53 bits.

What the measurements show (and the tests assert):
  - the 128 products of an output are summed in 16 aligned groups of 8
    consecutive k;
  - inside a group every product is aligned to the group's largest one and
    truncated toward zero below 2^-13 of that product's leading bit: 14
    significant bits, the H800 figure;
  - the 16 group sums are added at FP32 precision or better.
So the per-block FP32 promotion is the right interval on this machine too:
within one instruction the error is bounded by the group truncation, and
the FP32 accumulators keep it from growing with K.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_token_amd import binding as B
from fp8_fine_grained_token_amd import inputs as I

from .gpu_util import dev, host, log, torch

pytestmark = pytest.mark.gpu

K = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    t.cuda.synchronize()


def code(v: float) -> int:
    """E4M3 code of a value the format represents exactly."""
    c = int(oracle.e4m3_encode(np.float32(v)).reshape(-1)[0])
    assert oracle.e4m3_value(c) == v, v
    return c


def mfma_sum(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """C[m][n] = the matrix core's sum over k of dec(a[m][k]) dec(w[n][k])."""
    M, N = a.shape[0], w.shape[0]
    sa = np.ones((M, 1), np.float32)
    sw = np.ones((N // 128, 1), np.float32)
    c = B.fp8_block_gemm(dev(a), dev(sa), dev(w), dev(sw), out_dtype="f32")
    return host(c).astype(np.float64)


def exact_sum(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    return oracle.block_gemm(a, np.ones((a.shape[0], 1), np.float32), w,
                             np.ones((w.shape[0] // 128, 1), np.float32))


def test_small_addend_survives_only_within_14_bits_of_its_group_max():
    """One product 2^16 at k = b and one product 2^(16 - d) at k = k_n.  In
    the same group of 8 the small one survives exactly for d <= 13 and is
    lost for d >= 14; in any other group it survives (d <= 23, what an FP32
    output next to 2^16 can show)."""
    s_rows = np.arange(15)                      # a = 2^(8 - s)
    big = code(256.0)
    for b in (0, 37, 127):
        a = np.zeros((s_rows.size, K), np.uint8)
        a[:, :] = np.array([code(2.0 ** (8 - s)) for s in s_rows], np.uint8)[:, None]
        a[:, b] = big
        w = np.zeros((128, K), np.uint8)
        t_col = 9 * (np.arange(128) % 2)        # w = 2^(8 - t), t in {0, 9}
        # addend positions b - 32 .. b + 31 (mod 128): two groups on each
        # side and b's own; k = b itself is replaced by b's pair neighbour
        k_col = np.array([(b - 32 + n // 2) % K for n in range(128)])
        k_col[k_col == b] = b ^ 1
        for n in range(128):
            w[n, b] = big
            w[n, k_col[n]] = code(2.0 ** (8 - t_col[n]))
        c = mfma_sum(a, w)
        exact = exact_sum(a, w)
        for m, s in enumerate(s_rows):
            for n in range(128):
                d = s + t_col[n]
                same_group = k_col[n] // 8 == b // 8
                want = 2.0 ** 16 + (0.0 if (same_group and d >= 14) else 2.0 ** (16 - d))
                assert exact[m, n] == 2.0 ** 16 + 2.0 ** (16 - d)
                assert c[m, n] == want, (b, int(k_col[n]), int(d), c[m, n] - 2.0 ** 16)
    log("  addends 2^-d of the group max: exact for d <= 13, dropped for d >= 14, "
        "kept when in another group of 8")


def test_truncation_toward_zero_in_the_group():
    """2^16 and v at k = 0, 1 (one group): v is cut to a multiple of
    2^(16 - 13) = 8, toward zero, for either sign."""
    vals = [2.0, 3.0, 4.0, 6.0, 7.0, 8.0, 9.0, 11.0, 12.0, 13.0, 14.0, 15.0, 20.0, 28.0]
    vals = vals + [-v for v in vals]
    a = np.zeros((len(vals), K), np.uint8)
    a[:, 0] = code(256.0)
    for m, v in enumerate(vals):
        a[m, 1] = code(v)
    w = np.zeros((128, K), np.uint8)
    w[:, 0] = code(256.0)
    w[:, 1] = code(1.0)
    c = mfma_sum(a, w)
    for m, v in enumerate(vals):
        want = 2.0 ** 16 + 8.0 * np.trunc(v / 8.0)
        assert c[m, 0] == want, (v, c[m, 0] - 2.0 ** 16)


def test_group_sums_add_at_fp32_precision():
    """Group 0 holds 2^16, group g (g = 1..15) the single product 2^(-7):
    one FP32 unit in the last place of 2^16 each.  All fifteen survive."""
    a = np.zeros((16, K), np.uint8)
    a[:, 0] = code(256.0)
    w = np.zeros((128, K), np.uint8)
    w[:, 0] = code(256.0)
    for g in range(1, 16):
        a[:, 8 * g + 3] = code(2.0 ** -3)
        w[:, 8 * g + 3] = code(2.0 ** -4)
    c = mfma_sum(a, w)
    assert np.all(c == 2.0 ** 16 + 15 * 2.0 ** -7), np.unique(c - 2.0 ** 16)


@pytest.mark.parametrize("seed", [0, 1])
def test_error_within_the_group_truncation_bound(seed):
    """Seeded activations (1% outlier channels x50) and weights, quantized by
    the oracle: every output's error against the exact sum is within what
    the truncation allows, sum over groups of 7 * 2^(e_g - 13) (e_g the
    exponent of the group's largest |product|), plus 16 FP32 roundings of
    the group additions."""
    g = I.gemm_inputs(64, 256, K, seed=seed, outlier_frac=0.01, outlier_mult=50.0)
    qa, _ = oracle.quant_act_1x128(g.a_bf16)
    qw, _ = oracle.quant_weight_128x128(g.w_bf16)
    c = mfma_sum(qa, qw)
    exact = exact_sum(qa, qw)
    lut = np.array([oracle.e4m3_value(i) if (i & 0x7F) != 0x7F else 0.0 for i in range(256)])
    p = lut[qa][:, None, :] * lut[qw][None, :, :]              # [M][N][K] exact products
    gmax = np.abs(p).reshape(p.shape[0], p.shape[1], 16, 8).max(axis=3)
    with np.errstate(divide="ignore"):
        e = np.where(gmax > 0, np.floor(np.log2(np.where(gmax > 0, gmax, 1.0))), -np.inf)
    trunc = (7.0 * np.exp2(e - 13)).sum(axis=2)
    bound = trunc + 16 * 2.0 ** -24 * np.abs(p).sum(axis=2)
    err = np.abs(c - exact)
    ratio = float((err / bound).max())
    scale = np.abs(p).sum(axis=2)
    log(f"  seed {seed}: max |error| / bound = {ratio:.3f}, "
        f"max |error| / sum |products| = {float((err / np.maximum(scale, 1e-30)).max()):.2e}")
    assert np.all(err <= bound)
    assert np.any(err > 0), "the matrix core was exact on every output"
