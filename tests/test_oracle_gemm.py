"""Pins for the oracle's block-scaled GEMM references (CPU only).

The pages fix that the GEMMs take FP8 operands with per-group scales running
along the inner dimension K, multiplied in as the dequantization step, with
FP32 (high-precision) accumulation and BF16/FP32 output (page "dssusan.co.kr
qna 93378", passages on scaling along K and on the GEMM operand formats).  The
plain definition the method approximates is the exact sum of dequantized
products; the oracle evaluates it in binary64.  Checked here against closed
forms, exact rational brute force, an independent dequantize (torch's float8
decode) + numpy matmul, and block additivity.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_token_amd import inputs as I

BF16_ONE = np.uint16(0x3F80)


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant(q, s, rows_per_scale):
    """Independent dequantization: torch decode times the group's scale."""
    v = torch_decode(q)
    G = s.shape[1]
    ss = np.repeat(np.repeat(s.astype(np.float64), rows_per_scale, axis=0), 128, axis=1)
    return v * ss[: q.shape[0], : q.shape[1]]


def quantized(M, N, K, seed=0, **kw):
    g = I.gemm_inputs(M, N, K, seed, **kw)
    qa, sa = oracle.quant_act_1x128(g.a_bf16)
    qw, sw = oracle.quant_weight_128x128(g.w_bf16)
    return qa, sa, qw, sw


def test_all_ones_closed_form():
    M, N, K = 4, 256, 384
    a = np.full((M, K), BF16_ONE, np.uint16)
    w = np.full((N, K), BF16_ONE, np.uint16)
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_weight_128x128(w)
    assert np.all(qa == 0x7E) and np.all(qw == 0x7E)
    s = float(np.float32(1.0) / np.float32(448.0))
    assert np.all(sa == np.float32(s)) and np.all(sw == np.float32(s))
    R = oracle.block_gemm(qa, sa, qw, sw)
    v = 448.0 * s  # exact in binary64
    expect = K * v * v
    # the oracle sums K rounded binary64 products: allow K half-ulps
    assert np.allclose(R, expect, rtol=K * 2.0 ** -53, atol=0)
    assert abs(expect - K) < K * 2.0 ** -20


def test_identity_weight_closed_form():
    # W = I (N = K): diagonal blocks hold 1.0 (-> 0x7E, s = fl32(1/448)) and
    # the off-diagonal blocks are all zero (s = 0, bytes 0), so every output is
    # a single product val(qa[m,n]) * sa[m][n/128] * 448 * fl32(1/448).
    M, K = 8, 384
    g = I.gemm_inputs(M, K, K, seed=21)
    w = np.zeros((K, K), np.uint16)
    np.fill_diagonal(w, BF16_ONE)
    qa, sa = oracle.quant_act_1x128(g.a_bf16)
    qw, sw = oracle.quant_weight_128x128(w)
    s = float(np.float32(1.0) / np.float32(448.0))
    assert np.all(np.diag(sw) == np.float32(s))
    assert np.all(sw[~np.eye(3, dtype=bool)] == 0)
    R = oracle.block_gemm(qa, sa, qw, sw)
    adeq = torch_decode(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    expect = adeq * (448.0 * s)
    assert np.allclose(R, expect, rtol=2.0 ** -52, atol=0)


def test_one_hot_activation_closed_form():
    # Row m is 1.0 at column k_m and zero elsewhere: only k_m's group is
    # nonzero, so R[m, n] = 448*fl32(1/448) * val(qw[n, k_m]) * sw[n/128][k_m/128].
    N, K = 256, 512
    rng = np.random.default_rng(22)
    cols = np.array([0, 127, 128, 300, 511])
    a = np.zeros((cols.size, K), np.uint16)
    a[np.arange(cols.size), cols] = BF16_ONE
    w = I.weights(rng, (N, K))
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_weight_128x128(w)
    R = oracle.block_gemm(qa, sa, qw, sw)
    s = float(np.float32(1.0) / np.float32(448.0))
    wv = torch_decode(qw)
    for m, k in enumerate(cols):
        expect = 448.0 * s * wv[:, k] * np.repeat(sw[:, k // 128].astype(np.float64), 128)
        assert np.allclose(R[m], expect, rtol=2.0 ** -51, atol=0)


@pytest.mark.parametrize("M,N,K", [(3, 5, 128), (2, 8, 256), (4, 3, 384)])
def test_exact_rational_brute_force(M, N, K):
    # exact sum over blocks of sa * sw * sum_k val * val, in rationals
    qa, sa, qw, sw = quantized(M, N, K, seed=M * 100 + K, outlier_frac=0.02,
                               outlier_mult=30.0)
    R = oracle.block_gemm(qa, sa, qw, sw)
    va = torch_decode(qa)
    vw = torch_decode(qw)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            mag = Fraction(0)
            for kb in range(K // 128):
                blk = sum(Fraction(va[m, k]) * Fraction(vw[n, k])
                          for k in range(kb * 128, kb * 128 + 128))
                babs = sum(abs(Fraction(va[m, k]) * Fraction(vw[n, k]))
                           for k in range(kb * 128, kb * 128 + 128))
                sc = Fraction(float(sa[m, kb])) * Fraction(float(sw[n // 128, kb]))
                tot += sc * blk
                mag += abs(sc) * babs
            # binary64 summation of K terms: error <= K * 2^-53 * sum |terms|
            assert abs(Fraction(R[m, n]) - tot) <= Fraction(K, 2 ** 53) * mag


def test_matches_independent_dequant_and_numpy_matmul():
    M, N, K = 40, 384, 1024
    qa, sa, qw, sw = quantized(M, N, K, seed=31, outlier_frac=0.01, outlier_mult=50.0)
    R = oracle.block_gemm(qa, sa, qw, sw)
    A = dequant(qa, sa, 1)
    W = dequant(qw, sw, 128)
    ref = A @ W.T
    bound = 1e-13 * (np.abs(A) @ np.abs(W).T)
    assert np.all(np.abs(R - ref) <= bound)


def test_block_additivity():
    M, N, K = 6, 256, 256
    qa, sa, qw, sw = quantized(M, N, K, seed=41)
    R = oracle.block_gemm(qa, sa, qw, sw)
    h = [(slice(0, 128), slice(0, 1)), (slice(128, 256), slice(1, 2))]
    parts = [oracle.block_gemm(np.ascontiguousarray(qa[:, ks]), np.ascontiguousarray(sa[:, gs]),
                               np.ascontiguousarray(qw[:, ks]), np.ascontiguousarray(sw[:, gs]))
             for ks, gs in h]
    A = dequant(qa, sa, 1)
    W = dequant(qw, sw, 128)
    bound = 1e-14 * (np.abs(A) @ np.abs(W).T)
    assert np.all(np.abs(R - (parts[0] + parts[1])) <= bound)


def test_row_subset_equals_full():
    qa, sa, qw, sw = quantized(20, 128, 256, seed=51)
    R = oracle.block_gemm(qa, sa, qw, sw)
    rows = np.array([19, 0, 7, 7])
    assert np.array_equal(oracle.block_gemm(qa, sa, qw, sw, rows), R[rows])


def test_grouped_equals_per_expert_dense():
    E, T, N, K = 5, 70, 128, 256
    counts = np.array([20, 0, 33, 1, 10])  # 64 of 70 rows routed; 6 spare rows
    gi = I.grouped_inputs(E, T, N, K, seed=61, counts=counts)
    qa, sa = oracle.quant_act_1x128(gi.a_bf16)
    qw, sw = oracle.quant_weight_128x128(gi.w_bf16.reshape(E * N, K))
    qw = qw.reshape(E, N, K)
    sw = sw.reshape(E, N // 128, K // 128)
    R, found = oracle.grouped_gemm(qa, sa, qw, sw, gi.offsets)
    off = gi.offsets
    assert found[: off[-1]].all() and not found[off[-1]:].any()
    assert np.isnan(R[off[-1]:]).all()
    for e in range(E):
        if counts[e] == 0:
            continue
        rows = np.arange(off[e], off[e + 1])
        ref = oracle.block_gemm(qa, sa, qw[e], sw[e], rows)
        assert np.array_equal(R[rows], ref)


def test_grouped_weight_quant_is_per_expert():
    # Because N % 128 == 0, quantizing [E*N][K] in one call equals quantizing
    # each expert's [N][K] on its own.
    rng = np.random.default_rng(71)
    w = I.weights(rng, (3, 256, 384))
    qa, sa = oracle.quant_weight_128x128(w.reshape(-1, 384))
    for e in range(3):
        qe, se = oracle.quant_weight_128x128(w[e])
        assert np.array_equal(qa[e * 256:(e + 1) * 256], qe)
        assert np.array_equal(sa[e * 2:(e + 1) * 2], se)
