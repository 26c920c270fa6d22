"""Pins for the oracle's E4M3 codec (CPU only).

The pages fix E4M3 (4-bit exponent, 3-bit mantissa) on all tensors (page
"dssusan.co.kr qna 93378", passage contrasting E4M3 everywhere with the hybrid
E4M3/E5M2 format); the variant (OCP E4M3FN, largest finite 448) and the
rounding (nearest, ties to even) are the readings adopted.  The oracle's table
and bisection encoder are checked against format facts and against an
independent implementation: torch's CPU float8_e4m3fn decode and cast.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_token_amd.inputs import bf16_bits_to_f32

pytestmark = pytest.mark.filterwarnings("ignore")


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_format_fixed_points():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -9          # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert v(0x08) == 2.0 ** -6          # smallest normal
    assert v(0x38) == 1.0
    assert v(0x7E) == 448.0              # largest finite
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0xFE) == -448.0


def test_table_matches_torch_decode_all_codes():
    ours = np.array([oracle.e4m3_value(c) for c in range(256)])
    ref = torch_decode(np.arange(256))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_table_strictly_increasing_127_magnitudes():
    mags = np.array([oracle.e4m3_value(c) for c in range(127)])
    assert np.all(np.diff(mags) > 0)
    assert mags.size == 127


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = np.array([oracle.e4m3_value(c) for c in codes], dtype=np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def _midpoints_and_neighbours():
    mags = np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    pts = np.concatenate([mids, up, dn, mags.astype(np.float32)])
    return np.concatenate([pts, -pts])


def test_encode_matches_torch_cast_on_ties_and_neighbours():
    y = _midpoints_and_neighbours()
    assert np.array_equal(oracle.e4m3_encode(y), torch_encode(y))


def test_ties_go_to_even_mantissa():
    mags = np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    codes = oracle.e4m3_encode(mids)
    assert np.all(codes % 2 == 0)
    # the subnormal/normal boundary: 7.5 * 2^-9 ties to 0x08 (even)
    assert oracle.e4m3_encode(np.float32(7.5 * 2 ** -9)).item() == 0x08


def test_encode_matches_torch_cast_on_every_bf16_within_range():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0)
    y = f[keep]
    assert np.array_equal(oracle.e4m3_encode(y), torch_encode(y))


def test_encode_matches_torch_cast_on_random_float32():
    rng = np.random.default_rng(1234)
    parts = []
    # uniform bit patterns restricted to |y| <= 448 (covers fp32 subnormals)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    parts.append(f[np.isfinite(f) & (np.abs(f) <= 448.0)])
    # log-uniform magnitudes over the e4m3 range and below
    mag = np.exp2(rng.uniform(-160, np.log2(448.0), size=1_000_000)).astype(np.float32)
    sign = np.where(rng.random(mag.size) < 0.5, -1, 1).astype(np.float32)
    parts.append(np.minimum(mag, np.float32(448.0)) * sign)
    y = np.concatenate(parts)
    assert np.array_equal(oracle.e4m3_encode(y), torch_encode(y))


def test_signed_zero_and_tiny_negatives():
    y = np.array([0.0, -0.0, -1e-30, 1e-30, -2.0 ** -11, 2.0 ** -11,
                  -(2.0 ** -10) * 1.0000001], dtype=np.float32)
    got = oracle.e4m3_encode(y)
    # |y| <= 2^-10 is at most half of the smallest subnormal: rounds to zero,
    # except that exactly 2^-10 ties to the even code 0; above it -> 0x81.
    assert got.tolist() == [0x00, 0x80, 0x80, 0x00, 0x80, 0x00, 0x81]


def test_saturation_at_and_above_448():
    y = np.array([448.0, 450.0, 463.9, 1e6, -448.0, -1e6], dtype=np.float32)
    assert oracle.e4m3_encode(y).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_encode_is_monotone_and_within_half_ulp():
    rng = np.random.default_rng(7)
    y = np.sort(np.exp2(rng.uniform(-12, np.log2(448.0), 200_000)).astype(np.float32))
    codes = oracle.e4m3_encode(y)
    assert np.all(np.diff(codes.astype(np.int64)) >= 0)
    vals = torch_decode(codes)
    e = np.floor(np.log2(y.astype(np.float64)))
    ulp = np.where(y >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)
    err = np.abs(y.astype(np.float64) - vals)
    assert np.all(err <= ulp / 2)
