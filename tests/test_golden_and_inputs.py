"""Oracle regression fixture and input-generator determinism (CPU only)."""
import json
import os

import numpy as np

from fp8_fine_grained_token_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_reproduces_golden_fixture():
    from tests.golden.make_golden import compute
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        stored = json.load(f)
    assert compute() == stored


def test_generator_is_deterministic_and_seeded():
    a = I.gemm_inputs(16, 128, 256, seed=3, outlier_frac=0.01, outlier_mult=50.0)
    b = I.gemm_inputs(16, 128, 256, seed=3, outlier_frac=0.01, outlier_mult=50.0)
    c = I.gemm_inputs(16, 128, 256, seed=4, outlier_frac=0.01, outlier_mult=50.0)
    assert I.sha256(a.a_bf16) == I.sha256(b.a_bf16)
    assert I.sha256(a.w_bf16) == I.sha256(b.w_bf16)
    assert I.sha256(a.a_bf16) != I.sha256(c.a_bf16)


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -2.5, 3.0e38], dtype=np.float32)
    b = I.f32_to_bf16_bits(f)
    # 1+2^-8 ties to even (1.0); 1+3*2^-8 ties up to 1+2^-6; just above a tie
    # rounds up
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F62]
    assert np.array_equal(I.bf16_bits_to_f32(b)[:1], np.float32([1.0]))


def test_outlier_channels_count_and_scale():
    x, chans = I.config_quant(seed=0, M=64)
    assert chans.size == 7  # round(0.001 * 7168)
    f = I.bf16_bits_to_f32(x)
    col_rms = np.sqrt((f.astype(np.float64) ** 2).mean(axis=0))
    assert np.all(col_rms[chans] > 30)
    assert np.median(col_rms) < 1.5


def test_zipf_routing_counts():
    rng = np.random.default_rng(0)
    counts = I.zipf_counts(rng, 8192, 32, 1.1, cap=1024)
    assert counts.sum() == 8192 and counts.max() <= 1024 and counts.min() >= 0
    assert counts[0] == 1024  # hottest expert hits the cap
    off = I.offsets_from_counts(counts)
    assert off[0] == 0 and off[-1] == 8192 and np.all(np.diff(off) == counts)
