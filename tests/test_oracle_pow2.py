"""Pins for the oracle's power-of-two-scale quantizers (CPU only).

Page "kailasan.com recruit 147436", passage recommending that matrix units
take the per-group scaling factors and do the group-scaled MMA themselves;
gfx950's block-scaled MFMA takes power-of-two (E8M0) scales.  The pages give
no rule for such scales.  Reading: s = the smallest power of two with
448 s >= amax, at least 2^-126; q = E4M3 RNE of x / s (an exact quotient); an
all-zero group keeps s = 2^-126 and zero bytes.  The checks are the defining
properties of that s, an independent library cast for the codes, and the
relation to the amax / 448 quantizer, none reusing the oracle's code.
"""
import numpy as np
import torch

import oracle
from fp8_fine_grained_token_amd import inputs as I
from fp8_fine_grained_token_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits

FLOOR = 2.0 ** -126


def torch_encode(y):
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def is_normal_power_of_two(s):
    bits = np.asarray(s, np.float32).view(np.uint32)
    e = bits >> 23
    return ((bits & 0x7FFFFF) == 0) & (e >= 1) & (e <= 254)


def test_scale_is_the_smallest_power_of_two_for_every_bf16_amax():
    x, amax = I.every_amax_groups(21)
    q, s = oracle.quant_act_1x128_pow2(x)
    s = s[:, 0].astype(np.float64)
    a = amax.astype(np.float64)
    assert np.all(is_normal_power_of_two(s[:, None].astype(np.float32)))
    assert np.all(448.0 * s >= a)
    # minimal: half of it would not cover amax, unless it sits at the floor
    assert np.all((s == FLOOR) | (448.0 * (s / 2) < a))
    assert np.all(s[a < 448.0 * FLOOR] == FLOOR)


def test_codes_equal_the_library_cast_of_the_exact_quotient():
    # x / s is a power-of-two scaling, exact in binary64 and in binary32
    # (|x / s| <= 448); torch's RNE cast of it must give the oracle's bytes.
    x, _ = I.every_amax_groups(21)
    q, s = oracle.quant_act_1x128_pow2(x)
    y64 = bf16_bits_to_f32(x).astype(np.float64) / s.astype(np.float64)
    y = y64.astype(np.float32)
    assert np.array_equal(y.astype(np.float64), y64)
    assert np.abs(y).max() <= 448.0
    assert np.array_equal(q, torch_encode(y))


def test_amax_element_lands_in_the_top_binade():
    # 448 s / 2 < amax <= 448 s, so amax / s is in (224, 448] (away from the
    # floor), and its code has the largest exponent field.
    x, amax = I.every_amax_groups(21)
    q, s = oracle.quant_act_1x128_pow2(x)
    ok = amax >= 448.0 * FLOOR
    v = torch_decode(q[:, 0] & 0x7F)
    assert np.all((v[ok] >= 224.0) & (v[ok] <= 448.0))
    assert np.array_equal(q[:, 0] >> 7, (x[:, 0] >> 15).astype(np.uint8))


def test_equals_the_amax_over_448_quantizer_when_that_scale_is_a_power_of_two():
    rng = np.random.default_rng(22)
    for j in (-60, -9, 0, 5, 30):
        amax = np.float32(448.0 * 2.0 ** j)
        amax_bits = f32_to_bf16_bits(np.array([amax]))[0]
        rest = f32_to_bf16_bits(amax * rng.random((64, 127), dtype=np.float32))
        rest = np.minimum(rest, amax_bits)
        x = np.concatenate([np.full((64, 1), amax_bits, np.uint16), rest], 1)
        x |= (rng.random(x.shape) < 0.5).astype(np.uint16) << np.uint16(15)
        qp, sp = oracle.quant_act_1x128_pow2(x)
        qs, ss = oracle.quant_act_1x128(x)
        assert np.all(sp == np.float32(2.0 ** j))
        assert np.array_equal(qp, qs) and np.array_equal(sp, ss), j


def test_scale_within_a_factor_two_above_amax_over_448():
    x, _ = I.config_quant(seed=23, M=64, K=7168)
    _, sp = oracle.quant_act_1x128_pow2(x)
    _, ss = oracle.quant_act_1x128(x)
    assert np.all(sp >= ss) and np.all(sp < 2 * ss)


def test_zero_group_keeps_the_floor_scale_and_zero_bytes():
    x = np.zeros((3, 300), dtype=np.uint16)
    x[1, :] = 0x8000  # -0.0 everywhere: still an all-zero group
    x[2, 130] = 0x3F80  # 1.0 in the second group of row 2
    q, s = oracle.quant_act_1x128_pow2(x)
    assert np.all(q[0] == 0) and np.all(q[1] == 0)
    assert np.all(s[:2] == np.float32(FLOOR)) and s[2, 0] == np.float32(FLOOR)
    # 1.0: the smallest 2^E with 448 * 2^E >= 1 is 2^-8 (448 / 256 = 1.75)
    assert s[2, 1] == np.float32(2.0 ** -8)
    assert q[2, 130] == torch_encode(np.float32(256.0))
    assert np.all(np.delete(q[2], 130) == 0)


def test_round_trip_within_half_ulp():
    x, _ = I.config_quant(seed=24, M=32, K=7168)
    q, s = oracle.quant_act_1x128_pow2(x)
    f = bf16_bits_to_f32(x).reshape(32, 56, 128).astype(np.float64)
    y = (f / s[:, :, None]).reshape(32, -1)
    v = torch_decode(q)
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)
    assert np.all(np.abs(y - v) <= ulp / 2)


def test_weight_blocks_and_partial_blocks():
    rng = np.random.default_rng(25)
    w = I.weights(rng, (200, 300))
    q, s = oracle.quant_weight_128x128_pow2(w)
    assert s.shape == (2, 3)
    f = bf16_bits_to_f32(w)
    for nb, (r0, r1) in enumerate(((0, 128), (128, 200))):
        for g, (c0, c1) in enumerate(((0, 128), (128, 256), (256, 300))):
            blk = f[r0:r1, c0:c1]
            amax = float(np.abs(blk).max())
            sb = float(s[nb, g])
            assert is_normal_power_of_two(np.float32(sb))
            assert 448.0 * sb >= amax and (sb == FLOOR or 448.0 * sb / 2 < amax)
            y = (blk.astype(np.float64) / sb).astype(np.float32)
            assert np.array_equal(q[r0:r1, c0:c1], torch_encode(y))
    # N = 1: a weight block is one 1x128 group, as in the activation quantizer
    x, _ = I.config_quant(seed=26, M=1, K=1000)
    qa, sa = oracle.quant_act_1x128_pow2(x)
    qw, sw = oracle.quant_weight_128x128_pow2(x)
    assert np.array_equal(qa, qw) and np.array_equal(sa, sw)
