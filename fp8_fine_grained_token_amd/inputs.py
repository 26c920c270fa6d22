"""Seeded synthetic inputs for the quantizers and the block-scaled GEMMs.

This module only draws random numbers and rounds them to bf16 storage; it
holds none of the quantization or GEMM arithmetic, so both the HIP path and
the CPU oracle can be fed from it.  Everything is numpy (PCG64 via
``default_rng``); bf16 tensors are returned as ``uint16`` bit patterns.

Recipe (shapes from the five workloads the library is measured on; the pages
fix no tensor shape):
  * activations ~ N(0, 1) in float32; a fraction of channels (chosen with
    ``rng.choice(K, round(frac*K), replace=False)`` after the main draw) is
    multiplied by an outlier factor, which exercises the per-group scaling
    that the pages motivate by outliers (page "dssusan.co.kr qna 93378",
    passage on Figure 7 (a));
  * weights ~ N(0, 0.02) in float32;
  * float32 -> bf16 by round-to-nearest-even on the dropped 16 bits;
  * MoE routing: expert popularity p_e ~ (e+1)^-1.1 (Zipf, s = 1.1), token
    counts ~ Multinomial(T, p) then capped at a per-expert maximum by
    re-drawing the excess over the experts below the cap; tokens are stored
    sorted by expert, so offsets are the exclusive prefix sum of the counts.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "normal_bf16", "activations",
    "weights", "zipf_counts", "offsets_from_counts", "sha256",
    "GemmInputs", "GroupedInputs", "config_tiny", "config_quant",
    "config_dense", "config_decode", "config_grouped", "gemm_inputs",
    "grouped_inputs",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.
    Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) drawn in float32, rounded to bf16 bits."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def activations(rng: np.random.Generator, M: int, K: int,
                outlier_frac: float = 0.0, outlier_mult: float = 1.0):
    """Token activations [M][K]: N(0,1) float32, then round(frac*K) outlier
    channels scaled by ``outlier_mult``, then bf16.  Returns (bits, channels)."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    chans = np.zeros(0, dtype=np.int64)
    if n_out > 0:
        chans = np.sort(rng.choice(K, n_out, replace=False))
        x[:, chans] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x), chans


def weights(rng: np.random.Generator, shape, sigma: float = 0.02) -> np.ndarray:
    return normal_bf16(rng, shape, sigma)


def every_amax_groups(seed: int) -> tuple[np.ndarray, np.ndarray]:
    """One 128-element bf16 group per positive finite bf16 value A (32,639
    groups): A itself, then 127 random magnitudes <= A, random signs.
    Returns (bits [32639][128], A as float32)."""
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(seed)
    amax = bf16_bits_to_f32(amax_bits)
    rest = f32_to_bf16_bits(amax[:, None] * rng.random((amax.size, 127), dtype=np.float32))
    rest = np.minimum(rest, amax_bits[:, None])
    sign = (rng.random((amax.size, 128)) < 0.5).astype(np.uint16) << np.uint16(15)
    return np.concatenate([amax_bits[:, None], rest], axis=1) | sign, amax


def zipf_counts(rng: np.random.Generator, T: int, E: int, s: float = 1.1,
                cap: int | None = None) -> np.ndarray:
    """Tokens per expert: Multinomial(T, p_e ~ (e+1)^-s), expert 0 hottest.
    With ``cap``, counts above it are clipped and the excess is re-drawn over
    the experts still below the cap (renormalised p), until none exceeds it."""
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    counts = rng.multinomial(T, p).astype(np.int64)
    if cap is not None:
        if cap * E < T:
            raise ValueError("cap too small for the token count")
        while (counts > cap).any():
            excess = int(np.maximum(counts - cap, 0).sum())
            counts = np.minimum(counts, cap)
            open_ = counts < cap
            q = np.where(open_, p, 0.0)
            q /= q.sum()
            counts = counts + rng.multinomial(excess, q)
    return counts


def offsets_from_counts(counts: np.ndarray) -> np.ndarray:
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@dataclass
class GemmInputs:
    name: str
    M: int
    N: int
    K: int
    a_bf16: np.ndarray          # uint16 [M][K]
    w_bf16: np.ndarray          # uint16 [N][K]
    out_dtype: str              # "f32" or "bf16"
    outlier_channels: np.ndarray = field(default_factory=lambda: np.zeros(0))


@dataclass
class GroupedInputs:
    name: str
    E: int
    T: int
    N: int
    K: int
    counts: np.ndarray          # int64 [E]
    offsets: np.ndarray         # int32 [E+1]
    a_bf16: np.ndarray          # uint16 [T][K], rows sorted by expert
    w_bf16: np.ndarray          # uint16 [E][N][K]
    out_dtype: str


def gemm_inputs(M: int, N: int, K: int, seed: int = 0, out_dtype: str = "bf16",
                outlier_frac: float = 0.0, outlier_mult: float = 1.0,
                w_sigma: float = 0.02, name: str = "custom") -> GemmInputs:
    """Dense GEMM operands: activations first, then weights, one generator."""
    rng = np.random.default_rng(seed)
    a, chans = activations(rng, M, K, outlier_frac, outlier_mult)
    w = weights(rng, (N, K), w_sigma)
    return GemmInputs(name, M, N, K, a, w, out_dtype, chans)


def grouped_inputs(E: int, T: int, N: int, K: int, seed: int = 0,
                   cap: int | None = None, counts=None, out_dtype: str = "bf16",
                   w_sigma: float = 0.02, name: str = "custom") -> GroupedInputs:
    """Grouped GEMM operands: routing counts first (unless given), then
    activations [T][K] (already in expert order), then weights [E][N][K]."""
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = zipf_counts(rng, T, E, 1.1, cap)
    counts = np.asarray(counts, dtype=np.int64)
    if counts.sum() > T:
        raise ValueError("counts exceed T")
    a, _ = activations(rng, T, K)
    w = weights(rng, (E, N, K), w_sigma)
    return GroupedInputs(name, E, T, N, K, counts, offsets_from_counts(counts),
                         a, w, out_dtype)


# ---- the five measured workloads ------------------------------------------

def config_tiny(seed: int = 0) -> GemmInputs:
    """Tiny GEMM: M=128 tokens, K=512, N=256; 1% outlier channels x50;
    FP32 output."""
    return gemm_inputs(128, 256, 512, seed, "f32", 0.01, 50.0, name="tiny_128x256x512")


def config_quant(seed: int = 0, M: int = 4096, K: int = 7168):
    """Activation quantizer workload: 4096 tokens x 7168 channels, 0.1%
    outlier channels x100.  Returns (bits [M][K], outlier channels)."""
    rng = np.random.default_rng(seed)
    return activations(rng, M, K, 0.001, 100.0)


def config_dense(seed: int = 0) -> GemmInputs:
    """Prefill-shaped dense GEMM: M=4096, N=7168, K=7168, BF16 output."""
    return gemm_inputs(4096, 7168, 7168, seed, "bf16", name="dense_4096x7168x7168")


def config_decode(seed: int = 0) -> GemmInputs:
    """Decode-shaped small-M GEMM: M=256, N=2048, K=7168, BF16 output."""
    return gemm_inputs(256, 2048, 7168, seed, "bf16", name="decode_256x2048x7168")


def config_grouped(seed: int = 0) -> GroupedInputs:
    """Grouped MoE GEMM: 32 experts, 8192 tokens, Zipf(1.1) routing capped at
    1024 per expert, K=7168, N=4096 per expert, BF16 output."""
    return grouped_inputs(32, 8192, 4096, 7168, seed, cap=1024,
                          name="grouped_e32_t8192_n4096_k7168")
