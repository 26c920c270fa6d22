// Device helpers shared by the fp8blk kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

// Largest finite OCP E4M3FN magnitude; the per-group scale is amax / 448.
constexpr float kE4M3Max = 448.0f;
constexpr int kGroup = 128;

// bf16 -> fp32 is exact: the bf16 bits are the top half of the binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Max over the 16 lanes of one DPP row: two quad permutations, then the
// half-row mirror and the row mirror; every lane of the row ends with it.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
    return v;
}

// Max over a whole wave64 (used by the offline weight quantizer).
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Power-of-two scale (the block-scaled-MFMA variant): the smallest 2^E with
// 448 * 2^E >= amax, and at least 2^-126 (so every scale is a normal fp32
// whose exponent field is its E8M0 code).  With amax = (1 + f) 2^(e - 127)
// (e the exponent field) and 448 = 1.75 * 2^8, 448 * 2^E >= amax holds from
// E = e - 135 on when 1 + f <= 1.75, else from e - 134.  Zero or subnormal
// amax gives the floor.
__device__ __forceinline__ float scale_pow2(float amax) {
    const uint32_t b = __float_as_uint(amax);
    const int e = (int)(b >> 23);  // amax >= 0
    int E = e - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    E = (e == 0 || E < -126) ? -126 : E;
    return __uint_as_float((uint32_t)(E + 127) << 23);
}

// Per-group quotient context.  The quantized value is E4M3_RNE(fl32(x / s)).
// For amax >= 2^-60 the correctly rounded quotient is obtained from the
// correctly rounded reciprocal r = fl32(1/s) with one FMA correction
// (Markstein's method: q0 = |x| r, e = |x| - s q0 exactly by FMA,
// q = q0 + e r); where that differs from fl32(|x|/s) both values are below
// 2^-12 and encode to the same signed zero.  Smaller amax (subnormal or tiny
// s) falls back to the IEEE divide.  The sign is taken from x so that -0
// and tiny negatives keep it.
// An all-zero group (amax = 0, so s = 0) encodes every element as +0.
// With power-of-two scales (pow2) r = 1/s is exact, so the FMA quotient is
// the correctly rounded one for every amax; an all-zero group keeps the
// floor scale 2^-126 and also encodes as +0.
struct QuotientCtx {
    float s, r;
    bool fast, zero;
    __device__ __forceinline__ explicit QuotientCtx(float amax, bool pow2 = false) {
        if (pow2) {
            s = scale_pow2(amax);
            zero = !(amax > 0.0f);
            fast = true;
            r = 1.0f / s;
        } else {
            s = amax / kE4M3Max;
            zero = !(s > 0.0f);
            fast = amax >= 0x1p-60f;
            r = fast ? 1.0f / s : 0.0f;
        }
    }
    __device__ __forceinline__ float operator()(float x) const {
        float y;
        if (zero) {
            y = 0.0f;
        } else if (fast) {
            float a = fabsf(x);
            float q0 = a * r;
            float e = __builtin_fmaf(-q0, s, a);
            y = __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
        } else {
            y = x / s;
        }
        // |y| <= ~448.9 for every bf16 group, which rounds to 448; the clamp
        // keeps the hardware conversion from treating it as an overflow.
        return __builtin_amdgcn_fmed3f(y, -kE4M3Max, kE4M3Max);
    }
};

// fl32(amax / 448) for amax >= 2^-60 by division by a constant: with
// R = fl32(1/448), q0 = amax R is within an ulp, the residual amax - 448 q0
// is exact by FMA, and q0 + residual R rounds to the correctly rounded
// quotient (Markstein's method; equal to the IEEE divide for every bf16
// amax in that range).
__device__ __forceinline__ float scale_fast(float amax) {
    constexpr float R = 1.0f / kE4M3Max;
    const float q0 = amax * R;
    const float e = __builtin_fmaf(-q0, kE4M3Max, amax);
    return __builtin_fmaf(e, R, q0);
}

// Quotient of the fast path (amax >= 2^-60, see QuotientCtx), clamped.
__device__ __forceinline__ float quot_fast(float x, float s, float r) {
    const float a = fabsf(x);
    const float q0 = a * r;
    const float e = __builtin_fmaf(-q0, s, a);
    const float y = __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
    return __builtin_amdgcn_fmed3f(y, -kE4M3Max, kE4M3Max);
}

// Two fp32 -> two OCP E4M3 bytes (gfx950 v_cvt_pk_fp8_f32, round to nearest
// even) packed into the low (kHi = false) or high 16 bits of `old`.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// Quantize 8 fp32 values of one group with a prepared context into 8 bytes.
__device__ __forceinline__ uint2 quant8(const float (&f)[8], const QuotientCtx &qc) {
    uint32_t lo = 0, hi = 0;
    lo = cvt_pk_e4m3<false>(qc(f[0]), qc(f[1]), lo);
    lo = cvt_pk_e4m3<true>(qc(f[2]), qc(f[3]), lo);
    hi = cvt_pk_e4m3<false>(qc(f[4]), qc(f[5]), hi);
    hi = cvt_pk_e4m3<true>(qc(f[6]), qc(f[7]), hi);
    return make_uint2(lo, hi);
}

__device__ __forceinline__ void unpack8(const uint4 &v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ float absmax8(const float (&f)[8]) {
    float m = fabsf(f[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    return m;
}

}  // namespace fp8blk
