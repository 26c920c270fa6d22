// 1x128 activation and 128x128 weight quantization to OCP E4M3 (gfx950).
//
// Method: page "dssusan.co.kr qna 93378", Figure 7 (a): one scale per token
// per 128 channels for activations and per 128x128 block for weights, with
// the scale following each small group's own maximum.  Page "why-be.co.kr
// as_center 36949", passage on the quantization round trip: the activation
// quantizer reads 128 BF16 values per group and writes FP8 back, so it is a
// pure HBM stream (about 3 bytes moved per element) and is built as one.
//
// Activation kernel layout: a 16-lane DPP row owns one group; each lane
// loads 8 bf16 (16 bytes), so a wave64 streams four groups = 1 KiB per load
// instruction and stores 512 contiguous E4M3 bytes.  The group maximum is a
// 4-step DPP reduction inside the row; the scale is stored by the row's
// first lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8blk {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQuantThreads = 256;

// Fast path: K % 128 == 0, x and q 16-byte aligned.  The tensor is a flat
// sequence of 128-element groups.  Eight lanes own one group, 16 elements
// (32 bytes) each: unit c (16 elements) belongs to group c / 8, whose scale
// index is that group index (scales are [M][K/128]).  A wave streams 2 KiB
// of bf16 per unit step and stores 1 KiB of E4M3.  When every group of the
// wave has amax >= 2^-60 (the normal case) a branch-free path runs: scale
// by constant division, reciprocal by one IEEE divide per lane, and the
// reciprocal + FMA quotient per element; otherwise the wave takes the
// general per-group selection (all-zero, tiny or ordinary groups).
// One unit per thread: more, shorter workgroups keep more of the stream in
// flight than two or four units per thread (measured ~5% faster on
// 4096 x 7168).
// kPow2: power-of-two scales (scale_pow2); the reciprocal is then exact and
// the fast path serves every group with amax > 0.
constexpr int kFlatUnroll = 1;  // 16-element units per thread per block

template <bool kPow2>
__global__ __launch_bounds__(kQuantThreads) void quant_act_flat_kernel(
    const u32x4 *__restrict__ x, u32x4 *__restrict__ q, float *__restrict__ scales,
    int64_t n_units) {
    const int64_t base = (int64_t)blockIdx.x * (kQuantThreads * kFlatUnroll) + threadIdx.x;
    u32x4 v[kFlatUnroll][2];
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
        const int64_t c = base + (int64_t)u * kQuantThreads;
        if (c < n_units) {
            v[u][0] = __builtin_nontemporal_load(x + 2 * c);
            v[u][1] = __builtin_nontemporal_load(x + 2 * c + 1);
        } else {
            v[u][0] = u32x4{0, 0, 0, 0};
            v[u][1] = u32x4{0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) {
        const int64_t c = base + (int64_t)u * kQuantThreads;
        const bool in = c < n_units;
        float f[16];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 t = v[u][h];
            f[8 * h + 0] = bf16_lo(t.x); f[8 * h + 1] = bf16_hi(t.x);
            f[8 * h + 2] = bf16_lo(t.y); f[8 * h + 3] = bf16_hi(t.y);
            f[8 * h + 4] = bf16_lo(t.z); f[8 * h + 5] = bf16_hi(t.z);
            f[8 * h + 6] = bf16_lo(t.w); f[8 * h + 7] = bf16_hi(t.w);
        }
        float m = fabsf(f[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, fabsf(f[i]));
        // n_units is a multiple of 8 and groups start at multiples of 8, so
        // an 8-lane group is entirely in or out of range.
        const float amax = row8_max(m);
        float y[16];
        float s;
        if (__all(!in || (kPow2 ? amax > 0.0f : amax >= 0x1p-60f))) {
            s = kPow2 ? scale_pow2(amax) : scale_fast(amax);
            const float r = 1.0f / s;
#pragma unroll
            for (int i = 0; i < 16; ++i) y[i] = quot_fast(f[i], s, r);
        } else {
            const QuotientCtx qc(amax, kPow2);
            s = qc.s;
#pragma unroll
            for (int i = 0; i < 16; ++i) y[i] = qc(f[i]);
        }
        u32x4 o;
        uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
        w0 = cvt_pk_e4m3<false>(y[0], y[1], w0);
        w0 = cvt_pk_e4m3<true>(y[2], y[3], w0);
        w1 = cvt_pk_e4m3<false>(y[4], y[5], w1);
        w1 = cvt_pk_e4m3<true>(y[6], y[7], w1);
        w2 = cvt_pk_e4m3<false>(y[8], y[9], w2);
        w2 = cvt_pk_e4m3<true>(y[10], y[11], w2);
        w3 = cvt_pk_e4m3<false>(y[12], y[13], w3);
        w3 = cvt_pk_e4m3<true>(y[14], y[15], w3);
        o.x = w0;
        o.y = w1;
        o.z = w2;
        o.w = w3;
        if (in) {
            // default cache policy: the GEMM that follows reads q back
            q[c] = o;
            if ((threadIdx.x & 7) == 0) scales[c >> 3] = s;
        }
    }
}

// General path: any K and alignment.  One DPP row per group (m, g); lane j
// covers channels [128 g + 8 j, +8) clipped to K.  kVec: K % 8 == 0 with x
// 16-byte and q 8-byte aligned, so every in-range chunk is a full vector.
template <bool kVec, bool kPow2>
__global__ __launch_bounds__(kQuantThreads) void quant_act_general_kernel(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q, float *__restrict__ scales,
    int64_t M, int64_t K, int64_t G) {
    const int64_t grp = (int64_t)blockIdx.x * (kQuantThreads / 16) + (threadIdx.x >> 4);
    const int j = threadIdx.x & 15;
    const bool grp_ok = grp < M * G;
    const int64_t m = grp_ok ? grp / G : 0;
    const int64_t g = grp_ok ? grp - m * G : 0;
    const int64_t k0 = g * kGroup + 8 * j;
    const int64_t off = m * K + k0;
    int n = 0;
    if (grp_ok && k0 < K) n = (K - k0) < 8 ? (int)(K - k0) : 8;
    float f[8];
    if (kVec && n == 8) {
        unpack8(*reinterpret_cast<const uint4 *>(x + off), f);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            f[i] = i < n ? __uint_as_float((uint32_t)x[off + i] << 16) : 0.0f;
    }
    const float amax = row16_max(absmax8(f));
    const QuotientCtx qc(amax, kPow2);
    const uint2 out = quant8(f, qc);
    if (kVec && n == 8) {
        *reinterpret_cast<uint2 *>(q + off) = out;
    } else {
        const uint8_t *b = reinterpret_cast<const uint8_t *>(&out);
        for (int i = 0; i < n; ++i) q[off + i] = b[i];
    }
    if (grp_ok && j == 0) scales[grp] = qc.s;
}

// 128x128 weight blocks: one workgroup (4 waves) per block (nb, g), with the
// flat block index nb * G + g in blockIdx.x.  Thread t
// covers chunk c = t + 256 i (i < 8): block row c / 16, channels 8 (c % 16)
// .. +8.  Block maximum: per-thread, per-wave DPP/shuffle, then across the
// four waves through LDS.  Offline work (weights are quantized once).
template <bool kVec, bool kPow2>
__global__ __launch_bounds__(kQuantThreads) void quant_weight_kernel(
    const uint16_t *__restrict__ w, uint8_t *__restrict__ q, float *__restrict__ scales,
    int64_t N, int64_t K, int64_t G) {
    __shared__ float wave_amax[kQuantThreads / 64];
    const int64_t nb = blockIdx.x / G, g = blockIdx.x - (blockIdx.x / G) * G;
    const int64_t n0 = nb * kGroup, k0 = g * kGroup;
    float f[8][8];
    int cnt[8];
    int64_t off[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + kQuantThreads * i;
        const int64_t n = n0 + (c >> 4);
        const int64_t k = k0 + 8 * (c & 15);
        int cn = 0;
        if (n < N && k < K) cn = (K - k) < 8 ? (int)(K - k) : 8;
        cnt[i] = cn;
        off[i] = n * K + k;
        if (kVec && cn == 8) {
            unpack8(*reinterpret_cast<const uint4 *>(w + off[i]), f[i]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f[i][e] = e < cn ? __uint_as_float((uint32_t)w[off[i] + e] << 16) : 0.0f;
        }
        amax = fmaxf(amax, absmax8(f[i]));
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));
    const QuotientCtx qc(amax, kPow2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint2 out = quant8(f[i], qc);
        if (kVec && cnt[i] == 8) {
            *reinterpret_cast<uint2 *>(q + off[i]) = out;
        } else {
            const uint8_t *b = reinterpret_cast<const uint8_t *>(&out);
            for (int e = 0; e < cnt[i]; ++e) q[off[i] + e] = b[e];
        }
    }
    if (threadIdx.x == 0) scales[nb * G + g] = qc.s;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <bool kPow2>
hipError_t quant_act(const void *x, int64_t M, int64_t K, void *q, float *scales,
                     hipStream_t stream) {
    const int64_t G = (K + kGroup - 1) / kGroup;
    const bool vec = (K % 8 == 0) && aligned(x, 16) && aligned(q, 8);
    if (K % kGroup == 0 && aligned(x, 16) && aligned(q, 16)) {
        const int64_t n_units = M * K / 16;
        const int64_t per_block = (int64_t)kQuantThreads * kFlatUnroll;
        const int64_t blocks = (n_units + per_block - 1) / per_block;
        hipLaunchKernelGGL(quant_act_flat_kernel<kPow2>, dim3((unsigned)blocks),
                           dim3(kQuantThreads), 0, stream, static_cast<const u32x4 *>(x),
                           static_cast<u32x4 *>(q), scales, n_units);
    } else {
        const int64_t groups = M * G;
        const int64_t per_block = kQuantThreads / 16;
        const int64_t blocks = (groups + per_block - 1) / per_block;
        if (vec)
            hipLaunchKernelGGL((quant_act_general_kernel<true, kPow2>), dim3((unsigned)blocks),
                               dim3(kQuantThreads), 0, stream, static_cast<const uint16_t *>(x),
                               static_cast<uint8_t *>(q), scales, M, K, G);
        else
            hipLaunchKernelGGL((quant_act_general_kernel<false, kPow2>), dim3((unsigned)blocks),
                               dim3(kQuantThreads), 0, stream, static_cast<const uint16_t *>(x),
                               static_cast<uint8_t *>(q), scales, M, K, G);
    }
    return hipGetLastError();
}

template <bool kPow2>
hipError_t quant_weight(const void *w, int64_t N, int64_t K, void *q, float *scales,
                        hipStream_t stream) {
    const int64_t G = (K + kGroup - 1) / kGroup;
    const int64_t NB = (N + kGroup - 1) / kGroup;
    const bool vec = (K % 8 == 0) && aligned(w, 16) && aligned(q, 8);
    const dim3 grid((unsigned)(NB * G));
    if (vec)
        hipLaunchKernelGGL((quant_weight_kernel<true, kPow2>), grid, dim3(kQuantThreads), 0,
                           stream, static_cast<const uint16_t *>(w), static_cast<uint8_t *>(q),
                           scales, N, K, G);
    else
        hipLaunchKernelGGL((quant_weight_kernel<false, kPow2>), grid, dim3(kQuantThreads), 0,
                           stream, static_cast<const uint16_t *>(w), static_cast<uint8_t *>(q),
                           scales, N, K, G);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_act_1x128(const void *x, int64_t M, int64_t K, void *q, float *scales,
                                  bool pow2, hipStream_t stream) {
    return pow2 ? quant_act<true>(x, M, K, q, scales, stream)
                : quant_act<false>(x, M, K, q, scales, stream);
}

hipError_t launch_quant_weight_128x128(const void *w, int64_t N, int64_t K, void *q,
                                       float *scales, bool pow2, hipStream_t stream) {
    return pow2 ? quant_weight<true>(w, N, K, q, scales, stream)
                : quant_weight<false>(w, N, K, q, scales, stream);
}

}  // namespace fp8blk
