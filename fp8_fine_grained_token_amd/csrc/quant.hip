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

// Fast path: K % 128 == 0, x 16-byte and q 8-byte aligned.  The tensor is a
// flat sequence of 128-element groups (the scale index of a group is its
// index: scales are [M][K/128]).  A wave takes 4 kFlatLoads consecutive
// groups in kFlatLoads load instructions: in load h, lane l reads elements
// 512 h + 8 l .. + 8 of the wave's range, so each instruction reads 1 KiB
// contiguously, and the 16 lanes of a DPP row hold one group (group 4 h +
// l / 16 of the wave).  The group maximum is a 16-lane DPP reduction; each
// lane stores 8 bytes, 512 contiguous bytes per store instruction.  When
// every group of the wave has amax >= 2^-60 (the normal case) a branch-free
// path runs: scale by constant division, reciprocal by one IEEE divide per
// lane, and the reciprocal + FMA quotient per element; otherwise the wave
// takes the general per-group selection (all-zero, tiny or ordinary
// groups).
// kPow2: power-of-two scales (scale_pow2); the reciprocal is then exact and
// the fast path serves every group with amax > 0.
constexpr int kFlatLoads = 2;    // 16-byte loads per lane; 1 or 4 measured slower
constexpr int kFlatThreads = 64;  // one wave per workgroup: ~1% faster than 256, 3-5% than 512-1024

template <bool kPow2>
__global__ __launch_bounds__(kFlatThreads) void quant_act_flat_kernel(
    const u32x4 *__restrict__ x, uint2 *__restrict__ q, float *__restrict__ scales,
    int64_t n_groups) {
    const int lane = threadIdx.x & 63;
    const int64_t g0 = ((int64_t)blockIdx.x * (kFlatThreads / 64) + (threadIdx.x >> 6)) * (4 * kFlatLoads);
    int64_t g[kFlatLoads], chunk[kFlatLoads];
    bool in[kFlatLoads];
    u32x4 v[kFlatLoads];
#pragma unroll
    for (int h = 0; h < kFlatLoads; ++h) {
        g[h] = g0 + 4 * h + (lane >> 4);
        chunk[h] = g0 * 16 + 64 * h + lane;  // 8-element chunk lane % 16 of group g[h]
        in[h] = g[h] < n_groups;             // the 16 lanes of a group agree
        v[h] = in[h] ? __builtin_nontemporal_load(x + chunk[h]) : u32x4{0, 0, 0, 0};
    }
    float f[kFlatLoads][8], amax[kFlatLoads];
#pragma unroll
    for (int h = 0; h < kFlatLoads; ++h) {
        unpack8(make_uint4(v[h].x, v[h].y, v[h].z, v[h].w), f[h]);
        amax[h] = row16_max(absmax8(f[h]));
    }
    auto fast_ok = [&](int h) {
        return !in[h] || (kPow2 ? amax[h] > 0.0f : amax[h] >= 0x1p-60f);
    };
    float y[kFlatLoads][8], s[kFlatLoads];
    bool all_fast = true;
#pragma unroll
    for (int h = 0; h < kFlatLoads; ++h) all_fast = all_fast && fast_ok(h);
    if (__all(all_fast)) {
#pragma unroll
        for (int h = 0; h < kFlatLoads; ++h) {
            s[h] = kPow2 ? scale_pow2(amax[h]) : scale_fast(amax[h]);
            const float r = 1.0f / s[h];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[h][i] = quot_fast(f[h][i], s[h], r);
        }
    } else {
#pragma unroll
        for (int h = 0; h < kFlatLoads; ++h) {
            const QuotientCtx qc(amax[h], kPow2);
            s[h] = qc.s;
#pragma unroll
            for (int i = 0; i < 8; ++i) y[h][i] = qc(f[h][i]);
        }
    }
#pragma unroll
    for (int h = 0; h < kFlatLoads; ++h) {
        uint32_t lo = 0, hi = 0;
        lo = cvt_pk_e4m3<false>(y[h][0], y[h][1], lo);
        lo = cvt_pk_e4m3<true>(y[h][2], y[h][3], lo);
        hi = cvt_pk_e4m3<false>(y[h][4], y[h][5], hi);
        hi = cvt_pk_e4m3<true>(y[h][6], y[h][7], hi);
        if (in[h]) {
            // default cache policy: the GEMM that follows reads q back
            q[chunk[h]] = make_uint2(lo, hi);
            if ((lane & 15) == 0) scales[g[h]] = s[h];
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

// 128x1 tiles written transposed (the Wgrad operands: 128 tokens of one
// channel per group, token axis contiguous in the output).  A tile is 128
// rows x 128 columns of x [M][K] (256 contiguous bytes of each row).  Its
// rows go to LDS as bf16; four lanes per column then take 32 rows each,
// reduce the column's amax over its 128 rows with two xor shuffles and
// quantize with the 1x128 kernels' quotient; the E4M3 bytes go to a second
// LDS tile laid out as the output, q_t[k][m0 .. +128), and leave it in
// whole 128-byte rows.  Rows past M load as zero, which leaves every amax
// unchanged.
//
// Memory access (kVec: K % 8 == 0 and x 16-byte aligned; kVecOut: M % 16 ==
// 0 and q_t 16-byte aligned): load instruction v of thread t moves 16-byte
// chunk (512 v + t) of the tile in row-major order, so a wave reads four
// whole 256-byte row pieces per instruction; store instruction v writes
// 16-byte piece (512 v + t) of the output tile, eight whole 128-byte rows
// per wave.  Without kVec the tile is loaded element by element, without
// kVecOut stored byte by byte.
//
// In the bf16 tile, element (r, c) sits at column c ^ 16 ((r / 32) % 4): the
// four lanes of a column read rows 32 apart, which the 66-word row pitch
// maps to one bank group; the swizzle gives each of them its own.
//
// Workgroups are persistent: each takes tiles blockIdx.x, + gridDim.x, ...
// With kVec the next tile's chunks are fetched into registers as soon as
// the current tile is in LDS, so they are in flight while it is quantized
// and stored.
constexpr int kTRows = 128, kTCols = 128;
constexpr int kTThreads = 4 * kTCols;  // four lanes per column
constexpr int kTPitch = kTCols + 4;    // bf16 per LDS row: 8-byte aligned rows
constexpr int kTOutPitch = 9;          // 16-byte pieces per output row in LDS (8 + 1 pad)
constexpr int kTBlocksPerCU = 2;       // resident workgroups per CU (VGPR-bound)
constexpr int kTCUs = 256;
__device__ __forceinline__ int tswz(int r) { return 16 * ((r >> 5) & 3); }

template <bool kVec, bool kVecOut, bool kPow2>
__global__ __launch_bounds__(kTThreads) void quant_act_128x1_t_kernel(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q_t, float *__restrict__ scales_t,
    int64_t M, int64_t K, int64_t GM, int64_t KT) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[kTRows][kTPitch];
    __shared__ uint4 qs[kTCols][kTOutPitch];
    const int t = threadIdx.x;
    const int64_t ntiles = GM * KT;
    uint4 d[4];
    // chunk 512 v + t: tile row (512 v + t) / 16, columns 8 ((512 v + t) % 16) .. + 8
    auto fetch = [&](int64_t id) {
        const int64_t m0 = (id / KT) * kTRows, k0 = (id % KT) * kTCols;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int q = kTThreads * v + t;
            const int64_t m = m0 + (q >> 4), k = k0 + 8 * (q & 15);  // all 8 in or all out
            d[v] = (m < M && k < K) ? *reinterpret_cast<const uint4 *>(x + m * K + k)
                                    : make_uint4(0, 0, 0, 0);
        }
    };
    if (kVec && (int64_t)blockIdx.x < ntiles) fetch(blockIdx.x);
    for (int64_t id = blockIdx.x; id < ntiles; id += gridDim.x) {
        const int64_t mb = id / KT;
        const int64_t k0 = (id % KT) * kTCols, m0 = mb * kTRows;
        __syncthreads();  // every lane is done with the previous tile's LDS
        if (kVec) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int q = kTThreads * v + t, r = q >> 4;
                uint2 *row = reinterpret_cast<uint2 *>(&tile[r][(8 * (q & 15)) ^ tswz(r)]);
                row[0] = make_uint2(d[v].x, d[v].y);
                row[1] = make_uint2(d[v].z, d[v].w);
            }
        } else {
            const int lr = t >> 2, lc0 = (t & 3) * 32;
            const int64_t m = m0 + lr;
            for (int c = 0; c < 32; ++c) {
                const int64_t k = k0 + lc0 + c;
                tile[lr][(lc0 + c) ^ tswz(lr)] = (m < M && k < K) ? x[m * K + k] : (uint16_t)0;
            }
        }
        __syncthreads();
        if (kVec && id + gridDim.x < ntiles) fetch(id + gridDim.x);

        const int c = t >> 2, part = t & 3;
        float f[32];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            f[i] = __uint_as_float((uint32_t)tile[32 * part + i][c ^ (16 * part)] << 16);
            amax = fmaxf(amax, fabsf(f[i]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        // As in the 1x128 kernel: when every column of the wave has amax >=
        // 2^-60 (with power-of-two scales: amax > 0), one branch-free path
        // (constant-division or power-of-two scale, reciprocal + FMA
        // quotients) serves the wave; otherwise the per-group selection.
        float y[32], s;
        if (__all(kPow2 ? amax > 0.0f : amax >= 0x1p-60f)) {
            s = kPow2 ? scale_pow2(amax) : scale_fast(amax);
            const float r = 1.0f / s;
#pragma unroll
            for (int i = 0; i < 32; ++i) y[i] = quot_fast(f[i], s, r);
        } else {
            const QuotientCtx qc(amax, kPow2);
            s = qc.s;
#pragma unroll
            for (int i = 0; i < 32; ++i) y[i] = qc(f[i]);
        }
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t o = 0;
            o = cvt_pk_e4m3<false>(y[4 * j], y[4 * j + 1], o);
            o = cvt_pk_e4m3<true>(y[4 * j + 2], y[4 * j + 3], o);
            w[j] = o;
        }
        qs[c][2 * part] = make_uint4(w[0], w[1], w[2], w[3]);
        qs[c][2 * part + 1] = make_uint4(w[4], w[5], w[6], w[7]);
        if (part == 0 && k0 + c < K) scales_t[(k0 + c) * GM + mb] = s;
        __syncthreads();
        // piece 512 v + t of the output tile: row (512 v + t) / 8, tokens
        // 16 ((512 v + t) % 8) .. + 16
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int q = kTThreads * v + t;
            const int kk = q >> 3, pc = q & 7;
            const int64_t k = k0 + kk, m = m0 + 16 * pc;
            if (k < K && m < M) {
                const uint4 o = qs[kk][pc];
                uint8_t *dst = q_t + k * M + m;
                if (kVecOut) {
                    *reinterpret_cast<uint4 *>(dst) = o;  // M % 16 == 0: all 16 in range
                } else {
                    const uint8_t *b = reinterpret_cast<const uint8_t *>(&o);
                    const int cnt = M - m < 16 ? (int)(M - m) : 16;
                    for (int i = 0; i < cnt; ++i) dst[i] = b[i];
                }
            }
        }
    }
}

// Transpose of E4M3 weights in 128 x 128 tiles through LDS: q [N][K] ->
// q_t [K][N], and the tile's block scale s[nb][kb] -> s_t[kb][nb] (a block's
// scale serves whichever way the block is read).  Offline work, once per
// weight update.  This is the byte-wise path for shapes and pointers the
// vector kernel below does not take.
__global__ __launch_bounds__(kQuantThreads) void transpose_weight_scalar_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ s, uint8_t *__restrict__ q_t,
    float *__restrict__ s_t, int64_t N, int64_t K, int64_t NB, int64_t G) {
    __shared__ uint8_t tile[128][128 + 16];
    const int64_t nb = (int64_t)blockIdx.x / G, kb = (int64_t)blockIdx.x % G;
    const int64_t n0 = nb * 128, k0 = kb * 128;
    const int t = threadIdx.x;
    const int r = t >> 1, h = (t & 1) * 64;
    {  // tile row r = q row n0 + r, bytes k0 + h .. + 64
        const int64_t n = n0 + r;
        for (int j = 0; j < 64; ++j) {
            const int64_t k = k0 + h + j;
            tile[r][h + j] = (n < N && k < K) ? q[n * K + k] : 0;
        }
    }
    __syncthreads();
    {  // q_t row k0 + r, bytes n0 + h .. + 64, gathered from tile column r
        const int64_t k = k0 + r;
        if (k < K) {
            for (int j = 0; j < 64; ++j) {
                const int64_t n = n0 + h + j;
                if (n < N) q_t[k * N + n] = tile[h + j][r];
            }
        }
    }
    if (t == 0) s_t[kb * NB + nb] = s[nb * G + kb];
}

// Vector path (K % 16 == 0 and N % 16 == 0, q and q_t 16-byte aligned).  A
// workgroup of 256 threads moves one 128 x 128-byte tile:
//   - load v of thread t brings 16-byte chunk 256 v + t of the tile in
//     row-major order (a wave reads eight whole 128-byte rows per
//     instruction) into an LDS tile of 32-bit words, where word (r, c) sits
//     in row r ^ ((r / 16) % 2) at column c ^ 8 ((r / 32) % 4);
//   - thread t then reads the 16 x 4-byte block of rows 16 (t % 8) .. + 16
//     and byte columns 4 (t / 8) .. + 4 as 16 words (the row and column
//     swizzles put the wave's 64 reads on 64 different banks) and
//     transposes it in registers with byte permutes, four 4 x 4 blocks of
//     eight v_perm_b32 each;
//   - it writes the four transposed rows, 16 bytes each, to q_t rows k0 + 4
//     (t / 8) .. + 4 at bytes n0 + 16 (t % 8): a wave's store instruction
//     fills eight whole 128-byte rows.
__device__ __forceinline__ int wt_row(int r) { return r ^ ((r >> 4) & 1); }
__device__ __forceinline__ int wt_col(int r, int c) { return c ^ (8 * ((r >> 5) & 3)); }

__global__ __launch_bounds__(kQuantThreads) void transpose_weight_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ s, uint8_t *__restrict__ q_t,
    float *__restrict__ s_t, int64_t N, int64_t K, int64_t NB, int64_t G) {
    __shared__ __attribute__((aligned(16))) uint32_t tile[128][32];
    const int64_t nb = (int64_t)blockIdx.x / G, kb = (int64_t)blockIdx.x % G;
    const int64_t n0 = nb * 128, k0 = kb * 128;
    const int t = threadIdx.x;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int c = kQuantThreads * v + t, r = c >> 3;
        const int64_t n = n0 + r, k = k0 + 16 * (c & 7);  // all 16 bytes in or all out
        const uint4 d = (n < N && k < K) ? *reinterpret_cast<const uint4 *>(q + n * K + k)
                                         : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(&tile[wt_row(r)][wt_col(r, 4 * (c & 7))]) = d;
    }
    __syncthreads();
    const int g = t & 7, kg = t >> 3;
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = tile[wt_row(16 * g + i)][wt_col(16 * g + i, kg)];
    // out[j][h]: bytes (rows 16 g + 4 h .. + 4, byte column 4 kg + j).
    // v_perm_b32 picks result byte i from {src0 (bytes 4-7), src1 (bytes
    // 0-3)} by selector byte i: first interleave two rows' bytes pairwise,
    // then pairs of pairs.
    uint32_t out[4][4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t lo01 = __builtin_amdgcn_perm(w[4 * h + 1], w[4 * h], 0x05010400u);
        const uint32_t hi01 = __builtin_amdgcn_perm(w[4 * h + 1], w[4 * h], 0x07030602u);
        const uint32_t lo23 = __builtin_amdgcn_perm(w[4 * h + 3], w[4 * h + 2], 0x05010400u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w[4 * h + 3], w[4 * h + 2], 0x07030602u);
        out[0][h] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
        out[1][h] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
        out[2][h] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
        out[3][h] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
    }
    const int64_t n = n0 + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t k = k0 + 4 * kg + j;
        if (k < K && n < N)  // N % 16 == 0: all 16 bytes in range
            *reinterpret_cast<uint4 *>(q_t + k * N + n) =
                make_uint4(out[j][0], out[j][1], out[j][2], out[j][3]);
    }
    if (t == 0) s_t[kb * NB + nb] = s[nb * G + kb];
}

template <bool kPow2>
hipError_t quant_act(const void *x, int64_t M, int64_t K, void *q, float *scales,
                     hipStream_t stream) {
    const int64_t G = (K + kGroup - 1) / kGroup;
    const bool vec = (K % 8 == 0) && aligned(x, 16) && aligned(q, 8);
    if (K % kGroup == 0 && aligned(x, 16) && aligned(q, 8)) {
        const int64_t n_groups = M * K / kGroup;
        const int64_t per_block = (int64_t)(kFlatThreads / 64) * 4 * kFlatLoads;
        const int64_t blocks = (n_groups + per_block - 1) / per_block;
        hipLaunchKernelGGL(quant_act_flat_kernel<kPow2>, dim3((unsigned)blocks),
                           dim3(kFlatThreads), 0, stream, static_cast<const u32x4 *>(x),
                           static_cast<uint2 *>(q), scales, n_groups);
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

namespace {

template <bool kPow2>
hipError_t quant_act_128x1_t(const void *x, int64_t M, int64_t K, void *q_t, float *scales_t,
                             hipStream_t stream) {
    const int64_t GM = (M + kTRows - 1) / kTRows;
    const int64_t KT = (K + kTCols - 1) / kTCols;
    const int64_t ntiles = GM * KT;
    const dim3 grid((unsigned)(ntiles < kTCUs * kTBlocksPerCU ? ntiles : kTCUs * kTBlocksPerCU));
    const bool vec = (K % 8 == 0) && aligned(x, 16);
    const bool vec_out = (M % 16 == 0) && aligned(q_t, 16);
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    uint8_t *qq = static_cast<uint8_t *>(q_t);
    if (vec && vec_out)
        hipLaunchKernelGGL((quant_act_128x1_t_kernel<true, true, kPow2>), grid, dim3(kTThreads),
                           0, stream, xx, qq, scales_t, M, K, GM, KT);
    else if (vec)
        hipLaunchKernelGGL((quant_act_128x1_t_kernel<true, false, kPow2>), grid,
                           dim3(kTThreads), 0, stream, xx, qq, scales_t, M, K, GM, KT);
    else if (vec_out)
        hipLaunchKernelGGL((quant_act_128x1_t_kernel<false, true, kPow2>), grid,
                           dim3(kTThreads), 0, stream, xx, qq, scales_t, M, K, GM, KT);
    else
        hipLaunchKernelGGL((quant_act_128x1_t_kernel<false, false, kPow2>), grid,
                           dim3(kTThreads), 0, stream, xx, qq, scales_t, M, K, GM, KT);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_act_128x1_t(const void *x, int64_t M, int64_t K, void *q_t,
                                    float *scales_t, bool pow2, hipStream_t stream) {
    return pow2 ? quant_act_128x1_t<true>(x, M, K, q_t, scales_t, stream)
                : quant_act_128x1_t<false>(x, M, K, q_t, scales_t, stream);
}

hipError_t launch_transpose_weight(const void *q, const float *s, int64_t N, int64_t K,
                                   void *q_t, float *s_t, hipStream_t stream) {
    const int64_t NB = (N + 127) / 128, G = (K + 127) / 128;
    const dim3 grid((unsigned)(NB * G));
    const bool vec = K % 16 == 0 && N % 16 == 0 && aligned(q, 16) && aligned(q_t, 16);
    const uint8_t *qq = static_cast<const uint8_t *>(q);
    uint8_t *qt = static_cast<uint8_t *>(q_t);
    if (vec)
        hipLaunchKernelGGL(transpose_weight_kernel, grid, dim3(kQuantThreads), 0, stream, qq, s,
                           qt, s_t, N, K, NB, G);
    else
        hipLaunchKernelGGL(transpose_weight_scalar_kernel, grid, dim3(kQuantThreads), 0, stream,
                           qq, s, qt, s_t, N, K, NB, G);
    return hipGetLastError();
}

hipError_t launch_quant_weight_128x128(const void *w, int64_t N, int64_t K, void *q,
                                       float *scales, bool pow2, hipStream_t stream) {
    return pow2 ? quant_weight<true>(w, N, K, q, scales, stream)
                : quant_weight<false>(w, N, K, q, scales, stream);
}

}  // namespace fp8blk
