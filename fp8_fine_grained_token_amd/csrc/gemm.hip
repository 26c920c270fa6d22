// Block-scaled FP8 GEMM and its grouped (MoE) variant for gfx950.
//
// What is computed (page "dssusan.co.kr qna 93378", passages on per-group
// scaling along the inner dimension K and on FP8-in / BF16-or-FP32-out GEMMs;
// page "kailasan.com recruit 147436", Figure 7 (b): partial sums are scaled
// and added into FP32 registers at a fixed K interval):
//   C[m][n] = sum_kb sa[m][kb] * sw[n/128][kb] * P_kb[m][n],
//   P_kb[m][n] = sum_{k in [128 kb, 128 kb + 128)} a[m][k] * w[n][k].
//
// On CDNA4 one V_MFMA_F32_16X16X128_F8F6F4 instruction computes P_kb for a
// 16x16 output tile exactly (FP8 products, FP32 sum inside the matrix core),
// so the promotion interval is one instruction: the MFMA runs with a zero
// accumulator and the result is folded into FP32 accumulators in VGPRs with
// one FMA by sa*sw.  There is no separate "CUDA core" copy: the MFMA result
// already lands in the register file the FMAs read.
//
// Structure of one workgroup tile (BM x BN, K stepped 128 at a time):
//   - A (BM x 128 bytes) and W (BN x 128 bytes) tiles plus the tile's
//     activation scales for the K block are staged in LDS, double buffered:
//     the next block's global loads are in flight while the MFMAs of the
//     current one run; one barrier per K block.
//   - LDS rows are 128 bytes; 16-byte chunk j of row r is stored at chunk
//     j ^ (r & 7), so the MFMA operand reads (16 rows x 32 bytes per lane
//     group) and the tile stores are bank-conflict free.
//   - Waves are arranged (BM/WM) x (BN/WN); each owns a WM x WN sub-tile of
//     (WM/16) x (WN/16) MFMA tiles and their FP32 accumulators.
//   - blockIdx is remapped so that each XCD (hardware dispatches consecutive
//     workgroups round-robin over the 8 XCDs, each with its own L2) works on
//     a contiguous, compact range of output tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8blk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kNumXcd = 8;

// 16x16x128 E4M3 x E4M3 -> FP32 product of one K block with a zero
// accumulator.  The scaled-MFMA builtin with zero scale operands selects the
// plain (unscaled) instruction.
__device__ __forceinline__ v4f mfma_e4m3(const v8i &a, const v8i &b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutPartial = 2 };

struct GemmParams {
    const uint8_t *a;
    const float *sa;
    const uint8_t *w;
    const float *sw;
    void *c;
    float *partial;          // split-K partials [ksplit][M][N] (dense only)
    const int32_t *offsets;  // grouped only
    int64_t M, N, K;         // M = T for grouped
    int G;                   // K / 128
    int NB;                  // N / 128
    int tiles_m, tiles_n;
    int ntiles;              // real tiles (dense: tiles_m * tiles_n * ksplit)
    int ksplit, kb_per_split;
    int E;
    int group_m;             // tile-order grouping height (in M tiles)
};

template <int BM_, int BN_, int WAVES_M, int WAVES_N>
struct TileCfg {
    static constexpr int BM = BM_;
    static constexpr int BN = BN_;
    static constexpr int kWavesM = WAVES_M;
    static constexpr int kWavesN = WAVES_N;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int WM = BM / WAVES_M;
    static constexpr int WN = BN / WAVES_N;
    static constexpr int kTM = WM / 16;
    static constexpr int kTN = WN / 16;
    // direct global->LDS loads: one wave instruction fills 8 rows x 128 B
    static constexpr int kALoads = BM / 8 / kWaves;
    static constexpr int kBLoads = BN / 8 / kWaves;
    static constexpr int kSaLoads = BM / 64;  // one dword per lane per row
    static constexpr int kSwSlots = 64;
    static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "loader");
    static_assert(BM % 64 == 0 && kSaLoads <= kWaves - 1, "scale loader");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns sit in one 128-block");
};

template <int BM, int BN>
struct __align__(16) Smem {
    uint8_t a[2][BM * 128];
    uint8_t b[2][BN * 128];
    float sa[2][BM];
    float sw[2][64];
};

// 16-byte chunk j of LDS row r is stored at chunk j ^ swz(r).  Rows r and
// r ^ 1 sit in one 256-byte line, so the XOR key is taken from r >> 1: the
// 16 rows one MFMA operand read touches land on 16 distinct 16-byte bank
// groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int chunk) { return r * 128 + ((chunk ^ swz(r)) << 4); }

__device__ __forceinline__ v8i make_v8i(const uint4 &lo, const uint4 &hi) {
    v8i v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *glb_ptr_t;

// Asynchronous global -> LDS copies (global_load_lds_dwordx4 / _dword): the
// wave's 64 lanes fill 64 * 16 (or 64 * 4) consecutive LDS bytes starting at
// the wave-uniform lds_wave_base, lane L at offset 16 L (4 L).
__device__ __forceinline__ void load_lds16(const void *g, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds((glb_ptr_t)(g), (lds_ptr_t)(lds_wave_base), 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void *g, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds((glb_ptr_t)(g), (lds_ptr_t)(lds_wave_base), 4, 0, 0);
}

// Runs K blocks [kb0, kb1) of one BM x BN tile and leaves the FP32
// accumulators in acc.  Rows are read at min(row0 + r, row_last) and columns
// at min(n0 + c, n_last), so a ragged edge never reads outside the operands
// (the extra rows/columns compute values that the caller does not store).
//
// Pipeline (two LDS stages): at the top of iteration kb every wave issues
// its direct global->LDS copies of block kb + 1 into the other stage, then
// runs the MFMAs of block kb from LDS, then waits for its copies and meets
// the others at one barrier.
template <class C>
__device__ __forceinline__ void tile_mainloop(
    const uint8_t *__restrict__ a, const float *__restrict__ sa, const uint8_t *__restrict__ w,
    const float *__restrict__ sw, int64_t row0, int64_t row_last, int64_t n0, int64_t n_last,
    int64_t K, int G, int kb0, int kb1, Smem<C::BM, C::BN> &sm, v4f (&acc)[C::kTM][C::kTN]) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::kWavesN;
    const int wn = wave % C::kWavesN;
    const int lr = lane & 15;  // row (A) / column (B) inside a 16x16 MFMA tile
    const int lk = lane >> 4;  // which 32-byte quarter of the 128-deep K block

#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Global source of this lane for each of its wave's copy instructions.
    // Copy t of wave w fills LDS rows [8 (w + kWaves t), +8); lane L writes
    // physical chunk L % 8 of row L / 8, which holds logical chunk
    // (L % 8) ^ swz(row).
    const uint8_t *ga[C::kALoads];
    const uint8_t *gb[C::kBLoads];
#pragma unroll
    for (int t = 0; t < C::kALoads; ++t) {
        const int r = 8 * (wave + C::kWaves * t) + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(r);
        ga[t] = a + min(row0 + r, row_last) * K + chunk * 16;
    }
#pragma unroll
    for (int t = 0; t < C::kBLoads; ++t) {
        const int r = 8 * (wave + C::kWaves * t) + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(r);
        gb[t] = w + min(n0 + r, n_last) * K + chunk * 16;
    }
    // Scales: waves 0 .. kSaLoads-1 copy 64 activation-scale rows each; the
    // last wave copies the weight scales of the tile's 128-column blocks.
    const float *gs;
    if (wave < C::kSaLoads)
        gs = sa + min(row0 + 64 * wave + lane, row_last) * G;
    else
        gs = sw + min((n0 >> 7) + lane, n_last >> 7) * G;

    auto issue = [&](int kb, int st) {
        const int64_t koff = (int64_t)kb * 128;
#pragma unroll
        for (int t = 0; t < C::kALoads; ++t)
            load_lds16(ga[t] + koff, &sm.a[st][1024 * (wave + C::kWaves * t)]);
#pragma unroll
        for (int t = 0; t < C::kBLoads; ++t)
            load_lds16(gb[t] + koff, &sm.b[st][1024 * (wave + C::kWaves * t)]);
        if (wave < C::kSaLoads)
            load_lds4(gs + kb, &sm.sa[st][64 * wave]);
        else if (wave == C::kWaves - 1)
            load_lds4(gs + kb, &sm.sw[st][0]);
    };

    issue(kb0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const int sw_slot = (int)(((n0 + wn * C::WN) >> 7) - (n0 >> 7));
    for (int kb = kb0; kb < kb1; ++kb) {
        const int st = (kb - kb0) & 1;
        if (kb + 1 < kb1) issue(kb + 1, st ^ 1);

        const uint8_t *la = sm.a[st];
        const uint8_t *lb = sm.b[st];
        v8i bfr[C::kTN];
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) {
            const int r = wn * C::WN + j * 16 + lr;
            const uint4 lo = *reinterpret_cast<const uint4 *>(lb + lds_off(r, 2 * lk));
            const uint4 hi = *reinterpret_cast<const uint4 *>(lb + lds_off(r, 2 * lk + 1));
            bfr[j] = make_v8i(lo, hi);
        }
        const float swv = sm.sw[st][sw_slot];
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            const int r = wm * C::WM + i * 16 + lr;
            const uint4 lo = *reinterpret_cast<const uint4 *>(la + lds_off(r, 2 * lk));
            const uint4 hi = *reinterpret_cast<const uint4 *>(la + lds_off(r, 2 * lk + 1));
            const v8i af = make_v8i(lo, hi);
            const float4 s4 =
                *reinterpret_cast<const float4 *>(&sm.sa[st][wm * C::WM + i * 16 + 4 * lk]);
            const float sc0 = s4.x * swv, sc1 = s4.y * swv, sc2 = s4.z * swv, sc3 = s4.w * swv;
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) {
                const v4f p = mfma_e4m3(af, bfr[j]);
                acc[i][j][0] = __builtin_fmaf(p[0], sc0, acc[i][j][0]);
                acc[i][j][1] = __builtin_fmaf(p[1], sc1, acc[i][j][1]);
                acc[i][j][2] = __builtin_fmaf(p[2], sc2, acc[i][j][2]);
                acc[i][j][3] = __builtin_fmaf(p[3], sc3, acc[i][j][3]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
}

// Writes the accumulators of one tile: rows [row0, row_end) and columns
// [n0, N) are stored; the MFMA output layout puts rows 4*(lane/16) + e and
// column lane % 16 of each 16x16 tile in a lane.
template <class C, int OUT>
__device__ __forceinline__ void tile_store(const v4f (&acc)[C::kTM][C::kTN], void *c, int64_t ldc,
                                           int64_t row0, int64_t row_end, int64_t n0,
                                           int64_t N) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::kWavesN;
    const int wn = wave % C::kWavesN;
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) {
            const int64_t col = n0 + wn * C::WN + j * 16 + (lane & 15);
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = row0 + wm * C::WM + i * 16 + 4 * (lane >> 4) + e;
                if (row >= row_end) continue;
                const float v = acc[i][j][e];
                if (OUT == kOutBF16)
                    static_cast<uint16_t *>(c)[row * ldc + col] = (uint16_t)f32_to_bf16_bits(v);
                else
                    static_cast<float *>(c)[row * ldc + col] = v;
            }
        }
}

// Logical tile index of this workgroup after the XCD remap (gridDim.x is a
// multiple of 8; each XCD gets a contiguous range of logical tiles).
__device__ __forceinline__ int xcd_logical_tile() {
    const int per = gridDim.x / kNumXcd;
    return (blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd;
}

template <class C, int OUT>
__global__ __launch_bounds__(C::kThreads) void dense_gemm_kernel(GemmParams p) {
    __shared__ Smem<C::BM, C::BN> sm;
    const int logical = xcd_logical_tile();
    if (logical >= p.ntiles) return;
    const int per_split = p.tiles_m * p.tiles_n;
    const int ks = logical / per_split;
    const int t = logical - ks * per_split;
    // Grouped raster: runs of group_m M tiles sweep across N, so consecutive
    // logical tiles share W columns (and nearby ones share A rows).
    const int span = p.group_m * p.tiles_n;
    const int grp = t / span;
    const int first_m = grp * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int in = t - grp * span;
    const int tm = first_m + in % gm;
    const int tn = in / gm;

    const int64_t row0 = (int64_t)tm * C::BM;
    const int64_t n0 = (int64_t)tn * C::BN;
    const int kb0 = ks * p.kb_per_split;
    const int kb1 = min(kb0 + p.kb_per_split, p.G);

    v4f acc[C::kTM][C::kTN];
    tile_mainloop<C>(p.a, p.sa, p.w, p.sw, row0, p.M - 1, n0, p.N - 1, p.K, p.G, kb0, kb1, sm, acc);
    if (OUT == kOutPartial)
        tile_store<C, kOutF32>(acc, p.partial + (int64_t)ks * p.M * p.N, p.N, row0, p.M, n0, p.N);
    else
        tile_store<C, OUT>(acc, p.c, p.N, row0, p.M, n0, p.N);
}

// Split-K reduction: C = sum over splits in fixed order 0..S-1, then the
// output conversion.  Four elements per thread (M*N is a multiple of 128).
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partial,
                                                            void *__restrict__ c, int64_t MN,
                                                            int S) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;
    float4 s = *reinterpret_cast<const float4 *>(partial + i);
    for (int k = 1; k < S; ++k) {
        const float4 v = *reinterpret_cast<const float4 *>(partial + (int64_t)k * MN + i);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if (OUT == kOutBF16) {
        uint2 o;
        o.x = f32_to_bf16_bits(s.x) | (f32_to_bf16_bits(s.y) << 16);
        o.y = f32_to_bf16_bits(s.z) | (f32_to_bf16_bits(s.w) << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(c) + i) = o;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(c) + i) = s;
    }
}

// Grouped GEMM.  Logical tiles are ordered expert by expert; inside an
// expert, N tile by N tile, and the expert's M tiles are consecutive, so the
// M tiles that share one W tile run next to each other on one XCD.  The
// offsets live on the device: thread 0 walks them (clamped to [0, T]; a
// decreasing range is empty) to find this tile's expert, and the grid is
// sized for the worst case (ceil(T/BM) + E) * tiles_n, surplus tiles exit.
template <class C, int OUT>
__global__ __launch_bounds__(C::kThreads) void grouped_gemm_kernel(GemmParams p) {
    __shared__ Smem<C::BM, C::BN> sm;
    __shared__ int64_t info[4];
    const int logical = xcd_logical_tile();
    if (threadIdx.x == 0) {
        int64_t rem = logical;
        int64_t e_hit = -1, r0 = 0, r1 = 0, tn = 0;
        for (int e = 0; e < p.E; ++e) {
            int64_t lo = p.offsets[e], hi = p.offsets[e + 1];
            lo = lo < 0 ? 0 : (lo > p.M ? p.M : lo);
            hi = hi < 0 ? 0 : (hi > p.M ? p.M : hi);
            const int64_t cnt = hi > lo ? hi - lo : 0;
            const int64_t mt = (cnt + C::BM - 1) / C::BM;
            const int64_t tiles = mt * p.tiles_n;
            if (rem < tiles) {
                e_hit = e;
                tn = rem / mt;
                r0 = lo + (rem - tn * mt) * C::BM;
                r1 = hi;
                break;
            }
            rem -= tiles;
        }
        info[0] = e_hit;
        info[1] = r0;
        info[2] = r1;
        info[3] = tn;
    }
    __syncthreads();
    const int64_t e = info[0];
    if (e < 0) return;
    const int64_t row0 = info[1], row_end = info[2];
    const int64_t n0 = info[3] * C::BN;

    const uint8_t *w = p.w + e * p.N * p.K;
    const float *sw = p.sw + e * (int64_t)p.NB * p.G;
    v4f acc[C::kTM][C::kTN];
    tile_mainloop<C>(p.a, p.sa, w, sw, row0, row_end - 1, n0, p.N - 1, p.K, p.G, 0, p.G, sm, acc);
    tile_store<C, OUT>(acc, p.c, p.N, row0, row_end, n0, p.N);
}

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Tile shapes: 256 x 256 on 8 waves (wave tile 128 x 64) for GEMMs that fill
// the GPU; 128 x 128 on 4 waves (wave tile 64 x 64) for small ones, with
// split-K when even those tiles cannot occupy the 256 CUs.
using BigTile = TileCfg<256, 256, 2, 4>;
using SmallTile = TileCfg<128, 128, 2, 2>;
constexpr int kCUs = 256;

struct Plan {
    bool big;
    int ksplit;
    int kb_per_split;
};

Plan plan_dense(int64_t M, int64_t N, int64_t K) {
    const int G = (int)(K / 128);
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (big_tiles >= kCUs) return {true, 1, G};
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    int s = 1;
    // Split K only when the output tiles cannot fill the CUs and each split
    // keeps at least 4 K blocks.
    while (tiles * s * 2 <= kCUs && G / (s * 2) >= 4) s *= 2;
    const int per = (G + s - 1) / s;
    s = (G + per - 1) / per;
    return {false, s, per};
}

template <class C, int OUT>
hipError_t launch_dense(const GemmParams &p0, hipStream_t stream) {
    GemmParams p = p0;
    p.tiles_m = (int)((p.M + C::BM - 1) / C::BM);
    p.tiles_n = (int)((p.N + C::BN - 1) / C::BN);
    p.ntiles = p.tiles_m * p.tiles_n * p.ksplit;
    const int grid = round_up(p.ntiles, kNumXcd);
    hipLaunchKernelGGL((dense_gemm_kernel<C, OUT>), dim3(grid), dim3(C::kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const Plan pl = plan_dense(M, N, K);
    if (pl.ksplit <= 1) return 0;
    return (size_t)pl.ksplit * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_block_gemm(const void *a, const float *sa, const void *w, const float *sw,
                             void *c, bool bf16_out, int64_t M, int64_t N, int64_t K,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    GemmParams p{};
    p.a = static_cast<const uint8_t *>(a);
    p.sa = sa;
    p.w = static_cast<const uint8_t *>(w);
    p.sw = sw;
    p.c = c;
    p.M = M;
    p.N = N;
    p.K = K;
    p.G = (int)(K / 128);
    p.NB = (int)(N / 128);
    p.group_m = 8;
    Plan pl = plan_dense(M, N, K);
    const size_t need = gemm_workspace_bytes(M, N, K);
    if (pl.ksplit > 1 && (workspace == nullptr || workspace_bytes < need)) pl = {false, 1, p.G};
    p.ksplit = pl.ksplit;
    p.kb_per_split = pl.kb_per_split;
    if (pl.big)
        return bf16_out ? launch_dense<BigTile, kOutBF16>(p, stream)
                        : launch_dense<BigTile, kOutF32>(p, stream);
    if (p.ksplit > 1) {
        p.partial = static_cast<float *>(workspace);
        hipError_t e = launch_dense<SmallTile, kOutPartial>(p, stream);
        if (e != hipSuccess) return e;
        const int64_t MN = M * N;
        const int64_t blocks = (MN / 4 + 255) / 256;
        if (bf16_out)
            hipLaunchKernelGGL(splitk_reduce_kernel<kOutBF16>, dim3((unsigned)blocks), dim3(256), 0,
                               stream, p.partial, c, MN, p.ksplit);
        else
            hipLaunchKernelGGL(splitk_reduce_kernel<kOutF32>, dim3((unsigned)blocks), dim3(256), 0,
                               stream, p.partial, c, MN, p.ksplit);
        return hipGetLastError();
    }
    return bf16_out ? launch_dense<SmallTile, kOutBF16>(p, stream)
                    : launch_dense<SmallTile, kOutF32>(p, stream);
}

hipError_t launch_grouped_gemm(const void *a, const float *sa, const void *w, const float *sw,
                               const int32_t *offsets, int64_t E, int64_t T, void *c,
                               bool bf16_out, int64_t N, int64_t K, hipStream_t stream) {
    using C = SmallTile;
    GemmParams p{};
    p.a = static_cast<const uint8_t *>(a);
    p.sa = sa;
    p.w = static_cast<const uint8_t *>(w);
    p.sw = sw;
    p.c = c;
    p.offsets = offsets;
    p.M = T;
    p.N = N;
    p.K = K;
    p.G = (int)(K / 128);
    p.NB = (int)(N / 128);
    p.E = (int)E;
    p.tiles_n = (int)((N + C::BN - 1) / C::BN);
    p.tiles_m = (int)((T + C::BM - 1) / C::BM) + (int)E;  // worst-case M tiles over all experts
    p.ntiles = p.tiles_m * p.tiles_n;
    p.ksplit = 1;
    p.kb_per_split = p.G;
    const int grid = round_up(p.ntiles, kNumXcd);
    if (bf16_out)
        hipLaunchKernelGGL((grouped_gemm_kernel<C, kOutBF16>), dim3(grid), dim3(C::kThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<C, kOutF32>), dim3(grid), dim3(C::kThreads), 0,
                           stream, p);
    return hipGetLastError();
}

}  // namespace fp8blk
