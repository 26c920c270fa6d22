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
// 16x16 output tile inside the matrix core (exact FP8 products; measured on
// gfx950: each aligned group of 8 products is summed to 14 significant bits,
// truncated, and the groups are added in FP32 -- tests/test_mfma_accum_gpu.py),
// so the promotion interval is one instruction: the MFMA runs with a zero
// accumulator and the result is folded into FP32 accumulators in VGPRs with
// one FMA by sa*sw.  No copy to other registers is needed: the MFMA result
// already lands in the register file the FMAs read.
//
// Structure of one workgroup tile (BM x BN, K stepped 128 at a time):
//   - A (BM x 128 bytes) and W (BN x 128 bytes) tiles plus the weight
//     scales of the K block are staged in LDS by direct global->LDS copies
//     (weights with the nontemporal cache policy), issued one or more blocks
//     ahead of the MFMAs that use them (see tile_mainloop).  The tile's
//     activation scales are fetched eight K blocks at a time into a separate
//     double buffer.
//   - LDS rows are 128 bytes; 16-byte chunk j of row r is stored at chunk
//     j ^ key(r), so the MFMA operand reads (16 rows x 32 bytes per lane
//     group) are bank-conflict free.
//   - Waves are arranged (BM/WM) x (BN/WN); each owns a WM x WN sub-tile of
//     (WM/16) x (WN/16) MFMA tiles and their FP32 accumulators.
//   - blockIdx is remapped so that each XCD (hardware dispatches consecutive
//     workgroups round-robin over the 8 XCDs, each with its own L2) works on
//     a contiguous, compact range of output tiles.
//   - The output tile leaves through LDS in whole 128-byte lines.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8blk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNumXcd = 8;

// 16x16x128 E4M3 x E4M3 -> FP32 product of one K block with a zero
// accumulator.  The scaled-MFMA builtin with zero scale operands selects the
// plain (unscaled) instruction.
__device__ __forceinline__ v4f mfma_e4m3(const v8i &a, const v8i &b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// The block-scaled form for power-of-two scales: c + 2^(ca - 127) 2^(cb -
// 127) (a . b), with E8M0 codes ca, cb in byte 0 of the scale operands.
// Each lane's code applies to the operand row it holds (and its 32-deep K
// quarter); here every lane holding a row passes that row's code.
__device__ __forceinline__ v4f mfma_e4m3_scaled(const v8i &a, const v8i &b, const v4f &c,
                                                int ca, int cb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ca, 0, cb);
}

// E8M0 code of a power-of-two fp32 scale (its exponent field), carried in
// a float register's bits.
__device__ __forceinline__ float e8m0_code(float s) {
    return __uint_as_float(__float_as_uint(s) >> 23);
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
    int tn1, tn2;            // two-kind plan: 256-wide and 192-wide N tiles
    int64_t n_split;         // two-kind plan: first column of the 192-wide tiles
    // quantization fused into the GEMM: bf16 activations in, and optionally
    // their E4M3 bytes and scales out
    const uint16_t *x;
    uint8_t *q_out;
    float *sa_out;
    // transposed weights (Dgrad): W is [K][N] (row length ldw = N bytes) and
    // its block scales [K/128][N/128]; the tiles read it transposed
    int64_t ldw;
};

// SCALE_PIECES: activation scales are staged in chunks of 4 * SCALE_PIECES K
// blocks.  ROW_SCALED_W: W has one scale per row and K block (1x128 tiles,
// the Wgrad operands) instead of one per 128-row block; those row scales are
// staged in chunks like the activation scales.
template <int BM_, int BN_, int WAVES_M, int WAVES_N, int STAGES, int SCALE_PIECES = 2,
          bool ROW_SCALED_W = false>
struct TileCfg {
    static constexpr int kStages = STAGES;
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
    // activation scales come in chunks of kScaleChunk K blocks: 16 bytes
    // (4 blocks, one piece) per lane, so one wave instruction fetches 64 row
    // pieces
    static constexpr int kScalePieces = SCALE_PIECES;
    static constexpr int kScaleChunk = 4 * SCALE_PIECES;
    static constexpr int kScaleCopies = SCALE_PIECES * BM / 64;  // per chunk, over all waves
    static constexpr int kScaleLoads = (kScaleCopies + kWaves - 1) / kWaves;  // per wave, at most
    static constexpr bool kRowScaledW = ROW_SCALED_W;
    static constexpr int kScaleCopiesW = ROW_SCALED_W ? SCALE_PIECES * BN / 64 : 0;
    static constexpr int kScaleLoadsW = (kScaleCopiesW + kWaves - 1) / kWaves;
    static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "loader");
    static_assert((SCALE_PIECES * BM) % 64 == 0 && (SCALE_PIECES * BN) % 64 == 0, "scale loader");
    static_assert(SCALE_PIECES == 1 || SCALE_PIECES == 2, "scale chunk pieces");
    static_assert(((BM + BN) * 128) % 4096 == 0, "stage size");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
    // A wave's columns sit in one 128-column weight-scale block when WN
    // divides 128 (tiles start at multiples of BN); otherwise each 16-column
    // fragment looks up its own block.
    static constexpr bool kWaveInOneBlock = WN <= 128 && 128 % WN == 0;
    static_assert(STAGES >= 2, "pipeline");
    // a scale chunk buffer is reloaded for the block kScaleChunk blocks after
    // its last user; with copies issued D <= STAGES - 1 blocks ahead, after a
    // barrier that every wave passes only once it finished the block before,
    // that user is done once D <= kScaleChunk
    static_assert(STAGES - 1 <= kScaleChunk, "scale chunk double buffer");
    // copy instructions each wave issues per K block (A, W; tiles that read W
    // transposed add their weight-scale copy); a scale chunk adds kScaleLoads
    // (+ kScaleLoadsW) + 1 more every kScaleChunk blocks
    static constexpr int kCopiesPerBlock = kALoads + kBLoads;
    static_assert((STAGES - 2) * kCopiesPerBlock <= 63, "vmcnt range");  // wait count in the loop
};

// One LDS pipeline stage: the A (token) and W (weight) tiles of one K block.
// Every 16-row operand tile starts 2 KiB-aligned (the bank layout below
// assumes it).
template <int BM, int BN>
struct __align__(4096) Stage {
    uint8_t a[BM * 128];
    uint8_t b[BN * 128];
};

// Activation scales of the tile's BM rows for kScaleChunk = 4 P consecutive
// K blocks (P pieces of 16 bytes), double buffered.  The scales are stored
// [M][K/128] in memory, so a row's scales for one K block each sit in a
// different cache line; fetching 4 P blocks per row at once makes one L2
// request serve several blocks instead of one.  Piece h of row r of buffer b
// holds blocks 4 P c + 4 h .. + 3 at float4 index (P b + h) ROWS + r: the 16
// lanes that read one M tile's rows hit 16 distinct 16-byte bank groups.
template <int ROWS, int P>
struct ScaleChunks {
    float v[2][P][ROWS][4];
};

// Everything a workgroup keeps in LDS: the operand stages, the activation
// scale chunks and the weight scales of the tile's 128-column blocks.  The
// weight scales are chunked like the activation scales: buffer b holds at
// word nb kScaleChunk + j the scale of the tile's column block nb for K block
// kScaleChunk c + j (one copy instruction per wave per chunk instead of one
// per K block).  Tiles that read W transposed keep one slot per stage
// instead, holding the stage's block scales at word nb (fetched per K block:
// chunked, that kernel measured ~3% slower).
template <class C>
struct TileLds {
    Stage<C::BM, C::BN> stages[C::kStages];
    ScaleChunks<C::BM, C::kScalePieces> chunks;
    float swc[C::kStages > 2 ? C::kStages : 2][64];
    // row-scaled W only: its rows' scales, chunked like the activation scales
    ScaleChunks<(C::kRowScaledW ? C::BN : 4), C::kScalePieces> wchunks;
};

// LDS layout of an operand tile: rows of 128 bytes (one K block); 16-byte
// chunk c of row r is stored at chunk c ^ key(r), key(r) = (r & 7) ^ ((r >> 3)
// & 1).  With it, an MFMA operand read (16 lanes reading one chunk of 16
// consecutive rows, four such groups) runs at the full 16 bytes per lane
// per ds_read_b128 issue slot without bank conflicts on gfx950 (found by
// measuring the LDS bank-conflict counters over candidate layouts; plain
// r & 7 costs twice the cycles).  Tile copies still write whole 128-byte
// rows.
__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ v8i make_v8i(const uint4 &lo, const uint4 &hi) {
    v8i v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads whose per-lane offset
// is at or past `bytes` return zero instead of reading memory.
__device__ __forceinline__ v4i make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(uint32_t)(uintptr_t)(lds_ptr_t)(const_cast<void *>(p)));
}

// Asynchronous global -> LDS copies (buffer_load_dwordx4 / _dword with the
// lds modifier): the wave's 64 lanes fill 64 * 16 (or 64 * 4) consecutive
// LDS bytes from the wave-uniform LDS address in M0, lane L at offset 16 L
// (4 L); voffset is the lane's byte offset in the buffer, soffset the K
// block's.  They are written as inline assembly on purpose: the compiler
// orders every LDS read after all outstanding LDS-DMA copies it knows of,
// which would serialize the next block's copy with this block's MFMAs.
// These instructions have no register results; the data they write is read
// only after an explicit "s_waitcnt vmcnt" that covers the copy and a
// barrier (see tile_mainloop).
//
// M0 is reserved to the compiler, so each copy saves it in a scratch SGPR,
// sets the LDS address, issues the load (which takes M0 at issue: copies
// back to back with different addresses land where they should) and puts
// the old value back.
//
// Race-check builds (FP8BLK_POISON_LDS defined): before each copy the wave
// first fills the LDS bytes the copy will write with 0x7F (an E4M3 NaN;
// 3.4e38 as an fp32 scale) and waits for those writes.  A wave that still
// read a stage after another wave began to refill it would then see poison
// at once, instead of the old data that a copy still in flight has not yet
// overwritten, and its outputs would be wrong.  Released builds leave this
// out.
#ifdef FP8BLK_POISON_LDS
__device__ __forceinline__ void poison_lds(uint32_t lds, int bytes_per_lane) {
    typedef __attribute__((address_space(3))) uint32_t *lds_u32_t;
    lds_u32_t p = (lds_u32_t)(uintptr_t)(lds + (uint32_t)(bytes_per_lane * (threadIdx.x & 63)));
    for (int i = 0; i < bytes_per_lane / 4; ++i) p[i] = 0x7F7F7F7Fu;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
#define FP8BLK_POISON(lds, bytes) poison_lds(lds, bytes)
#else
#define FP8BLK_POISON(lds, bytes) ((void)0)
#endif
__device__ __forceinline__ void copy16(const v4i &r, uint32_t voff, uint32_t soff, uint32_t lds) {
    FP8BLK_POISON(lds, 16);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(r), "s"(soff), "s"(lds)
        : "memory");
}
// The same copy with the nontemporal cache policy, for the weight tiles:
// streamed from HBM, plain copies of this pattern top out near 2.6 TB/s
// while nontemporal ones reach ~6.5 TB/s (measured with a streaming probe);
// the activation tiles, which neighbouring tiles re-read through L2, keep
// the default policy.
__device__ __forceinline__ void copy16_nt(const v4i &r, uint32_t voff, uint32_t soff,
                                          uint32_t lds) {
    FP8BLK_POISON(lds, 16);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(r), "s"(soff), "s"(lds)
        : "memory");
}
__device__ __forceinline__ void copy4(const v4i &r, uint32_t voff, uint32_t soff, uint32_t lds) {
    FP8BLK_POISON(lds, 4);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\t"
        "buffer_load_dword %1, %2, %3 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(r), "s"(soff), "s"(lds)
        : "memory");
}

// Per-tile operand view for the main loop.  Rows [row0, row0 + rows) of A
// and columns [n0, n0 + cols) of W are valid; the buffer bounds make every
// other row read as zero, so ragged edges need no clamping.
struct TileOperands {
    v4i a, w, sa, sw, swr;  // swr: W row scales (row-scaled W only)
    // weight-scale fetch: lane L of a chunk copy reads the scale of the
    // tile's 128-column block L / kScaleChunk for K block kScaleChunk c + L %
    // kScaleChunk, at byte offset (L / kScaleChunk) sw_lstride + (L %
    // kScaleChunk) sw_kstride (voffset) + kScaleChunk c sw_kstride (soffset)
    // of the sw view; with W read transposed, lane L of the per-block copy
    // reads block L for K block kb at L sw_lstride + kb sw_kstride
    uint32_t sw_lstride, sw_kstride;
    uint32_t ldw;           // transposed W only: bytes per row of W [K][N]
};

template <class C>
__device__ __forceinline__ TileOperands tile_operands(const uint8_t *a, const float *sa,
                                                      const uint8_t *w, const float *sw,
                                                      int64_t row0, int64_t rows, int64_t n0,
                                                      int64_t cols, int64_t K, int G) {
    TileOperands t;
    const int64_t ra = rows < C::BM ? rows : C::BM;
    const int64_t cw = cols < C::BN ? cols : C::BN;
    t.a = make_rsrc(a + row0 * K, (uint32_t)(ra * K));
    t.w = make_rsrc(w + n0 * K, (uint32_t)(cw * K));
    t.sa = make_rsrc(sa + row0 * G, (uint32_t)(ra * G * 4));
    if constexpr (C::kRowScaledW) {
        // sw is [cols][G]: rows n0 .. n0 + cw of it.  The weight-scale chunk
        // copy still runs (from an empty buffer) so the wait counts stay
        // those of the block-scaled layout.
        t.swr = make_rsrc(sw + n0 * G, (uint32_t)(cw * G * 4));
        t.sw = make_rsrc(sw, 0);
    } else {
        const int64_t nb0 = n0 >> 7, nbs = ((n0 + cw - 1) >> 7) - nb0 + 1;
        t.sw = make_rsrc(sw + nb0 * G, (uint32_t)(nbs * G * 4));
        t.swr = make_rsrc(sw, 0);
    }
    t.sw_lstride = (uint32_t)G * 4u;
    t.sw_kstride = 4u;
    t.ldw = 0;
    return t;
}

// Operands of a tile whose weights are stored transposed, W [K][N] with
// block scales [K/128][N/128] (the forward layer's weights, read for Dgrad):
// the tile's columns n0 .. n0 + cols of every row of W.  Columns past N read
// whatever follows in memory (other rows' bytes; zero past the end of W) and
// feed only outputs that are not stored.
template <class C>
__device__ __forceinline__ TileOperands tile_operands_transw(const uint8_t *a, const float *sa,
                                                             const uint8_t *w, const float *sw,
                                                             int64_t row0, int64_t rows,
                                                             int64_t n0, int64_t cols, int64_t K,
                                                             int G, int64_t ldw, int NB) {
    TileOperands t;
    const int64_t ra = rows < C::BM ? rows : C::BM;
    const int64_t cw = cols < C::BN ? cols : C::BN;
    t.a = make_rsrc(a + row0 * K, (uint32_t)(ra * K));
    t.sa = make_rsrc(sa + row0 * G, (uint32_t)(ra * G * 4));
    t.w = make_rsrc(w + n0, (uint32_t)(K * ldw - n0));
    const int64_t nb0 = n0 >> 7, nbs = ((n0 + cw - 1) >> 7) - nb0 + 1;
    // Lane L of the per-block copy reads sw[kb][nb0 + L] at offset 4 L +
    // kb NB 4 (soffset): the buffer range check covers voffset + soffset,
    // so the range runs to the end of the scales (lanes past the tile's
    // blocks read other blocks' scales into LDS words nobody uses; past the
    // end they read zero).
    t.sw = make_rsrc(sw + nb0, (uint32_t)(((int64_t)(G - 1) * NB + nbs) * 4));
    t.swr = make_rsrc(sw, 0);
    t.sw_lstride = 4u;
    t.sw_kstride = (uint32_t)NB * 4u;
    t.ldw = (uint32_t)ldw;
    return t;
}

// LDS layout of a transposed W tile: 128 rows (the K block) of BN bytes (the
// tile's columns); logical 16-byte chunk c of row r sits at physical chunk
// tw_phys(c, tw_key(r)): c ^ key for a power-of-two chunk count, else
// (c + key) mod chunks.  The transposed reads (ds_read_b64_tr_b8) of one
// instruction touch rows 32 lk + 8 q + (0..7) of four lane groups lk at one
// chunk; with this key the 16 rows of each half wave land on 16 distinct
// chunks for BN = 256 (256 B, every bank once; two rows per chunk for the
// 12 chunks of BN = 192).
__device__ __forceinline__ int tw_key(int r) { return (r & 7) | (((r >> 5) & 1) << 3); }
template <int BN>
__device__ __forceinline__ int tw_phys(int c, int key) {
    constexpr int n = BN / 16;
    if constexpr ((n & (n - 1)) == 0)
        return (c ^ key) & (n - 1);
    else
        return (c + key) % n;
}
template <int BN>
__device__ __forceinline__ int tw_logical(int p, int key) {
    constexpr int n = BN / 16;
    if constexpr ((n & (n - 1)) == 0)
        return (p ^ key) & (n - 1);
    else
        return (p - key % n + n) % n;
}

// Runs K blocks [kb0, kb1) of one BM x BN tile and leaves the FP32
// accumulators in acc.
//
// Pipeline over kStages LDS stages.  A block is computed row of 16-row tiles
// by row: each row's token fragment, then its MFMAs with the weight
// fragments, each followed by the promotion FMAs of the previous MFMA.  With
// two stages the copies of a block go in two groups issued half a block
// apart, with a barrier before each group's data is used, and the next
// block's weight fragments and scales are read during the current block's
// last row (details at the loop below).  With S >= 3 stages the copies run
// D = S - 1 blocks ahead: an iteration waits until at
// most the copies of the D - 1 newer blocks are outstanding, meets the
// others at a barrier, issues block kb + D into the stage last read in
// iteration kb - 1 and computes block kb.  Every wave issues the same
// copies, so the wait count is uniform; the activation-scale chunk of a
// block is issued before the block's operand copies, so the wait also
// covers it (an extra chunk copy among the newer ones only makes the wait
// stricter).
//
// Copy t of wave v fills LDS rows [8 (v + kWaves t), +8): lane L writes
// physical chunk L % 8 of row L / 8 of that block, i.e. the row's logical
// chunk (L % 8) ^ key(row).
//
// kPow2: the scales are powers of two.  Each MFMA then takes their E8M0 codes
// and accumulates into the FP32 accumulators itself (acc + sa sw P_kb in one
// instruction), so there is no promotion FMA.
//
// kTransW: W is stored transposed (see tile_operands_transw).  Its tile is
// copied as 128 rows of BN bytes and each MFMA weight fragment is read with
// four transposed LDS reads (ds_read_b64_tr_b8): in each 16-lane group,
// result byte b of lane i is byte i % 8 of the 8 bytes at the address of
// lane 2 b + i / 8, so lane s pointing at row 8 q + s / 2, bytes 8 (s % 2)
// .. + 8 of the fragment's 16 columns gives lane i the 8 K values 8 q ..
// 8 q + 7 of column i.
template <class C, bool kPow2 = false, bool kTransW = false>
__device__ __forceinline__ void tile_mainloop(const TileOperands &op, int64_t K, int G, int kb0,
                                              int kb1, int col_off,
                                              TileLds<C> &L,
                                              v4f (&acc)[C::kTM][C::kTN]) {
    using S = Stage<C::BM, C::BN>;
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

    // copy lane L fills physical chunk L % 8 of tile row 8 b + L / 8 (b = wave
    // + kWaves t, of the same parity as wave since kWaves is even), which
    // holds logical chunk (L % 8) ^ key(row)
    const uint32_t copy_voff = (uint32_t)(((lane >> 3) * K) +
                                          (((lane & 7) ^ ((lane >> 3) & 7) ^ (wave & 1)) << 4));
    const uint32_t rowstep = (uint32_t)(8 * C::kWaves * K);  // between copies t and t+1
    const uint32_t wave_voff = (uint32_t)(8 * wave * K) + copy_voff;
    // Scale chunk copy t of wave v fills float4 slots q = 64 (v + kWaves t) + L
    // of a chunk buffer: piece h = q / BM of row r = q % BM.
    // Offsets of the rarely issued scale copies are computed at each copy
    // from the lane index passed through an empty asm statement, so that
    // they do not occupy registers across the main loop.
    auto opaque_lane = [&] {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        return ln;
    };
    auto sa_voff = [&](int t) {
        const int q = 64 * (wave + C::kWaves * t) + opaque_lane();
        return (uint32_t)((q % C::BM) * G * 4 + (q / C::BM) * 16);
    };
    // Row-scaled W: W chunk copy t of wave v fills float4 slots q = 64 (v +
    // kWaves t) + L of a W chunk buffer, piece q / BN of W row q % BN.
    auto swr_voff = [&](int t) {
        const int q = 64 * (wave + C::kWaves * t) + opaque_lane();
        return (uint32_t)((q % C::BN) * G * 4 + (q / C::BN) * 16);
    };
    // weight-scale copies: per K block (transposed W; the lane's offset is
    // kept in a register) or per chunk (the offset is computed at each copy)
    constexpr bool kSwPerBlock = kTransW;
    const uint32_t sw_voff_blk = kSwPerBlock ? (uint32_t)lane * op.sw_lstride : 0u;
    auto sw_voff = [&] {
        if constexpr (kSwPerBlock) {
            return sw_voff_blk;
        } else {
            const int ln = opaque_lane();
            return (uint32_t)(ln / C::kScaleChunk) * op.sw_lstride +
                   (uint32_t)(ln % C::kScaleChunk) * op.sw_kstride;
        }
    };
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // for uniform branches
    // Transposed W: copy t of wave v fills bytes 1024 (v + kWaves t) .. +
    // 1024 of the stage's W tile (rows of BN bytes); lane L's 16 bytes at
    // tile offset pos = 1024 (v + kWaves t) + 16 L are row pos / BN,
    // physical chunk (pos % BN) / 16, which holds the logical chunk
    // tw_logical of it.
    static_assert(!kTransW || C::BN * 128 == C::kBLoads * C::kWaves * 1024,
                  "transposed W copies");
    // (computed at each copy from the lane index passed through an empty asm
    // statement, so these offsets do not occupy registers across the loop)
    auto wt_voff = [&](int t) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int pos = 1024 * (wave + C::kWaves * t) + 16 * ln;
        const int r = pos / C::BN;
        const int c = tw_logical<C::BN>((pos % C::BN) >> 4, tw_key(r));
        return (uint32_t)r * op.ldw + 16u * (uint32_t)c;
    };
    // LDS destinations of this wave's copies in stage 0 (stage s is s *
    // sizeof(S) bytes further) and in scale chunk buffer 0.
    const uint32_t lds_a0 = lds_addr(&L.stages[0].a[1024 * wave]);
    const uint32_t lds_b0 = lds_addr(&L.stages[0].b[1024 * wave]);
    const uint32_t lds_sw0 = lds_addr(&L.swc[0][0]);
    const uint32_t lds_sc0 =
        lds_addr(reinterpret_cast<const uint8_t *>(&L.chunks.v[0][0][0][0]) + 1024 * wave);
    const uint32_t lds_wc0 =
        lds_addr(reinterpret_cast<const uint8_t *>(&L.wchunks.v[0][0][0][0]) + 1024 * wave);

    // Copy t of A fills tile rows [8 kWaves t, +8 kWaves); with two stages
    // a block's A rows go in two halves: the rows of every wave's first
    // kTM / 2 M tiles, then the rest (see below).
    auto a_copy_in_half = [&](int t, int half) {
        return ((((8 * C::kWaves * t) % C::WM) < C::WM / 2) ? 0 : 1) == half;
    };
    auto issue_a = [&](const TileOperands &src, int kb, int st, int half) {
        const uint32_t soff = (uint32_t)kb * 128u;
        const uint32_t so = (uint32_t)(st * sizeof(S));
#pragma unroll
        for (int t = 0; t < C::kALoads; ++t)
            if (half < 0 || a_copy_in_half(t, half))
                copy16(src.a, wave_voff + t * rowstep, soff, lds_a0 + so + 1024 * C::kWaves * t);
    };
    auto issue_w = [&](const TileOperands &src, int kb, int st) {
        const uint32_t so = (uint32_t)(st * sizeof(S));
        if constexpr (kTransW) {
            // the K block's offset goes into voffset, which the buffer range
            // check covers (columns past N of the last rows stop at W's end)
            const uint32_t koff = (uint32_t)kb * 128u * op.ldw;
#pragma unroll
            for (int t = 0; t < C::kBLoads; ++t)
                copy16_nt(src.w, wt_voff(t) + koff, 0u, lds_b0 + so + 1024 * C::kWaves * t);
        } else {
            const uint32_t soff = (uint32_t)kb * 128u;
#pragma unroll
            for (int t = 0; t < C::kBLoads; ++t)
                copy16_nt(src.w, wave_voff + t * rowstep, soff,
                          lds_b0 + so + 1024 * C::kWaves * t);
        }
    };
    // A chunk that runs past the last K block (G not a multiple of
    // kScaleChunk) is fetched one dword per lane instead: a 16-byte piece of
    // the tile's last row would straddle the end of the scales, and the
    // buffer range check may treat such an access as wholly out of range
    // (losing the valid scales in it).  Here every lane's offset (voffset,
    // with the chunk's K offset in it) is checked on its own dword.  Dword copy u of a
    // chunk buffer fills its dwords 64 u .. + 63: dword d is block j = d % 4
    // of piece h = d / (4 ROWS) of row r = (d / 4) % ROWS.  More copies in a
    // block only make the pipeline's waits stricter.
    auto issue_chunk_dwords = [&](const v4i &rsrc, int rows, int c, uint32_t lds_buf) {
        const int copies = C::kScalePieces * rows / 16;  // over all waves
        // the lane index passes through an empty asm statement so that the
        // offsets below are computed here, in this rarely taken branch,
        // rather than hoisted out of the main loop into live registers
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int t = 0; t < (C::kScalePieces * (C::BM > C::BN ? C::BM : C::BN) / 16 + C::kWaves - 1) /
                                C::kWaves;
             ++t) {
            const int u = wave_u + C::kWaves * t;
            if (u < copies) {
                const int d = 64 * u + ln;
                const int h = d / (4 * rows), r = (d >> 2) % rows, j = d & 3;
                const uint32_t off =
                    (uint32_t)(r * G * 4 + (C::kScaleChunk * c + 4 * h + j) * 4);
                copy4(rsrc, off, 0u, lds_buf + 256u * (uint32_t)u);
            }
        }
    };
    // block kb's scales: the activation- and weight-scale chunks if one
    // starts there
    auto issue_scales = [&](const TileOperands &src, int kb, int st) {
        if (kb == kb0 || (kb & (C::kScaleChunk - 1)) == 0) {
            const int c = kb / C::kScaleChunk;
            const bool whole = (c + 1) * C::kScaleChunk <= G;
            const uint32_t so = (uint32_t)((c & 1) * sizeof(L.chunks.v[0]));
            if (whole) {
#pragma unroll
                for (int t = 0; t < C::kScaleLoads; ++t)
                    if (wave_u + C::kWaves * t < C::kScaleCopies)
                        copy16(src.sa, sa_voff(t), (uint32_t)c * (4u * C::kScaleChunk),
                               lds_sc0 + so + 1024 * C::kWaves * t);
            } else {
                issue_chunk_dwords(src.sa, C::BM, c, lds_addr(&L.chunks.v[0][0][0][0]) + so);
            }
            if constexpr (C::kRowScaledW) {
                const uint32_t sow = (uint32_t)((c & 1) * sizeof(L.wchunks.v[0]));
                if (whole) {
#pragma unroll
                    for (int t = 0; t < C::kScaleLoadsW; ++t)
                        if (wave_u + C::kWaves * t < C::kScaleCopiesW)
                            copy16(src.swr, swr_voff(t), (uint32_t)c * (4u * C::kScaleChunk),
                                   lds_wc0 + sow + 1024 * C::kWaves * t);
                } else {
                    issue_chunk_dwords(src.swr, C::BN, c,
                                       lds_addr(&L.wchunks.v[0][0][0][0]) + sow);
                }
            }
            // every wave fetches the chunk's weight scales to the same LDS
            // words (the duplicates carry identical values), so that every
            // wave issues the same number of copies
            if constexpr (!kSwPerBlock)
                copy4(src.sw, sw_voff(), (uint32_t)(c * C::kScaleChunk) * op.sw_kstride,
                      lds_sw0 + (uint32_t)((c & 1) * sizeof(L.swc[0])));
        }
        if constexpr (kSwPerBlock)
            copy4(src.sw, sw_voff(), (uint32_t)kb * op.sw_kstride,
                  lds_sw0 + (uint32_t)st * sizeof(L.swc[0]));
    };
    // all of block kb
    auto issue = [&](const TileOperands &src, int kb, int st) {
        issue_scales(src, kb, st);
        issue_a(src, kb, st, -1);
        issue_w(src, kb, st);
    };

    // LDS byte offsets of this lane's two 16-byte operand chunks inside a
    // 16-row tile (row lr of the tile; tiles start at multiples of 16 rows).
    const int frag0 = lr * 128 + (((2 * lk) ^ swz_key(lr)) << 4);
    const int frag1 = lr * 128 + (((2 * lk + 1) ^ swz_key(lr)) << 4);
    const int a_base = wm * C::WM * 128;
    const int b_base = wn * C::WN * 128;

    // The MFMA runs with the weight fragment as its A operand and the token
    // fragment as its B operand, so it produces the transposed 16x16 tile
    // D[n][m]: lane L holds outputs n = 4 (L / 16) + e (e < 4), m = L % 16.
    // The activation scale is then one value per lane per M tile and the
    // weight scale one value per wave (or per fragment, see kWaveInOneBlock).
    auto wfrag = [&](int s, int j) {
        if constexpr (kTransW) {
            typedef int v2i_t __attribute__((ext_vector_type(2)));
            typedef __attribute__((address_space(3))) v2i_t *lds_v2i;
            // rows 32 lk + 8 q + lr / 2 all have tw_key = (lr / 2) | (lk & 1) << 3,
            // so the four reads differ by immediate offsets 8 q BN
            // (the key passes through an empty asm statement so that the four
            // fragments' offsets are recomputed here instead of being hoisted
            // into registers held across the loop)
            const int c = (wn * C::WN + 16 * j) >> 4;
            int key = (lr >> 1) | ((lk & 1) << 3);
            asm volatile("" : "+v"(key));
            const uint8_t *p = L.stages[s].b + (32 * lk + (lr >> 1)) * C::BN + 8 * (lr & 1) +
                               (tw_phys<C::BN>(c, key) << 4);
            v2i_t r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_v2i)(lds_ptr_t)(const_cast<uint8_t *>(p + 8 * q * C::BN)));
            v8i v;
            v[0] = r[0][0]; v[1] = r[0][1]; v[2] = r[1][0]; v[3] = r[1][1];
            v[4] = r[2][0]; v[5] = r[2][1]; v[6] = r[3][0]; v[7] = r[3][1];
            return v;
        } else {
            const uint8_t *lb = L.stages[s].b + b_base;
            const uint4 lo = *reinterpret_cast<const uint4 *>(lb + j * 2048 + frag0);
            const uint4 hi = *reinterpret_cast<const uint4 *>(lb + j * 2048 + frag1);
            return make_v8i(lo, hi);
        }
    };
    // Scales of block kb (stage s): sc[i] = sa(i) * sw for waves inside one
    // weight-scale block, else sc[i] = sa(i) and swj[j] = sw(fragment j);
    // with power-of-two scales, sc[i] and swj[j] hold the E8M0 codes.  With
    // row-scaled W, sc[i] = sa(i) and swr[j][e] = the scale of W row 16 j +
    // 4 (lane / 16) + e of the wave's columns (the rows of this lane's four
    // outputs of fragment j).
    // FP32 row scales are held per output (swr) and reloaded for each block,
    // which the two-stage pipeline's early reads of the next block's scales
    // would overwrite; power-of-two row scales go to the MFMA as one code per
    // lane and fragment, like the block-scaled path's.
    static_assert(!C::kRowScaledW || kPow2 || C::kStages >= 3,
                  "FP32 row scales run the S >= 3 pipeline");
    float swr[C::kTN][4];
    auto load_scales = [&](int s, int kb, float (&sc)[C::kTM], float (&swj)[C::kTN]) {
        const int cb = (kb / C::kScaleChunk) & 1, piece = (kb >> 2) & (C::kScalePieces - 1);
        // weight scale of the tile's 128-column block nb for block kb
        auto wsc = [&](int nb) {
            if constexpr (kSwPerBlock)
                return L.swc[s][nb];
            else
                return L.swc[cb][nb * C::kScaleChunk + (kb & (C::kScaleChunk - 1))];
        };
        const float *sa_lane = &L.chunks.v[cb][piece][wm * C::WM + lr][kb & 3];
        if constexpr (C::kRowScaledW && kPow2) {
            // lane L holds row lr of W fragment j: its own row's code
            const float *sw_lane = &L.wchunks.v[cb][piece][wn * C::WN + lr][kb & 3];
#pragma unroll
            for (int i = 0; i < C::kTM; ++i) sc[i] = e8m0_code(sa_lane[64 * i]);
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) swj[j] = e8m0_code(sw_lane[64 * j]);
        } else if constexpr (C::kRowScaledW) {
            const float *sw_lane = &L.wchunks.v[cb][piece][wn * C::WN + 4 * lk][kb & 3];
#pragma unroll
            for (int i = 0; i < C::kTM; ++i) sc[i] = sa_lane[64 * i];
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) swr[j][e] = sw_lane[4 * (16 * j + e)];
        } else if constexpr (kPow2) {
#pragma unroll
            for (int i = 0; i < C::kTM; ++i) sc[i] = e8m0_code(sa_lane[64 * i]);
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) swj[j] = e8m0_code(wsc((col_off + 16 * j) >> 7));
        } else if constexpr (C::kWaveInOneBlock) {
            const float swv = wsc(col_off >> 7);
#pragma unroll
            for (int i = 0; i < C::kTM; ++i) sc[i] = sa_lane[64 * i] * swv;
        } else {
#pragma unroll
            for (int i = 0; i < C::kTM; ++i) sc[i] = sa_lane[64 * i];
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) swj[j] = wsc((col_off + 16 * j) >> 7);
        }
    };
    // Weight fragments and scales of the block being computed.  With two
    // stages they are already in registers when a block starts: the previous
    // block reloads each W fragment from the other stage right after its last
    // MFMA on it, and reads the next block's scales during its last row.
    v8i wfr[C::kTN];
    float sc[C::kTM], swj[C::kTN];
    v8i af_carry;  // two stages: the next block's first token fragment
    auto afrag_at = [&](int s, int i) {
        const uint8_t *la = L.stages[s].a + a_base;
        const uint4 lo = *reinterpret_cast<const uint4 *>(la + i * 2048 + frag0);
        const uint4 hi = *reinterpret_cast<const uint4 *>(la + i * 2048 + frag1);
        return make_v8i(lo, hi);
    };
    auto compute = [&](int s, int kb, auto &&mid, auto &&end) {
        constexpr bool kSplit = C::kStages == 2;
        const uint8_t *la = L.stages[s].a + a_base;
        if constexpr (!kSplit) {
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) wfr[j] = wfrag(s, j);
        }
        if constexpr (!kSplit) load_scales(s, kb, sc, swj);
        float sc_next[C::kTM], swj_next[C::kTN];
        // combined scale of M tile i and N fragment j: sa(i) * sw(j)
        auto scale = [&](int i, int j) {
            if constexpr (C::kWaveInOneBlock)
                return sc[i];
            else
                return sc[i] * swj[j];
        };
        auto afrag = [&](int i) {
            const uint4 lo = *reinterpret_cast<const uint4 *>(la + i * 2048 + frag0);
            const uint4 hi = *reinterpret_cast<const uint4 *>(la + i * 2048 + frag1);
            return make_v8i(lo, hi);
        };
        // The promotion of each MFMA result is issued after the next MFMA, so
        // the VALU FMAs never wait on the MFMA that produced their operand, and
        // the next A fragment is read from LDS one row of tiles ahead.
        auto promote = [&](int i, int j, const v4f &p) {
            if constexpr (C::kRowScaledW) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][j][e] = __builtin_fmaf(p[e], sc[i] * swr[j][e], acc[i][j][e]);
            } else {
                const float f = scale(i, j);
                acc[i][j][0] = __builtin_fmaf(p[0], f, acc[i][j][0]);
                acc[i][j][1] = __builtin_fmaf(p[1], f, acc[i][j][1]);
                acc[i][j][2] = __builtin_fmaf(p[2], f, acc[i][j][2]);
                acc[i][j][3] = __builtin_fmaf(p[3], f, acc[i][j][3]);
            }
        };
        v8i af;
        if constexpr (kSplit)
            af = af_carry;
        else
            af = afrag(0);
        v4f p_prev{};
        int pi = -1, pj = 0;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            // With two stages the barriers come one row early: the row's token
            // fragment is already in registers, and the next one (first of
            // the second half, or the next block's first) is read while the
            // row's MFMAs run.
            if (kSplit && i == C::kTM / 2 - 1) mid();  // second half of A in LDS from here
            if (kSplit && i == C::kTM - 1) end();      // next block's first half in LDS
            v8i af_next;
            if (i + 1 < C::kTM)
                af_next = afrag(i + 1);
            else if (kSplit)
                af_next = afrag_at(s ^ 1, 0);
            else
                af_next = af;
            if (kSplit && i == C::kTM - 1) load_scales(s ^ 1, kb + 1, sc_next, swj_next);
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) {
                if constexpr (kPow2) {
                    acc[i][j] = mfma_e4m3_scaled(wfr[j], af, acc[i][j], __float_as_int(swj[j]),
                                                 __float_as_int(sc[i]));
                    if (kSplit && i == C::kTM - 1) wfr[j] = wfrag(s ^ 1, j);  // next block's
                } else {
                    const v4f p = mfma_e4m3(wfr[j], af);
                    if (kSplit && i == C::kTM - 1) wfr[j] = wfrag(s ^ 1, j);  // next block's
                    if (pi >= 0) promote(pi, pj, p_prev);
                    p_prev = p;
                    pi = i;
                    pj = j;
                }
            }
            af = af_next;
        }
        if constexpr (!kPow2) promote(pi, pj, p_prev);
        if constexpr (kSplit) {
            af_carry = af;
#pragma unroll
            for (int i = 0; i < C::kTM; ++i) sc[i] = sc_next[i];
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) swj[j] = swj_next[j];
        }
    };

    if constexpr (C::kStages == 2) {
        // Two stages, each block's copies in two groups so that the copy pipe
        // never drains at a barrier:
        //   G1(j): the A rows of every wave's first kTM / 2 M tiles of block j;
        //   G2(j): the other A rows of block j + 1, the W tile of block j + 2
        //          and the scale chunks that start at block j + 2 (reading W
        //          transposed: and block j + 2's weight scales).
        // Block kb (stage st) runs as: rows 0 .. kTM/2 - 2; wait for G2(kb - 1)
        // (only the kG1 newer copies may stay outstanding), barrier, issue
        // G2(kb); rows kTM/2 - 1 .. kTM - 2; wait for G1(kb + 1) (kG2 newer
        // copies may stay outstanding), barrier, issue G1(kb + 2); row kTM - 1.
        // Each barrier comes one row before the data it guards is needed, so
        // the next token fragment is read while that row's MFMAs run.  In the
        // last row each W fragment of block kb + 1 (landed with G2(kb - 1)) is
        // reloaded right after its last MFMA in block kb, and block kb + 1's
        // scales and first token fragment are read.  Reuse is safe: G2(kb)
        // overwrites the other stage's second-half A rows (block kb - 1 was
        // finished before the last barrier) and this stage's W tile (read
        // into registers during block kb - 1's last row); G1(kb
        // + 2) overwrites this stage's first-half A rows (rows 0 .. kTM/2 - 1
        // of block kb are done).  Each group has one block of compute to land.
        constexpr int kAHalf = C::kALoads / 2;
        constexpr int kG1 = kAHalf;
        // G2 without a scale chunk; a chunk's copies come after the A and W
        // copies of G2, which only makes the wait for G1 stricter
        constexpr int kG2 = C::kALoads - kAHalf + C::kBLoads + (kSwPerBlock ? 1 : 0);
        static_assert((C::WM / 2) % (8 * C::kWaves) == 0 && C::kTM % 2 == 0, "split block");
        // Blocks past the end are copied from empty buffers (every lane out of
        // bounds: nothing is read, zeros land in regions no block uses) so
        // that the wait counts stay fixed and the loop body has no
        // data-dependent branches.
        TileOperands none = op;
        none.a[2] = none.w[2] = none.sa[2] = none.sw[2] = none.swr[2] = 0;
        auto src_for = [&](int kb) {
            const bool in = kb < kb1;
            TileOperands t;
            t.a = in ? op.a : none.a;
            t.w = in ? op.w : none.w;
            t.sa = in ? op.sa : none.sa;
            t.sw = in ? op.sw : none.sw;
            t.swr = in ? op.swr : none.swr;
            return t;
        };
        issue(op, kb0, 0);
        issue_w(src_for(kb0 + 1), kb0 + 1, 1);
        issue_scales(src_for(kb0 + 1), kb0 + 1, 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        issue_a(src_for(kb0 + 1), kb0 + 1, 1, 0);  // G1(kb0 + 1)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) wfr[j] = wfrag(0, j);
        load_scales(0, kb0, sc, swj);
        af_carry = afrag_at(0, 0);
        for (int kb = kb0; kb < kb1; ++kb) {
            const int st = (kb - kb0) & 1;
            compute(
                st, kb,
                [&] {
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kG1) : "memory");
                    __syncthreads();
                    issue_a(src_for(kb + 1), kb + 1, st ^ 1, 1);
                    const TileOperands next2 = src_for(kb + 2);
                    issue_w(next2, kb + 2, st);
                    issue_scales(next2, kb + 2, st);
                },
                [&] {
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kG2) : "memory");
                    __syncthreads();
                    issue_a(src_for(kb + 2), kb + 2, st, 0);  // G1(kb + 2)
                });
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        // S >= 3 stages: after the barrier of iteration kb every wave has
        // finished block kb - 1, so its stage takes block kb + D, D = S - 1;
        // before the barrier, only the copies of blocks kb + 1 .. kb + D - 1
        // may still be outstanding.
        constexpr int D = C::kStages - 1;
        for (int d = 0; d < D; ++d)
            if (kb0 + d < kb1) issue(op, kb0 + d, d);
        for (int kb = kb0; kb < kb1; ++kb) {
            const int i = kb - kb0;
            if (kb + D - 1 < kb1)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"((D - 1) * (C::kCopiesPerBlock +
                                                                (kSwPerBlock ? 1 : 0)))
                             : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (kb + D < kb1) issue(op, kb + D, (i + D) % C::kStages);
            compute(i % C::kStages, kb, [] {}, [] {});
        }
    }
}

// Writes the accumulators of one tile: rows [row0, row_end) and columns
// [n0, N) are stored.  acc[i][j] holds, for token m = 16 i + lane % 16 of the
// wave's rows, the four consecutive outputs n = 16 j + 4 (lane / 16) + e of
// the wave's columns.  Stored directly, one instruction would write 16 rows
// x 32 bytes (bf16); instead the tile goes through the (now free) LDS stages
// in row-major order and leaves in 16-byte pieces of whole rows, so that
// every store instruction writes full 128-byte lines.  Rows that do not fit
// in the stages at once (fp32 output of a 256 x 256 tile) go in passes of
// whole wave rows.  Inside an LDS row, the 32-byte piece q of row r is kept
// at piece q ^ (r % 16) (bounded by the row length; rotated by r instead
// for rows that are not a power of two long), which spreads the 16 rows a
// wave writes at once over the banks.
//
// Final outputs and split-K partials are each written once, with
// nontemporal stores (the reduction reads the partials back with
// nontemporal loads).
template <class C, int OUT, size_t kBufBytes>
__device__ __forceinline__ void tile_store_buf(const v4f (&acc)[C::kTM][C::kTN], uint8_t *buf,
                                               void *c, int64_t ldc, int64_t row0,
                                               int64_t row_end, int64_t n0, int64_t N) {
    constexpr int kOB = OUT == kOutBF16 ? 2 : 4;  // bytes per output element
    constexpr int kRB = C::BN * kOB;              // bytes per tile row
    constexpr int kFit = (int)(kBufBytes / kRB) / C::WM * C::WM;
    constexpr int kRowsPerPass = kFit < C::BM ? kFit : C::BM;
    static_assert(kRowsPerPass >= C::WM && C::BM % kRowsPerPass == 0, "store passes");
    constexpr int kPieces = kRB / 32;
    static_assert(kRB % 32 == 0, "row length");
    constexpr bool kPow2 = (kPieces & (kPieces - 1)) == 0;
    constexpr int kSwz = (kPieces < 16 ? kPieces : 16) - 1;  // XOR mask on the 32-byte piece
    // LDS byte offset of byte b of row r: the 32-byte piece b / 32 is XORed
    // (power-of-two rows) or rotated (other rows) by the row index
    auto lds_off = [](int r, int b) {
        const int q = b >> 5;
        const int qp = kPow2 ? (q ^ (r & kSwz)) : (q + r) % kPieces;
        return r * kRB + (qp << 5) + (b & 31);
    };
    constexpr int kUnitsPerRow = kRB / 16;
    constexpr int kUnits = kRowsPerPass * kUnitsPerRow;
    static_assert(kUnits % C::kThreads == 0, "store loop");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::kWavesN;
    const int wn = wave % C::kWavesN;
    const int wave_row0 = __builtin_amdgcn_readfirstlane(wm * C::WM);
#pragma unroll
    for (int pass = 0; pass < C::BM / kRowsPerPass; ++pass) {
        const int r_lo = pass * kRowsPerPass;
        __syncthreads();  // the stages (or the previous pass) are no longer read
        if (wave_row0 >= r_lo && wave_row0 < r_lo + kRowsPerPass) {
#pragma unroll
            for (int i = 0; i < C::kTM; ++i) {
                const int r = wave_row0 - r_lo + 16 * i + (lane & 15);
#pragma unroll
                for (int j = 0; j < C::kTN; ++j) {
                    const int cb = (wn * C::WN + 16 * j + 4 * (lane >> 4)) * kOB;
                    uint8_t *dst = buf + lds_off(r, cb);
                    const v4f v = acc[i][j];
                    if (OUT == kOutBF16) {
                        uint2 o;
                        o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(dst) = o;
                    } else {
                        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                    }
                }
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int u = tid; u < kUnits; u += C::kThreads) {
            const int r = u / kUnitsPerRow;
            const int cb = (u % kUnitsPerRow) * 16;
            const int64_t grow = row0 + r_lo + r;
            const int64_t gcol = n0 + cb / kOB;
            // N is a multiple of 128: a 16-byte piece is all in or all out
            if (grow < row_end && gcol < N) {
                const uint4 v = *reinterpret_cast<const uint4 *>(buf + lds_off(r, cb));
                u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<uint8_t *>(c) +
                                                       (grow * ldc + gcol) * kOB);
                const u32x4 w = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(w, dst);
            }
        }
    }
}

// The tile's LDS operand stages are free once the main loop is done and
// serve as the store buffer.
template <class C, int OUT>
__device__ __forceinline__ void tile_store(const v4f (&acc)[C::kTM][C::kTN], TileLds<C> &L,
                                           void *c, int64_t ldc, int64_t row0, int64_t row_end,
                                           int64_t n0, int64_t N) {
    tile_store_buf<C, OUT, sizeof(L.stages)>(
        acc, reinterpret_cast<uint8_t *>(&L.stages[0]), c, ldc, row0, row_end, n0, N);
}

// Tile shapes: 256 x 256 on 8 waves (wave tile 128 x 64, two LDS stages)
// for GEMMs that fill the GPU; 128 x 64 on 8 waves (wave tile 32 x 32,
// four stages: copies three K blocks ahead) for small ones, with split-K when
// even those tiles cannot occupy the 256 CUs (narrower tiles need half the
// splits, so half the partial sums, than 128 x 128 ones for the same
// occupancy); 128 x 256 on 8 waves (wave
// tile 64 x 64, three stages) for the grouped GEMM, whose experts' token
// counts make 128-row granularity worth keeping.
using BigTile = TileCfg<256, 256, 2, 4, 2>;
// 256 x 192 on 8 waves (wave tile 128 x 48): covers part of the columns
// when 256 x 256 tiles alone would leave a partly filled last round (see
// plan_two_kind).
using NarrowTile = TileCfg<256, 192, 2, 4, 2>;
// (8 waves rather than 4: the decode GEMM 256 x 2048 x 7168 took 18.2
// instead of 18.6 us one launch after a flush, 14.6 instead of 15.0 back to
// back)
using SmallTile = TileCfg<128, 64, 4, 2, 4>;
using MidTile = TileCfg<128, 256, 2, 4, 3>;
// Wgrad: both operands carry one scale per row and K block (128x1 token
// groups of dY and X, transposed).  128 x 256 tiles on 8 waves with three
// stages, and scale chunks of 4 K blocks for both operands so the W row
// chunks fit in LDS beside the stages.
using WgradTile = TileCfg<128, 256, 2, 4, 3, 1, true>;
// 128 x 192 on 8 waves (wave tile 64 x 48): covers part of the Wgrad columns
// when 128 x 256 tiles alone would leave a nearly empty last round (see
// plan_row_scaled_two_kind).  Row-scaled W has a scale per column, so a wave's
// 48 columns may straddle 128-column boundaries freely.
using WgradNarrowTile = TileCfg<128, 192, 2, 4, 3, 1, true>;
// Wgrad with power-of-two scales: the block-scaled MFMA applies each row's
// code itself and accumulates across K blocks, so no per-output scales sit
// in registers and the forward GEMM's 256 x 256 (and 256 x 192) tiles with
// two stages fit; scale chunks of 4 K blocks for both operands (128 KiB of
// stages + 2 x 8 KiB of chunks).
using WgradPow2Tile = TileCfg<256, 256, 2, 4, 2, 1, true>;
using WgradPow2NarrowTile = TileCfg<256, 192, 2, 4, 2, 1, true>;

// Logical tile index of this workgroup after the XCD remap (gridDim.x is a
// multiple of 8; each XCD gets a contiguous range of logical tiles).
__device__ __forceinline__ int xcd_logical_tile() {
    const int per = gridDim.x / kNumXcd;
    return (blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd;
}

template <class C, int OUT, bool kPow2, bool kTransW = false>
__global__ __launch_bounds__(C::kThreads) void dense_gemm_kernel(GemmParams p) {
    __shared__ TileLds<C> lds;
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
    const TileOperands op =
        kTransW ? tile_operands_transw<C>(p.a, p.sa, p.w, p.sw, row0, p.M - row0, n0, p.N - n0,
                                          p.K, p.G, p.ldw, p.NB)
                : tile_operands<C>(p.a, p.sa, p.w, p.sw, row0, p.M - row0, n0, p.N - n0, p.K,
                                   p.G);
    const int wn = (threadIdx.x >> 6) % C::kWavesN;
    tile_mainloop<C, kPow2, kTransW>(op, p.K, p.G, kb0, kb1, (int)(n0 & 127) + wn * C::WN, lds,
                                     acc);
    // Partial sums are written and read back once, both with the
    // nontemporal policy (see splitk_reduce_kernel).
    if (OUT == kOutPartial)
        tile_store<C, kOutF32>(acc, lds, p.partial + (int64_t)ks * p.M * p.N, p.N, row0, p.M,
                               n0, p.N);
    else
        tile_store<C, OUT>(acc, lds, p.c, p.N, row0, p.M, n0, p.N);
}

// One 256-row tile of the dense GEMM at (row0, n0), full K.
template <class C, int OUT, bool kPow2, bool kTransW = false>
__device__ __forceinline__ void dense_tile(const GemmParams &p, TileLds<C> &lds, int64_t row0,
                                           int64_t n0) {
    v4f acc[C::kTM][C::kTN];
    const TileOperands op =
        kTransW ? tile_operands_transw<C>(p.a, p.sa, p.w, p.sw, row0, p.M - row0, n0, p.N - n0,
                                          p.K, p.G, p.ldw, p.NB)
                : tile_operands<C>(p.a, p.sa, p.w, p.sw, row0, p.M - row0, n0, p.N - n0, p.K,
                                   p.G);
    const int wn = (threadIdx.x >> 6) % C::kWavesN;
    tile_mainloop<C, kPow2, kTransW>(op, p.K, p.G, 0, p.G, (int)(n0 & 127) + wn * C::WN, lds,
                                     acc);
    tile_store<C, OUT>(acc, lds, p.c, p.N, row0, p.M, n0, p.N);
}

// Grouped raster over a tiles_m x tiles_n grid (runs of group_m M tiles
// sweep across N).
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int group_m, int &tm,
                                       int &tn) {
    const int span = group_m * tiles_n;
    const int grp = t / span;
    const int first_m = grp * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in = t - grp * span;
    tm = first_m + in % gm;
    tn = in / gm;
}

// Tile of a two-kind plan: slots [0, per1) of each XCD take its contiguous
// share of the CB tiles (columns [0, n_split)), the rest its share of the CN
// tiles (columns [n_split, N)).  The wide tiles are dispatched first; the
// LDS union holds either layout.
template <class CB, class CN, int OUT, bool kPow2, bool kTransW = false>
__device__ __forceinline__ void two_kind_tile(const GemmParams &p, TileLds<CB> &lds_b,
                                              TileLds<CN> &lds_n) {
    static_assert(CB::kThreads == CN::kThreads && CB::BM == CN::BM, "two-kind tiles");
    const int t1 = p.tiles_m * p.tn1, t2 = p.tiles_m * p.tn2;
    const int per1 = (t1 + kNumXcd - 1) / kNumXcd, per2 = (t2 + kNumXcd - 1) / kNumXcd;
    const int xcd = blockIdx.x % kNumXcd;
    const int slot = blockIdx.x / kNumXcd;
    int tm, tn;
    if (slot < per1) {
        const int t = xcd * per1 + slot;
        if (t >= t1) return;
        raster(t, p.tiles_m, p.tn1, p.group_m, tm, tn);
        dense_tile<CB, OUT, kPow2, kTransW>(p, lds_b, (int64_t)tm * CB::BM,
                                            (int64_t)tn * CB::BN);
    } else {
        const int t = xcd * per2 + (slot - per1);
        if (slot - per1 >= per2 || t >= t2) return;
        raster(t, p.tiles_m, p.tn2, p.group_m, tm, tn);
        dense_tile<CN, OUT, kPow2, kTransW>(p, lds_n, (int64_t)tm * CN::BM,
                                            p.n_split + (int64_t)tn * CN::BN);
    }
}

// Dense GEMM with two tile widths.  When 256 x 256 tiles alone would leave
// the last round of workgroups partly filled, columns [0, n_split) are
// covered by 256 x 256 tiles and [n_split, N) by 256 x 192 tiles, chosen so
// that each kind fills whole rounds (e.g. 4096 x 7168: 256 of each, one of
// each per CU instead of two 256 x 256 tiles on 192 CUs and one on the
// rest).  Each XCD takes a contiguous share of each kind, the wide tiles
// first; the LDS holds either layout.
template <int OUT, bool kPow2, bool kTransW = false>
__global__ __launch_bounds__(BigTile::kThreads) void dense_gemm_two_kind_kernel(GemmParams p) {
    __shared__ union DenseLds {
        TileLds<BigTile> big;
        TileLds<NarrowTile> narrow;
    } lds;
    two_kind_tile<BigTile, NarrowTile, OUT, kPow2, kTransW>(p, lds.big, lds.narrow);
}

// Wgrad with 128 x 256 tiles on columns [0, n_split) and 128 x 192 tiles on
// the rest (plan_row_scaled_two_kind); with power-of-two scales, 256 x 256 and
// 256 x 192 tiles.
template <class CW, class CN, int OUT, bool kPow2>
__global__ __launch_bounds__(CW::kThreads) void wgrad_two_kind_kernel(GemmParams p) {
    __shared__ union WgradLds {
        TileLds<CW> wide;
        TileLds<CN> narrow;
    } lds;
    two_kind_tile<CW, CN, OUT, kPow2>(p, lds.wide, lds.narrow);
}

// Split-K reduction: C = sum over splits in fixed order 0..S-1, then the
// output conversion.  Four elements per thread (M*N is a multiple of 128).
// The partials are loaded eight splits at a time before any is added, so
// their latencies overlap instead of adding up; only splits that exist are
// loaded (a uniform branch per load: re-reading the last split in the unused
// slots instead cost 0.8 us of a 15.7 us decode call).  The partials are
// stored and loaded with
// the nontemporal policy: on back-to-back decode-sized calls (256 x 2048 x
// 7168 over rotating operand sets) that took a call from 18.2 to 16.2 us,
// the streamed partials no longer displacing the next call's operands in the
// caches; either half alone gained at most 1.5%.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partial,
                                                            void *__restrict__ c, int64_t MN,
                                                            int S) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;
    auto load = [&](int k) {
        const v4f t =
            __builtin_nontemporal_load(reinterpret_cast<const v4f *>(partial + (int64_t)k * MN + i));
        return make_float4(t[0], t[1], t[2], t[3]);
    };
    float4 s = load(0);
    for (int k0 = 1; k0 < S; k0 += 8) {
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (k0 + j < S) v[j] = load(k0 + j);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (k0 + j < S) {
                s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
            }
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
// offsets live on the device: the first wave scans them (64 experts per
// step), counts the real tiles R,
// gives each XCD a contiguous range of ceil(R / 8) of them (the grid is
// sized for the worst case (ceil(T / BM) + E) * tiles_n, so sizing the
// ranges by the grid would leave the last XCDs idle) and finds this tile's
// expert; surplus workgroups exit.  Expert e's rows are [lo_e, hi_e) with
// lo_e = max(clamp(off[e]), hi_{e-1}) and hi_e = max(lo_e, clamp(off[e+1])),
// clamp to [0, T]: the same as [off[e], off[e + 1]) for valid
// (non-decreasing) offsets, and disjoint ranges within [0, T] for any
// others, so the tile count never exceeds the worst case.
template <class C, int OUT, bool kPow2>
__global__ __launch_bounds__(C::kThreads) void grouped_gemm_kernel(GemmParams p) {
    __shared__ TileLds<C> lds;
    __shared__ int64_t info[4];
    if (threadIdx.x < 64) {
        // Wave 0 finds this workgroup's tile.  Expert e's rows are
        // [PM(e), PM(e + 1)) with PM(i) = max_{j <= i} clamp(off[j]): the
        // ranges above unrolled (hi_e is the running maximum of the clamped
        // offsets up to off[e + 1], and lo_e the one up to off[e]).  Lane l
        // of a chunk handles expert e0 + l: a prefix maximum across the
        // lanes gives PM, a prefix sum the tile counts before each expert.
        const int lane = threadIdx.x;
        const int T = (int)p.M;
        const int E = p.E;
        auto clamped = [&](int i) {
            const int v = p.offsets[i];
            return v < 0 ? 0 : (v > T ? T : v);
        };
        struct Chunk {
            int lo, hi, incl, own;  // expert rows [lo, hi); tiles up to and of this expert
        };
        auto chunk = [&](int e0, int carry_hi) {
            const int e = e0 + lane;
            Chunk c;
            c.hi = e < E ? clamped(e + 1) : 0;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int t = __shfl_up(c.hi, d);
                if (lane >= d) c.hi = t > c.hi ? t : c.hi;
            }
            c.hi = carry_hi > c.hi ? carry_hi : c.hi;
            c.lo = __shfl_up(c.hi, 1);
            if (lane == 0) c.lo = carry_hi;
            c.own = e < E ? (c.hi - c.lo + C::BM - 1) / C::BM * p.tiles_n : 0;
            c.incl = c.own;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int t = __shfl_up(c.incl, d);
                if (lane >= d) c.incl += t;
            }
            return c;
        };
        const int pm0 = E > 0 ? clamped(0) : 0;
        Chunk first{};
        int total = 0;
        {
            int carry = pm0;
            for (int e0 = 0; e0 < E; e0 += 64) {
                const Chunk c = chunk(e0, carry);
                if (e0 == 0) first = c;
                total += __shfl(c.incl, 63);
                carry = __shfl(c.hi, 63);
            }
        }
        const int per = (total + kNumXcd - 1) / kNumXcd;
        const int slot = (int)blockIdx.x / kNumXcd;
        const int rem = ((int)blockIdx.x % kNumXcd) * per + slot;
        int64_t e_hit = -1, r0 = 0, r1 = 0, tn = 0;
        if (slot < per && rem < total) {
            int carry = pm0, base = 0;
            for (int e0 = 0; e0 < E; e0 += 64) {
                const Chunk c = e0 == 0 ? first : chunk(e0, carry);
                const int r = rem - base;
                const unsigned long long hit =
                    __ballot(c.own > 0 && r >= c.incl - c.own && r < c.incl);
                if (hit) {
                    const int h = __builtin_ctzll(hit);
                    const int lo = __shfl(c.lo, h), hi = __shfl(c.hi, h);
                    const int local = r - (__shfl(c.incl, h) - __shfl(c.own, h));
                    const int mt = (hi - lo + C::BM - 1) / C::BM;
                    e_hit = e0 + h;
                    tn = local / mt;
                    r0 = lo + (int64_t)(local - tn * mt) * C::BM;
                    r1 = hi;
                    break;
                }
                base += __shfl(c.incl, 63);
                carry = __shfl(c.hi, 63);
            }
        }
        if (lane == 0) {
            info[0] = e_hit;
            info[1] = r0;
            info[2] = r1;
            info[3] = tn;
        }
    }
    __syncthreads();
    const int64_t e = info[0];
    if (e < 0) return;
    const int64_t row0 = info[1], row_end = info[2];
    const int64_t n0 = info[3] * C::BN;

    const uint8_t *w = p.w + e * p.N * p.K;
    const float *sw = p.sw + e * (int64_t)p.NB * p.G;
    v4f acc[C::kTM][C::kTN];
    const TileOperands op =
        tile_operands<C>(p.a, p.sa, w, sw, row0, row_end - row0, n0, p.N - n0, p.K, p.G);
    const int wn = (threadIdx.x >> 6) % C::kWavesN;
    tile_mainloop<C, kPow2>(op, p.K, p.G, 0, p.G, (int)(n0 & 127) + wn * C::WN, lds, acc);
    tile_store<C, OUT>(acc, lds, p.c, p.N, row0, row_end, n0, p.N);
}


// ---- Activation quantization fused into the GEMM ---------------------------
//
// The standalone quantizer reads 128 BF16 values per group from HBM, writes
// the FP8 bytes back, and the GEMM reads them again (page "why-be.co.kr
// as_center 36949", passage on that round trip and on fusing the FP8 cast
// with the transfer of activations from global memory).  This kernel takes
// the bf16 activations itself: each K block's bf16 A tile is copied to LDS,
// quantized there (the 1x128 rule of the standalone quantizer, with the same
// arithmetic, so the bytes and scales are identical) into the E4M3 tile the
// MFMAs read, and the scale goes straight into the promotion.  Optionally
// the workgroups of the first N tile also write the bytes and scales out.
//
// The cost moves from HBM to the VALU: every N tile quantizes its A tile
// again (N / 256 times in all), and A comes in at 2 bytes per element.  It
// pays where few N tiles share an A tile; where many do, the standalone
// quantizer plus the plain GEMM is faster.
//
// Tile 64 x 256 on 8 waves (2 x 4, wave tile 32 x 64).  Per K block each
// wave copies 8 bf16 rows (two 1 KiB copies) and a quarter of the W tile; it
// quantizes exactly the 8 rows it copied, so the bf16 tile needs no barrier.
// Pipeline: bf16 A, streamed from HBM, in three stages (copies two blocks
// ahead of their quantization, which runs one block ahead of the MFMAs); W,
// re-read by every M tile and mostly an L2 hit, in two stages (one block
// ahead); E4M3 A and its scales double buffered.
// When the tiles alone would not fill the CUs, K is split over workgroups
// as in the plain GEMM (partials in the caller's workspace, then the fixed-
// order reduction).
struct FusedCfg {
    static constexpr int BM = 64, BN = 256;
    static constexpr int kWavesM = 2, kWavesN = 4, kWaves = 8, kThreads = 512;
    static constexpr int WM = BM / kWavesM, WN = BN / kWavesN;
    static constexpr int kTM = WM / 16, kTN = WN / 16;
    static constexpr int kStagesW = 2, kStagesA = 3;
    static constexpr int kWLoads = BN / 8 / kWaves;            // 8 rows of 128 B per copy
    static constexpr int kALoads = BM * 256 / 1024 / kWaves;   // 4 rows of 256 B per copy
    static_assert(kALoads == 2, "each wave copies the 8 bf16 rows it quantizes");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns in one weight-scale block");
};

struct __align__(4096) FusedLds {
    uint8_t w[FusedCfg::kStagesW][FusedCfg::BN * 128];
    uint8_t a16[FusedCfg::kStagesA][FusedCfg::BM * 256];
    uint8_t a8[2][FusedCfg::BM * 128];  // swizzled like Stage::a
    float sa[2][FusedCfg::BM];
    // weight scales in chunks of 8 K blocks, as in TileLds: buffer b holds
    // at word 8 nb + j the scale of column block nb for K block 8 c + j
    float swc[2][64];
};

template <int OUT>
__global__ __launch_bounds__(FusedCfg::kThreads) void fused_quant_gemm_kernel(GemmParams p) {
    using C = FusedCfg;
    __shared__ FusedLds L;
    const int logical = xcd_logical_tile();
    if (logical >= p.ntiles) return;
    const int per_split = p.tiles_m * p.tiles_n;
    const int ks = logical / per_split;
    int tm, tn;
    raster(logical - ks * per_split, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int64_t K = p.K;
    const int G = p.G;
    const int kb0 = ks * p.kb_per_split;
    const int kb1 = min(kb0 + p.kb_per_split, G);
    const int64_t row0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t ra = p.M - row0 < C::BM ? p.M - row0 : C::BM;
    const int64_t cw = p.N - n0 < C::BN ? p.N - n0 : C::BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::kWavesN, wn = wave % C::kWavesN;
    const int lr = lane & 15, lk = lane >> 4;
    const bool write_q = p.q_out != nullptr && tn == 0;

    const v4i rx = make_rsrc(p.x + row0 * K, (uint32_t)(ra * K * 2));
    const v4i rw = make_rsrc(p.w + n0 * K, (uint32_t)(cw * K));
    const int64_t nb0 = n0 >> 7, nbs = ((n0 + cw - 1) >> 7) - nb0 + 1;
    const v4i rsw = make_rsrc(p.sw + nb0 * G, (uint32_t)(nbs * G * 4));
    v4i rx0 = rx, rw0 = rw;  // empty views for blocks past the end
    rx0[2] = rw0[2] = 0;

    // W copy t of wave v fills W-stage rows 8 (v + 8 t) .. + 8 (as in
    // tile_mainloop: lane L -> physical chunk L % 8 of row L / 8, holding
    // logical chunk (L % 8) ^ key(row)).
    const uint32_t w_voff = (uint32_t)(8 * wave * K + (lane >> 3) * K +
                                       (((lane & 7) ^ ((lane >> 3) & 7) ^ (wave & 1)) << 4));
    const uint32_t w_rowstep = (uint32_t)(64 * K);
    // bf16 copy t of wave v: rows 4 (v + 8 t) + L / 16, 16-byte chunk L % 16
    // (1 KiB of the stage from byte 1024 (v + 8 t)).
    const uint32_t a_voff = (uint32_t)((4 * wave + (lane >> 4)) * 2 * K + (lane & 15) * 16);
    const uint32_t a_rowstep = (uint32_t)(32 * 2 * K);
    const uint32_t lds_w0 = lds_addr(&L.w[0][1024 * wave]);
    const uint32_t lds_a0 = lds_addr(&L.a16[0][1024 * wave]);
    const uint32_t lds_sw0 = lds_addr(&L.swc[0][0]);
    const uint32_t sw_voff = (uint32_t)((lane >> 3) * G * 4 + (lane & 7) * 4);

    // bf16 A of block k (this wave's 8 rows); the W tile of block k, and the
    // weight-scale chunk starting at block k if one does (at the split's
    // first block and every 8 blocks).  A and W of blocks past the split
    // read from empty views.  The loop's waits leave only the newest bf16
    // copies outstanding, so the chunk copies need no count of their own;
    // the prologue's wait counts the chunk that starts at the split's first
    // block.
    auto issue_a = [&](int k) {
        const bool in = k < kb1;
        const v4i &a_r = in ? rx : rx0;
        const int kc = in ? k : kb0;
        const uint32_t a_st = (uint32_t)((k % C::kStagesA) * sizeof(L.a16[0]));
#pragma unroll
        for (int t = 0; t < C::kALoads; ++t)
            copy16(a_r, a_voff + t * a_rowstep, (uint32_t)kc * 256u,
                   lds_a0 + a_st + 1024u * C::kWaves * t);
    };
    auto issue_w = [&](int k) {
        const bool in = k < kb1;
        const v4i &w_r = in ? rw : rw0;
        const int kc = in ? k : kb0;
        const uint32_t w_st = (uint32_t)((k % C::kStagesW) * sizeof(L.w[0]));
#pragma unroll
        for (int t = 0; t < C::kWLoads; ++t)
            copy16_nt(w_r, w_voff + t * w_rowstep, (uint32_t)kc * 128u,
                      lds_w0 + w_st + 1024u * C::kWaves * t);
        // (none past the split: such a copy would land in a buffer that the
        // split's last chunk may still occupy)
        if (in && (k == kb0 || (k & 7) == 0))
            copy4(rsw, sw_voff, (uint32_t)(k & ~7) * 4u,
                  lds_sw0 + (uint32_t)(((k >> 3) & 1) * sizeof(L.swc[0])));
    };

    // Quantize block kb from its bf16 stage (this wave's 8 rows) into E4M3
    // buffer kb % 2 and its scales; rows past M quantize to zero bytes.
    auto quant = [&](int kb) {
#pragma unroll
        for (int t = 0; t < C::kALoads; ++t) {
            const int r = 4 * (wave + C::kWaves * t) + (lane >> 4), j = lane & 15;
            const bool in = row0 + r < p.M;
            const uint4 v = *reinterpret_cast<const uint4 *>(
                &L.a16[kb % C::kStagesA][r * 256 + j * 16]);
            float f[8];
            unpack8(v, f);
            const float amax = row16_max(absmax8(f));
            float y[8], s;
            if (__all(!in || amax >= 0x1p-60f)) {
                s = in ? scale_fast(amax) : 1.0f;
                const float rc = 1.0f / s;
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = quot_fast(f[i], s, rc);
            } else {
                const QuotientCtx qc(amax, false);
                s = qc.s;
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = qc(f[i]);
            }
            if (!in) s = 0.0f;
            uint32_t lo = 0, hi = 0;
            lo = cvt_pk_e4m3<false>(y[0], y[1], lo);
            lo = cvt_pk_e4m3<true>(y[2], y[3], lo);
            hi = cvt_pk_e4m3<false>(y[4], y[5], hi);
            hi = cvt_pk_e4m3<true>(y[6], y[7], hi);
            const int chunk = (j >> 1) ^ swz_key(r);
            *reinterpret_cast<uint2 *>(&L.a8[kb & 1][r * 128 + chunk * 16 + (j & 1) * 8]) =
                make_uint2(lo, hi);
            if (j == 0) L.sa[kb & 1][r] = s;
            if (write_q && in) {
                *reinterpret_cast<uint2 *>(p.q_out + (row0 + r) * K + (int64_t)kb * 128 + 8 * j) =
                    make_uint2(lo, hi);
                if (j == 0) p.sa_out[(row0 + r) * G + kb] = s;
            }
        }
    };

    const int frag0 = lr * 128 + (((2 * lk) ^ swz_key(lr)) << 4);
    const int frag1 = lr * 128 + (((2 * lk + 1) ^ swz_key(lr)) << 4);
    const int col_off = (int)(n0 & 127) + wn * C::WN;
    v4f acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Block kb: W stage kb % 2, E4M3 A buffer kb % 2.  The MFMA takes the
    // weight fragment as its A operand, so lane L holds outputs n = 4 (L /
    // 16) + e, m = L % 16 of each 16 x 16 tile (see tile_mainloop).
    auto compute = [&](int kb) {
        const uint8_t *lw = L.w[kb % C::kStagesW] + wn * C::WN * 128;
        const uint8_t *la = L.a8[kb & 1] + wm * C::WM * 128;
        v8i wfr[C::kTN];
#pragma unroll
        for (int j = 0; j < C::kTN; ++j)
            wfr[j] = make_v8i(*reinterpret_cast<const uint4 *>(lw + j * 2048 + frag0),
                              *reinterpret_cast<const uint4 *>(lw + j * 2048 + frag1));
        const float swv = L.swc[(kb >> 3) & 1][(col_off >> 7) * 8 + (kb & 7)];
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            const v8i af = make_v8i(*reinterpret_cast<const uint4 *>(la + i * 2048 + frag0),
                                    *reinterpret_cast<const uint4 *>(la + i * 2048 + frag1));
            const float f = L.sa[kb & 1][wm * C::WM + 16 * i + lr] * swv;
            v4f pr[C::kTN];
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) pr[j] = mfma_e4m3(wfr[j], af);
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(pr[j][e], f, acc[i][j][e]);
        }
    };

    // Prologue: bf16 A of block kb0, W and scales of block kb0, bf16 A of
    // blocks kb0 + 1 and kb0 + 2; block kb0's rows are quantized by the wave
    // that copied them (no barrier needed) once its two copies have landed.
    issue_a(kb0);
    issue_w(kb0);
    issue_a(kb0 + 1);
    issue_a(kb0 + 2);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::kWLoads + 1 + 2 * C::kALoads) : "memory");
    quant(kb0);
    for (int kb = kb0; kb < kb1; ++kb) {
        // Iteration kb - 1 issued W(kb), its scales, then bf16 A(kb + 2):
        // with only A(kb + 2) outstanding, W(kb) and the older A(kb + 1)
        // have landed.
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::kALoads) : "memory");
        __syncthreads();
        // W stage (kb + 1) % 2 was last read by block kb - 1 and bf16 stage
        // (kb + 3) % 3 held block kb's rows, quantized in the previous
        // iteration (every wave is past both)
        issue_w(kb + 1);
        issue_a(kb + 3);
        compute(kb);
        if (kb + 1 < kb1) quant(kb + 1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (p.ksplit > 1)
        tile_store_buf<C, kOutF32, sizeof(L.w)>(acc, &L.w[0][0],
                                                 p.partial + (int64_t)ks * p.M * p.N, p.N, row0,
                                                 p.M, n0, p.N);
    else
        tile_store_buf<C, OUT, sizeof(L.w)>(acc, &L.w[0][0], p.c, p.N, row0, p.M, n0, p.N);
}

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

constexpr int kCUs = 256;

struct Plan {
    bool big;
    int ksplit;
    int kb_per_split;
    int tn1 = 0, tn2 = 0;  // two-kind plan (big only): 256-wide and 192-wide N tiles
};

// Two-kind plan for 256-row tiles: tn1 256-wide N tiles then tn2 192-wide
// ones, used when both kinds fill whole rounds of the CUs and the estimated
// time (a 256 x 192 tile costs ~0.85 of a 256 x 256 one: its copies are 7/8
// and its MFMAs 3/4) beats whole-width tiles.  Returns false if none does.
bool plan_two_kind(int64_t M, int64_t N, int &tn1, int &tn2) {
    const int64_t tm = (M + 255) / 256;
    const int64_t tn_big = (N + 255) / 256;
    const double base = (double)((tm * tn_big + kCUs - 1) / kCUs);
    double best = base;
    bool found = false;
    for (int64_t a = 0; a <= N / 256; ++a) {
        const int64_t rest = N - 256 * a;
        const int64_t b = (rest + 191) / 192;
        if (b == 0 || (tm * a) % kCUs != 0 || (tm * b) % kCUs != 0) continue;
        const double cost = (double)(tm * a / kCUs) + 0.85 * (double)(tm * b / kCUs);
        if (cost < best - 1e-9) {
            best = cost;
            tn1 = (int)a;
            tn2 = (int)b;
            found = true;
        }
    }
    return found;
}

// Wgrad column split: 128 x 256 tiles on columns [0, 256 a), 128 x 192
// tiles on the rest (the last one possibly ragged).  With 56 row tiles (7168
// rows) neither kind can fill whole rounds, so the split is chosen by
// modelling the dispatch: each XCD's 32 CUs take its share of wide tiles
// first, then its narrow ones, each tile going to the CU that is free first;
// a narrow tile costs kWgradNarrowCost of a wide one.  The busiest XCD (the
// first, whose shares are the largest) sets the finishing time.  A split is
// used when it finishes at least 3% before the wide tiles alone: for
// dW 7168 x 7168, a = 16 and b = 16 model at 6.46 wide-tile times against 7.
constexpr double kWgradNarrowCost = 0.82;
// The same model for the power-of-two Wgrad's 256 x 256 and 256 x 192 tiles,
// whose narrow tile costs ~0.85 of a wide one (as in plan_two_kind): for dW
// 7168 x 7168, a = 4 and b = 32 model at 3.55 wide-tile times against 4.
constexpr double kWgradPow2NarrowCost = 0.85;

// Finishing time of one XCD, in wide-tile times.  After the wide tiles, the
// 32 - rem CUs holding q of them are free at q, the rem CUs holding q + 1 at
// q + 1.  Each narrow tile goes to the CU free first, so the narrow tiles end
// level by level: all CUs of the first group at q + r, q + 2r, ..., those
// of the second at q + 1 + r, ..., merged in time order.
double xcd_finish(int64_t wide, int64_t narrow, double r) {
    constexpr int kCUsPerXcd = kCUs / kNumXcd;
    const int64_t q = wide / kCUsPerXcd, rem = wide % kCUsPerXcd;
    double end = (double)(q + (rem ? 1 : 0));
    int64_t left = narrow, k_lo = 1, k_hi = 1;
    while (left > 0) {
        const double t_lo = (double)q + (double)k_lo * r;
        const double t_hi = (double)(q + 1) + (double)k_hi * r;
        if (rem == 0 || t_lo <= t_hi) {
            left -= kCUsPerXcd - rem;
            end = t_lo > end ? t_lo : end;
            ++k_lo;
        } else {
            left -= rem;
            end = t_hi > end ? t_hi : end;
            ++k_hi;
        }
    }
    return end;
}

// CW: the wide tile, CN: the narrow one (same rows), r: the narrow tile's
// cost in wide-tile times.
template <class CW, class CN>
bool plan_row_scaled_two_kind(int64_t M, int64_t N, double r, int &tn1, int &tn2) {
    static_assert(CW::BM == CN::BM, "two-kind tiles");
    // the same shapes come back every training step (one cache per tile pair)
    thread_local int64_t last_m = -1, last_n = -1;
    thread_local int last_a = 0, last_b = 0;
    if (M == last_m && N == last_n) {
        tn1 = last_a;
        tn2 = last_b;
        return last_b > 0;
    }
    const int64_t tm = (M + CW::BM - 1) / CW::BM;
    const int64_t tn_wide = (N + CW::BN - 1) / CW::BN;
    const double base = xcd_finish((tm * tn_wide + kNumXcd - 1) / kNumXcd, 0, r);
    double best = 0.97 * base;
    int best_a = (int)tn_wide, best_b = 0;
    // a grid of at most one round of wide tiles finishes in one tile time
    // either way
    const int64_t a_end = tm * tn_wide > kCUs ? (N + CW::BN - 1) / CW::BN : 0;
    for (int64_t a = 0; a < a_end; ++a) {
        const int64_t rest = N - CW::BN * a;
        if (rest <= 0) break;
        const int64_t b = (rest + CN::BN - 1) / CN::BN;
        const double t = xcd_finish((tm * a + kNumXcd - 1) / kNumXcd,
                                    (tm * b + kNumXcd - 1) / kNumXcd, r);
        if (t < best) {
            best = t;
            best_a = (int)a;
            best_b = (int)b;
        }
    }
    last_m = M;
    last_n = N;
    last_a = tn1 = best_a;
    last_b = tn2 = best_b;
    return best_b > 0;
}

Plan plan_dense(int64_t M, int64_t N, int64_t K) {
    const int G = (int)(K / 128);
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (big_tiles >= kCUs) {
        Plan pl{true, 1, G};
        int a, b;
        if (plan_two_kind(M, N, a, b)) {
            pl.tn1 = a;
            pl.tn2 = b;
        }
        return pl;
    }
    const int64_t tiles = ((M + SmallTile::BM - 1) / SmallTile::BM) * ((N + SmallTile::BN - 1) / SmallTile::BN);
    int s = 1;
    // Split K only when the output tiles cannot fill the CUs and each split
    // keeps at least 4 K blocks.
    while (tiles * s * 2 <= kCUs && G / (s * 2) >= 4) s *= 2;
    const int per = (G + s - 1) / s;
    s = (G + per - 1) / per;
    return {false, s, per};
}

// With FP8BLK_LOG set in the environment (to anything but "" or "0"), every
// GEMM call prints the plan it launches, one line on stderr: the entry, the
// output and inner sizes, the tile shapes, the K splits and the grid.
bool plan_log_on() {
    static const bool on = [] {
        const char *v = getenv("FP8BLK_LOG");
        return v != nullptr && *v != 0 && strcmp(v, "0") != 0;
    }();
    return on;
}

void log_plan(const char *entry, int64_t M, int64_t N, int64_t K, const char *tiles, int tn1,
              int tn2, int ksplit, int grid) {
    if (!plan_log_on()) return;
    if (tn2 > 0)
        fprintf(stderr,
                "fp8blk: %s M=%lld N=%lld K=%lld tiles=%s (%d + %d column tiles) ksplit=%d "
                "grid=%d\n",
                entry, (long long)M, (long long)N, (long long)K, tiles, tn1, tn2, ksplit, grid);
    else
        fprintf(stderr, "fp8blk: %s M=%lld N=%lld K=%lld tiles=%s ksplit=%d grid=%d\n", entry,
                (long long)M, (long long)N, (long long)K, tiles, ksplit, grid);
}

// Plan of the dense GEMM family (forward and Dgrad) for the log line.
void log_dense_plan(const char *entry, const GemmParams &p, const Plan &pl) {
    if (!plan_log_on()) return;
    if (pl.big && pl.tn2 > 0) {
        const int tm = (int)((p.M + 255) / 256);
        const int grid = kNumXcd * ((tm * pl.tn1 + kNumXcd - 1) / kNumXcd +
                                    (tm * pl.tn2 + kNumXcd - 1) / kNumXcd);
        log_plan(entry, p.M, p.N, p.K, "256x256+256x192", pl.tn1, pl.tn2, 1, grid);
    } else if (pl.big) {
        const int t = (int)(((p.M + 255) / 256) * ((p.N + 255) / 256));
        log_plan(entry, p.M, p.N, p.K, "256x256", 0, 0, 1, round_up(t, kNumXcd));
    } else {
        const int t = (int)(((p.M + SmallTile::BM - 1) / SmallTile::BM) *
                            ((p.N + SmallTile::BN - 1) / SmallTile::BN));
        log_plan(entry, p.M, p.N, p.K, pl.ksplit > 1 ? "128x64 split-K + reduction" : "128x64", 0,
                 0, pl.ksplit, round_up(t * pl.ksplit, kNumXcd));
    }
}

template <class C, int OUT, bool kPow2, bool kTransW = false>
hipError_t launch_dense(const GemmParams &p0, hipStream_t stream) {
    GemmParams p = p0;
    p.tiles_m = (int)((p.M + C::BM - 1) / C::BM);
    p.tiles_n = (int)((p.N + C::BN - 1) / C::BN);
    p.ntiles = p.tiles_m * p.tiles_n * p.ksplit;
    const int grid = round_up(p.ntiles, kNumXcd);
    hipLaunchKernelGGL((dense_gemm_kernel<C, OUT, kPow2, kTransW>), dim3(grid),
                       dim3(C::kThreads), 0, stream, p);
    return hipGetLastError();
}

// Launches the planned dense GEMM for one output type and scale mode.
template <int OUT, bool kPow2>
hipError_t block_gemm(GemmParams p, const Plan &pl, void *c, hipStream_t stream) {
    if (pl.big && pl.tn2 > 0) {
        p.tiles_m = (int)((p.M + 255) / 256);
        p.tn1 = pl.tn1;
        p.tn2 = pl.tn2;
        p.n_split = (int64_t)pl.tn1 * BigTile::BN;
        const int per1 = (p.tiles_m * p.tn1 + kNumXcd - 1) / kNumXcd;
        const int per2 = (p.tiles_m * p.tn2 + kNumXcd - 1) / kNumXcd;
        const int grid = kNumXcd * (per1 + per2);
        hipLaunchKernelGGL((dense_gemm_two_kind_kernel<OUT, kPow2>), dim3(grid),
                           dim3(BigTile::kThreads), 0, stream, p);
        return hipGetLastError();
    }
    if (pl.big) return launch_dense<BigTile, OUT, kPow2>(p, stream);
    if (p.ksplit > 1) {
        hipError_t e = launch_dense<SmallTile, kOutPartial, kPow2>(p, stream);
        if (e != hipSuccess) return e;
        const int64_t MN = p.M * p.N;
        const int64_t blocks = (MN / 4 + 255) / 256;
        hipLaunchKernelGGL(splitk_reduce_kernel<OUT>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           p.partial, c, MN, p.ksplit);
        return hipGetLastError();
    }
    return launch_dense<SmallTile, OUT, kPow2>(p, stream);
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
                             void *workspace, size_t workspace_bytes, bool pow2,
                             hipStream_t stream) {
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
    p.partial = static_cast<float *>(workspace);
    log_dense_plan(pow2 ? "block_gemm_pow2" : "block_gemm", p, pl);
    if (pow2)
        return bf16_out ? block_gemm<kOutBF16, true>(p, pl, c, stream)
                        : block_gemm<kOutF32, true>(p, pl, c, stream);
    return bf16_out ? block_gemm<kOutBF16, false>(p, pl, c, stream)
                    : block_gemm<kOutF32, false>(p, pl, c, stream);
}

namespace {

// Wgrad on the tile pair CW (wide) / CN (narrow): the two-kind plan when
// it beats wide tiles alone, else wide tiles.
template <class CW, class CN, bool kPow2>
hipError_t launch_wgrad(GemmParams &p, bool bf16_out, double narrow_cost, const char *entry,
                        const char *kinds, const char *wide, hipStream_t stream) {
    int tn1, tn2;
    if (plan_row_scaled_two_kind<CW, CN>(p.M, p.N, narrow_cost, tn1, tn2)) {
        p.tiles_m = (int)((p.M + CW::BM - 1) / CW::BM);
        p.tn1 = tn1;
        p.tn2 = tn2;
        p.n_split = (int64_t)tn1 * CW::BN;
        const int per1 = (p.tiles_m * tn1 + kNumXcd - 1) / kNumXcd;
        const int per2 = (p.tiles_m * tn2 + kNumXcd - 1) / kNumXcd;
        const dim3 grid((unsigned)(kNumXcd * (per1 + per2)));
        log_plan(entry, p.M, p.N, p.K, kinds, tn1, tn2, 1, (int)grid.x);
        if (bf16_out)
            hipLaunchKernelGGL((wgrad_two_kind_kernel<CW, CN, kOutBF16, kPow2>), grid,
                               dim3(CW::kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((wgrad_two_kind_kernel<CW, CN, kOutF32, kPow2>), grid,
                               dim3(CW::kThreads), 0, stream, p);
        return hipGetLastError();
    }
    log_plan(entry, p.M, p.N, p.K, wide, 0, 0, 1,
             round_up((int)(((p.M + CW::BM - 1) / CW::BM) * ((p.N + CW::BN - 1) / CW::BN)),
                      kNumXcd));
    return bf16_out ? launch_dense<CW, kOutBF16, kPow2>(p, stream)
                    : launch_dense<CW, kOutF32, kPow2>(p, stream);
}

}  // namespace

hipError_t launch_block_gemm_wgrad(const void *a, const float *sa, const void *b,
                                   const float *sb, void *c, bool bf16_out, int64_t M, int64_t N,
                                   int64_t K, bool pow2, hipStream_t stream) {
    GemmParams p{};
    p.a = static_cast<const uint8_t *>(a);
    p.sa = sa;
    p.w = static_cast<const uint8_t *>(b);
    p.sw = sb;
    p.c = c;
    p.M = M;
    p.N = N;
    p.K = K;
    p.G = (int)(K / 128);
    p.NB = (int)(N / 128);
    p.group_m = 8;
    p.ksplit = 1;
    p.kb_per_split = p.G;
    if (pow2)
        return launch_wgrad<WgradPow2Tile, WgradPow2NarrowTile, true>(
            p, bf16_out, kWgradPow2NarrowCost, "block_gemm_wgrad_pow2", "256x256+256x192",
            "256x256", stream);
    return launch_wgrad<WgradTile, WgradNarrowTile, false>(
        p, bf16_out, kWgradNarrowCost, "block_gemm_wgrad", "128x256+128x192", "128x256", stream);
}

hipError_t launch_grouped_gemm(const void *a, const float *sa, const void *w, const float *sw,
                               const int32_t *offsets, int64_t E, int64_t T, void *c,
                               bool bf16_out, int64_t N, int64_t K, bool pow2,
                               hipStream_t stream) {
    using C = MidTile;
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
    const dim3 grid(round_up(p.ntiles, kNumXcd));
    log_plan(pow2 ? "block_grouped_gemm_pow2" : "block_grouped_gemm", T, N, K,
             "128x256 (tiles found on the device; grid sized for the worst case)", 0, 0, 1,
             (int)grid.x);
    if (pow2) {
        if (bf16_out)
            hipLaunchKernelGGL((grouped_gemm_kernel<C, kOutBF16, true>), grid, dim3(C::kThreads),
                               0, stream, p);
        else
            hipLaunchKernelGGL((grouped_gemm_kernel<C, kOutF32, true>), grid, dim3(C::kThreads),
                               0, stream, p);
    } else {
        if (bf16_out)
            hipLaunchKernelGGL((grouped_gemm_kernel<C, kOutBF16, false>), grid, dim3(C::kThreads),
                               0, stream, p);
        else
            hipLaunchKernelGGL((grouped_gemm_kernel<C, kOutF32, false>), grid, dim3(C::kThreads),
                               0, stream, p);
    }
    return hipGetLastError();
}

namespace {

// K splits of the fused GEMM: as for the plain GEMM's small tiles, doubled
// while the tiles times the splits still fit in the CUs and each split keeps
// at least 4 K blocks.
int fused_ksplit(int64_t M, int64_t N, int64_t K) {
    using C = FusedCfg;
    const int G = (int)(K / 128);
    const int64_t tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
    int s = 1;
    while (tiles * s * 2 <= kCUs && G / (s * 2) >= 4) s *= 2;
    const int per = (G + s - 1) / s;
    return (G + per - 1) / per;
}

}  // namespace

size_t fused_quant_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const int s = fused_ksplit(M, N, K);
    if (s <= 1) return 0;
    return (size_t)s * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_block_gemm_fused_quant(const void *x, const void *w, const float *sw, void *c,
                                         bool bf16_out, int64_t M, int64_t N, int64_t K,
                                         void *q_out, float *sa_out, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    using C = FusedCfg;
    GemmParams p{};
    p.x = static_cast<const uint16_t *>(x);
    p.w = static_cast<const uint8_t *>(w);
    p.sw = sw;
    p.c = c;
    p.q_out = static_cast<uint8_t *>(q_out);
    p.sa_out = sa_out;
    p.M = M;
    p.N = N;
    p.K = K;
    p.G = (int)(K / 128);
    p.NB = (int)(N / 128);
    p.tiles_m = (int)((M + C::BM - 1) / C::BM);
    p.tiles_n = (int)((N + C::BN - 1) / C::BN);
    int s = fused_ksplit(M, N, K);
    if (s > 1 && (workspace == nullptr || workspace_bytes < fused_quant_workspace_bytes(M, N, K)))
        s = 1;
    p.ksplit = s;
    p.kb_per_split = (p.G + s - 1) / s;
    p.partial = static_cast<float *>(workspace);
    p.ntiles = p.tiles_m * p.tiles_n * s;
    p.group_m = 8;
    const dim3 grid(round_up(p.ntiles, kNumXcd));
    log_plan("block_gemm_fused_quant", M, N, K,
             s > 1 ? "64x256 split-K + reduction" : "64x256", 0, 0, s, (int)grid.x);
    if (bf16_out)
        hipLaunchKernelGGL(fused_quant_gemm_kernel<kOutBF16>, grid, dim3(C::kThreads), 0, stream,
                           p);
    else
        hipLaunchKernelGGL(fused_quant_gemm_kernel<kOutF32>, grid, dim3(C::kThreads), 0, stream,
                           p);
    if (s > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t MN = M * N;
        const int64_t blocks = (MN / 4 + 255) / 256;
        if (bf16_out)
            hipLaunchKernelGGL(splitk_reduce_kernel<kOutBF16>, dim3((unsigned)blocks), dim3(256),
                               0, stream, p.partial, c, MN, s);
        else
            hipLaunchKernelGGL(splitk_reduce_kernel<kOutF32>, dim3((unsigned)blocks), dim3(256),
                               0, stream, p.partial, c, MN, s);
    }
    return hipGetLastError();
}

// Dgrad, dX [M][Kx] = dY [M][N] W [N][Kx]: the block GEMM with dY as the
// activations (inner dimension N) and W read transposed from its forward
// layout; the same plan as fp8_block_gemm for an M x Kx output over N
// (256 x 256 tiles, or 128 x 64 tiles with split-K for small M).
namespace {

// Launches the planned Dgrad (W read transposed) for one output type and
// scale mode: the forward GEMM's plans (see block_gemm).
template <int OUT, bool kPow2>
hipError_t dgrad_gemm(GemmParams p, const Plan &pl, void *dx, hipStream_t stream) {
    if (pl.big && pl.tn2 > 0) {
        // the forward GEMM's two tile widths
        p.tiles_m = (int)((p.M + 255) / 256);
        p.tn1 = pl.tn1;
        p.tn2 = pl.tn2;
        p.n_split = (int64_t)pl.tn1 * BigTile::BN;
        const int per1 = (p.tiles_m * p.tn1 + kNumXcd - 1) / kNumXcd;
        const int per2 = (p.tiles_m * p.tn2 + kNumXcd - 1) / kNumXcd;
        const int grid = kNumXcd * (per1 + per2);
        hipLaunchKernelGGL((dense_gemm_two_kind_kernel<OUT, kPow2, true>), dim3(grid),
                           dim3(BigTile::kThreads), 0, stream, p);
        return hipGetLastError();
    }
    if (pl.big) return launch_dense<BigTile, OUT, kPow2, true>(p, stream);
    if (p.ksplit > 1) {
        hipError_t e = launch_dense<SmallTile, kOutPartial, kPow2, true>(p, stream);
        if (e != hipSuccess) return e;
        const int64_t MN = p.M * p.N;
        const int64_t blocks = (MN / 4 + 255) / 256;
        hipLaunchKernelGGL(splitk_reduce_kernel<OUT>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           p.partial, dx, MN, p.ksplit);
        return hipGetLastError();
    }
    return launch_dense<SmallTile, OUT, kPow2, true>(p, stream);
}

}  // namespace

hipError_t launch_block_gemm_dgrad(const void *dy, const float *sdy, const void *w,
                                   const float *sw, void *dx, bool bf16_out, int64_t M,
                                   int64_t N, int64_t Kx, void *workspace, size_t workspace_bytes,
                                   bool pow2, hipStream_t stream) {
    GemmParams p{};
    p.a = static_cast<const uint8_t *>(dy);
    p.sa = sdy;
    p.w = static_cast<const uint8_t *>(w);
    p.sw = sw;
    p.c = dx;
    p.M = M;
    p.N = Kx;
    p.K = N;
    p.G = (int)(N / 128);
    p.NB = (int)(Kx / 128);
    p.ldw = Kx;
    p.group_m = 8;
    Plan pl = plan_dense(M, Kx, N);
    const size_t need = gemm_workspace_bytes(M, Kx, N);
    if (pl.ksplit > 1 && (workspace == nullptr || workspace_bytes < need)) pl = {false, 1, p.G};
    p.ksplit = pl.ksplit;
    p.kb_per_split = pl.kb_per_split;
    p.partial = static_cast<float *>(workspace);
    log_dense_plan(pow2 ? "block_gemm_dgrad_pow2 (W read transposed)"
                        : "block_gemm_dgrad (W read transposed)",
                   p, pl);
    if (pow2)
        return bf16_out ? dgrad_gemm<kOutBF16, true>(p, pl, dx, stream)
                        : dgrad_gemm<kOutF32, true>(p, pl, dx, stream);
    return bf16_out ? dgrad_gemm<kOutBF16, false>(p, pl, dx, stream)
                    : dgrad_gemm<kOutF32, false>(p, pl, dx, stream);
}

}  // namespace fp8blk


