/*
 * fp8blk — fine-grained FP8 quantization and block-scaled FP8 GEMM for
 * MI355X (gfx950).  C ABI.
 *
 * The method (page "dssusan.co.kr qna 93378", passage on Figure 7 (a) and the
 * passages that follow it):
 *   - activations are grouped and scaled per token per 128 channels (1x128
 *     tiles); weights per 128 input channels x 128 output channels (128x128
 *     blocks);
 *   - E4M3 is used for every FP8 tensor;
 *   - the per-group scaling factors run along the GEMM inner dimension K and
 *     are multiplied into the FP32 partial sums as the dequantization step
 *     (page "kailasan.com recruit 147436", passage on promotion, Figure 7 (b));
 *   - the GEMMs take FP8 operands and produce BF16 or FP32.
 * Readings where the pages are silent: OCP E4M3FN (largest finite 448), scale
 * s = fl32(amax / 448) per group, code = E4M3 round-to-nearest-even of
 * fl32(x / s), all-zero group -> s = 0 and zero bytes, promotion after every
 * 128-deep K block (one scale group).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronizes.  bf16 data is passed as raw 16-bit
 *     patterns, E4M3 data as bytes, scales as IEEE binary32.
 *   - All tensors are dense and row-major.
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously.  Device faults surface at the caller's
 *     next synchronization on that stream.
 *   - Arguments are validated before anything is enqueued; on any error
 *     nothing is written.  One exception: a split-K GEMM is two launches,
 *     and if the second (the reduction into C) fails with FP8_ERR_HIP the
 *     first may already be enqueued and write its partial sums into the
 *     workspace; C is then not written.  No C++ exception crosses this
 *     boundary.
 *   - Calls are reentrant and thread-safe (concurrent calls on different
 *     streams must not share output or workspace buffers), with one
 *     exception: fp8_block_gemm_noalloc.  The library's mutable state is
 *     small and internal: a per-thread cache of the last Wgrad tile plan
 *     (fp8_block_gemm_wgrad; the same shapes recur every step), and, for
 *     fp8_block_gemm_noalloc, a static device scratch array per GPU with a
 *     mutex-guarded table of its device addresses.
 *   - Sizes of zero (M = 0, T = 0, K = 0 for the quantizers) are valid no-ops.
 *   - Inputs must be finite; NaN/Inf inputs are outside the contract and are
 *     not checked.
 *   - Diagnostics: with the environment variable FP8BLK_LOG set (to anything
 *     but "" or "0") when the library first launches a GEMM, every GEMM call
 *     prints the plan it launches on stderr (entry, sizes, tile shapes, K
 *     splits, grid).  The variable is read once per process.
 */
#ifndef FP8BLK_H_
#define FP8BLK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8_OK = 0,
    FP8_ERR_NULL = 1,      /* a required pointer is NULL */
    FP8_ERR_SHAPE = 2,     /* negative size, or a GEMM size not a multiple of 128 */
    FP8_ERR_ALIGN = 3,     /* a GEMM operand pointer is not 16-byte aligned */
    FP8_ERR_DTYPE = 4,     /* out_dtype is not one of fp8_out_dtype */
    FP8_ERR_WORKSPACE = 5, /* workspace NULL with a nonzero size, or not 256-byte aligned */
    FP8_ERR_HIP = 6        /* a HIP launch failed (hipGetLastError after the launch) */
} fp8_status;

typedef enum { FP8_OUT_F32 = 0, FP8_OUT_BF16 = 1 } fp8_out_dtype;

/*
 * 1x128 activation quantization (page "dssusan.co.kr qna 93378", Figure 7 (a):
 * one scale per token per 128 channels; page "why-be.co.kr as_center 36949",
 * passage on the quantization round trip: 128 BF16 values in, FP8 out).
 *   x_bf16  [M][K] bf16, input
 *   q_e4m3  [M][K] E4M3 bytes, output
 *   scales  [M][ceil(K/128)] fp32, output; scales[m][g] = fl32(amax/448) of
 *           channels [128g, min(128g+128, K)) of token m
 * Any M, K >= 0 and any alignment (a partial last group holds K % 128
 * channels).  Errors: FP8_ERR_NULL (a pointer NULL while M*K > 0),
 * FP8_ERR_SHAPE (M or K negative), FP8_ERR_HIP.
 */
fp8_status fp8_quant_act_1x128(const void *x_bf16, int64_t M, int64_t K,
                               void *q_e4m3, float *scales, void *hip_stream);

/*
 * 128x128 weight block quantization (page "dssusan.co.kr qna 93378",
 * Figure 7 (a): one scale per 128 input x 128 output channels).
 *   w_bf16  [N][K] bf16 (row n = output channel), input
 *   q_e4m3  [N][K] E4M3 bytes, output
 *   scales  [ceil(N/128)][ceil(K/128)] fp32, output
 * Any N, K >= 0; edge blocks hold what remains.  A stack of E expert
 * matrices [E][N][K] with N % 128 == 0 is quantized as one [E*N][K] call.
 * Errors as for fp8_quant_act_1x128.
 */
fp8_status fp8_quant_weight_128x128(const void *w_bf16, int64_t N, int64_t K,
                                    void *q_e4m3, float *scales,
                                    void *hip_stream);

/*
 * Block-scaled FP8 GEMM (page "dssusan.co.kr qna 93378", passages on scaling
 * along the inner dimension K and on FP8-in / BF16-or-FP32-out GEMMs; page
 * "kailasan.com recruit 147436", Figure 7 (b): scaled partial sums added into
 * FP32 accumulators):
 *   C[m][n] = sum_kb a_scales[m][kb] * w_scales[n/128][kb]
 *                    * sum_{k in block kb} a[m][k] * w[n][k]
 *   a_e4m3    [M][K] E4M3, a_scales [M][K/128] fp32
 *   w_e4m3    [N][K] E4M3, w_scales [N/128][K/128] fp32
 *   c         [M][N], fp32 (FP8_OUT_F32) or bf16 by round-to-nearest-even of
 *             the fp32 accumulator (FP8_OUT_BF16)
 * K % 128 == 0, N % 128 == 0 and K < 2^24 are required (FP8_ERR_SHAPE
 * otherwise; a tile's operand rows are addressed with 32-bit offsets);
 * a_e4m3, w_e4m3 and c must be 16-byte aligned (FP8_ERR_ALIGN).  M may be
 * anything >= 0.
 *   workspace / workspace_bytes: optional caller-owned device scratch
 *   (256-byte aligned).  fp8_gemm_workspace_bytes() gives the size that
 *   enables the split-K path for small M; with less (or NULL and 0) the
 *   kernel runs without it.  Its contents need no initialization and are
 *   undefined afterwards.
 * Accumulation is FP32 in a fixed order: results are deterministic for a
 * given shape and workspace size.
 */
fp8_status fp8_block_gemm(const void *a_e4m3, const float *a_scales,
                          const void *w_e4m3, const float *w_scales, void *c,
                          int out_dtype, int64_t M, int64_t N, int64_t K,
                          void *workspace, size_t workspace_bytes,
                          void *hip_stream);

/*
 * Grouped (MoE) block-scaled FP8 GEMM over expert-sorted tokens (page
 * "kailasan.com recruit 147436", passage on the decoding stage: each expert
 * sees a small batch of tokens and only its own parameters are loaded).
 *   a_e4m3        [T][K] E4M3, rows sorted by expert; a_scales [T][K/128]
 *   w_e4m3        [E][N][K] E4M3; w_scales [E][N/128][K/128]
 *   group_offsets [E+1] int32 on the DEVICE: rows [off[e], off[e+1]) belong
 *                 to expert e for valid (non-decreasing) offsets.  Any others
 *                 are made safe: offsets are clamped to [0, T] and expert e's
 *                 range starts no earlier than expert e-1's ends (an empty
 *                 range if that is past its end), so ranges never overlap.
 *                 The host never reads them.
 *   c             [T][N] fp32 or bf16; rows outside every expert's range are
 *                 left untouched.
 * Each routed row r of expert e gets C[r] = block GEMM of (a[r], W[e]).
 * Requirements and errors as fp8_block_gemm, plus FP8_ERR_SHAPE for E <= 0
 * while T > 0.  The workspace is accepted for interface symmetry and unused.
 */
fp8_status fp8_block_grouped_gemm(const void *a_e4m3, const float *a_scales,
                                  const void *w_e4m3, const float *w_scales,
                                  const int32_t *group_offsets, int64_t E,
                                  int64_t T, void *c, int out_dtype, int64_t N,
                                  int64_t K, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/*
 * fp8_block_gemm on bf16 activations, with their 1x128 quantization fused
 * into the GEMM (page "why-be.co.kr as_center 36949", passages on the
 * quantization round trip through HBM, 128 BF16 values read and FP8 written
 * back to be read again, and on fusing the FP8 cast with the transfer of
 * activations from global memory):
 *   C = fp8_block_gemm(q, s, w_e4m3, w_scales) with (q, s) =
 *       fp8_quant_act_1x128(x_bf16), without q and s passing through memory.
 *   x_bf16        [M][K] bf16, 16-byte aligned
 *   w_e4m3, w_scales, c, out_dtype, M, N, K: as fp8_block_gemm
 *   q_e4m3_out    [M][K] E4M3 (8-byte aligned) and a_scales_out [M][K/128]
 *                 fp32: optional outputs (both NULL, or both given), which
 *                 receive exactly what fp8_quant_act_1x128 writes, e.g. to
 *                 keep the FP8 activations for the backward pass.
 *   workspace / workspace_bytes: optional (256-byte aligned); it selects
 *                 the plan:
 *     - workspace_bytes >= fp8_fused_quant_workspace_bytes(): the faster plan
 *       for the shape.  The fused kernel (quantization inside the GEMM, K
 *       split over workgroups when the output tiles alone would not fill
 *       the GPU) for C one 256-column tile wide (N <= 256) over at least
 *       2048 tokens; elsewhere, where every further 256-column tile would
 *       quantize its rows again, the staged plan: fp8_quant_act_1x128 into
 *       q_e4m3_out / a_scales_out (or into the workspace when they are NULL
 *       or q_e4m3_out is not 16-byte aligned), then fp8_block_gemm with its
 *       split-K partials in the workspace.
 *     - less (or NULL and 0): the fused kernel, with K split when
 *       workspace_bytes >= fp8_fused_quant_kernel_workspace_bytes() > 0.
 * The quantized values, the products and the accumulation are those of the
 * two-call path, so C is the same up to the FP32 summation order (bitwise
 * the same where both calls run the same K splits, e.g. both without a
 * workspace, and always under the staged plan).  Errors: as fp8_block_gemm,
 * plus FP8_ERR_NULL when only one of q_e4m3_out / a_scales_out is given, and
 * FP8_ERR_ALIGN for x_bf16 not 16-byte or q_e4m3_out not 8-byte aligned.
 * The staged plan enqueues two kernels; FP8_ERR_HIP from the second leaves
 * the first enqueued.
 */
fp8_status fp8_block_gemm_fused_quant(const void *x_bf16, const void *w_e4m3,
                                      const float *w_scales, void *c, int out_dtype,
                                      int64_t M, int64_t N, int64_t K, void *q_e4m3_out,
                                      float *a_scales_out, void *workspace,
                                      size_t workspace_bytes, void *hip_stream);

/*
 * Power-of-two-scale variants for the block-scaled matrix core (page
 * "kailasan.com recruit 147436", passage recommending that matrix units take
 * the per-group scaling factors and do the group-scaled MMA themselves; on
 * gfx950 V_MFMA_SCALE_F32_16X16X128_F8F6F4 takes one E8M0 power-of-two
 * scale per operand row and 32-deep K quarter).  The pages fix no rule for
 * power-of-two scales; the one used here: s = the smallest power of two
 * with 448 s >= amax, and at least 2^-126, so every scale is a normal fp32
 * power of two whose exponent field is its E8M0 code; code = E4M3
 * round-to-nearest-even of x / s (exact division); an all-zero group stores
 * s = 2^-126 and zero bytes.  Layouts, sizes and errors are those of
 * fp8_quant_act_1x128 / fp8_quant_weight_128x128.
 */
fp8_status fp8_quant_act_1x128_pow2(const void *x_bf16, int64_t M, int64_t K,
                                    void *q_e4m3, float *scales,
                                    void *hip_stream);
fp8_status fp8_quant_weight_128x128_pow2(const void *w_bf16, int64_t N,
                                         int64_t K, void *q_e4m3,
                                         float *scales, void *hip_stream);

/*
 * fp8_block_gemm / fp8_block_grouped_gemm with every scale a power of two
 * (as the _pow2 quantizers write them).  The same C is computed, but each
 * K block's product is scaled and added into the FP32 accumulators by the
 * matrix core itself (one block-scaled MFMA per 16x16 tile and K block), so
 * there is no separate promotion step.  Only the scales' exponent fields
 * are used: a scale with nonzero mantissa bits, or outside [2^-126, 2^127],
 * gives a result computed with its exponent alone (not checked).  Arguments,
 * layouts, workspace and errors are those of the plain entry points.
 */
fp8_status fp8_block_gemm_pow2(const void *a_e4m3, const float *a_scales,
                               const void *w_e4m3, const float *w_scales,
                               void *c, int out_dtype, int64_t M, int64_t N,
                               int64_t K, void *workspace,
                               size_t workspace_bytes, void *hip_stream);
fp8_status fp8_block_grouped_gemm_pow2(const void *a_e4m3,
                                       const float *a_scales,
                                       const void *w_e4m3,
                                       const float *w_scales,
                                       const int32_t *group_offsets,
                                       int64_t E, int64_t T, void *c,
                                       int out_dtype, int64_t N, int64_t K,
                                       void *workspace,
                                       size_t workspace_bytes,
                                       void *hip_stream);

/*
 * Backward pass (page "dssusan.co.kr qna 93378", passages on FP8 in Fprop,
 * Dgrad and Wgrad with E4M3 on every tensor, on keeping activations in FP8
 * for the Wgrad GEMM, and on per-group scales along each GEMM's inner
 * dimension; page "why-be.co.kr as_center 36949", passage recommending
 * transposed reads of matrices before the MMA).  The grouping along the
 * transposed axis is a reading:
 *   - Dgrad, dX[m][k] = sum_n dY[m][n] W[n][k]: dY is quantized in 1x128
 *     tiles along N by fp8_quant_act_1x128; W keeps its 128x128 blocks and is
 *     read transposed, so dX = fp8_block_gemm(dY, W^T) with W^T from
 *     fp8_transpose_weight_128x128 (once per weight update).
 *   - Wgrad, dW[n][k] = sum_m dY[m][n] X[m][k]: the sum runs over tokens, so
 *     dY and X are quantized in 128x1 tiles (128 tokens of one channel) and
 *     written transposed by fp8_quant_act_128x1_t; fp8_block_gemm_wgrad
 *     multiplies the two with one scale per row and K block on both.
 */

/*
 * 128x1 tiles written transposed.
 *   x_bf16    [M][K] bf16, input
 *   q_t       [K][M] E4M3 bytes, output: q_t[k][m] is the code of x[m][k]
 *   scales_t  [K][ceil(M/128)] fp32, output: scales_t[k][g] = fl32(amax/448)
 *             of x[m][k] for m in [128g, min(128g+128, M))
 * Quantization rule, sizes, alignment and errors as fp8_quant_act_1x128
 * (a partial last group holds M % 128 rows).
 */
fp8_status fp8_quant_act_128x1_t(const void *x_bf16, int64_t M, int64_t K,
                                 void *q_t, float *scales_t, void *hip_stream);

/*
 * Transpose of 128x128-quantized weights (for Dgrad).
 *   q_e4m3    [N][K] E4M3, scales [ceil(N/128)][ceil(K/128)] fp32, inputs
 *   q_t       [K][N] E4M3, scales_t [ceil(K/128)][ceil(N/128)] fp32, outputs
 * Any N, K >= 0.  Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_HIP.
 */
fp8_status fp8_transpose_weight_128x128(const void *q_e4m3,
                                        const float *scales, int64_t N,
                                        int64_t K, void *q_t, float *scales_t,
                                        void *hip_stream);

/*
 * Wgrad GEMM on 128x1-grouped operands (as fp8_quant_act_128x1_t writes
 * them):
 *   dw[n][k] = sum_g dy_t_scales[n][g] * x_t_scales[k][g]
 *                    * sum_{m in [128g, 128g+128)} dy_t[n][m] * x_t[k][m]
 *   dy_t [N][T] E4M3, dy_t_scales [N][T/128]; x_t [K][T] E4M3,
 *   x_t_scales [K][T/128]; dw [N][K] fp32 or bf16 (RNE), overwritten.
 * T % 128 == 0, T < 2^24 and K % 128 == 0 are required (FP8_ERR_SHAPE;
 * pad the token axis with zero rows before quantizing), N may be anything
 * >= 0; dy_t,
 * x_t and dw must be 16-byte aligned (FP8_ERR_ALIGN).  FP32 accumulation in
 * a fixed order: deterministic.
 */
fp8_status fp8_block_gemm_wgrad(const void *dy_t, const float *dy_t_scales,
                                const void *x_t, const float *x_t_scales,
                                void *dw, int out_dtype, int64_t N, int64_t K,
                                int64_t T, void *hip_stream);

/*
 * The backward pair with power-of-two scales (the rule of the _pow2
 * quantizers above, on the matrix core's block-scaled MFMA; page
 * "kailasan.com recruit 147436", passage on matrix units taking the
 * per-group scaling factors themselves).
 *   fp8_quant_act_128x1_t_pow2: fp8_quant_act_128x1_t with each 128x1
 *     group's scale the smallest power of two s with 448 s >= amax (at least
 *     2^-126; an all-zero group stores 2^-126 and zero bytes).
 *   fp8_block_gemm_wgrad_pow2: fp8_block_gemm_wgrad on such operands.  Each
 *     operand row's E8M0 code goes to the MFMA with that row, and the MFMA
 *     accumulates the scaled K blocks in FP32 itself, so no per-output
 *     scales are held and the tiles are 256 rows tall (the FP32-scale Wgrad
 *     uses 128).  Only the scales' exponent fields are read: a scale that is
 *     not a power of two gives a result computed with its exponent alone
 *     (not checked).
 * Arguments, layouts, requirements and errors are those of the plain entry
 * points.
 */
fp8_status fp8_quant_act_128x1_t_pow2(const void *x_bf16, int64_t M, int64_t K,
                                      void *q_t, float *scales_t,
                                      void *hip_stream);
fp8_status fp8_block_gemm_wgrad_pow2(const void *dy_t, const float *dy_t_scales,
                                     const void *x_t, const float *x_t_scales,
                                     void *dw, int out_dtype, int64_t N,
                                     int64_t K, int64_t T, void *hip_stream);

/*
 * fp8_block_gemm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, layouts, results and errors are those of fp8_block_gemm with no
 * workspace argument: where fp8_block_gemm would split K through a
 * workspace (fp8_gemm_workspace_bytes() > 0), this call puts the split-K
 * partial sums in a static device array of FP8_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends, and it
 * gives bitwise the same C as fp8_block_gemm with a workspace of
 * fp8_gemm_workspace_bytes().  It calls no allocator.
 *   - Shapes whose split-K partials would exceed FP8_NOALLOC_SCRATCH_BYTES
 *     are rejected with FP8_ERR_WORKSPACE (with the current tile plans none
 *     does: a plan splits at most 256 workgroups of 128 x 64 outputs).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (on different streams or host threads) race and give
 *     undefined results.  Calls on one stream are ordered and safe.
 *   - The array's device address is looked up (hipGetSymbolAddress) the
 *     first time a GPU is used; an error there returns FP8_ERR_HIP.
 */
#define FP8_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
fp8_status fp8_block_gemm_noalloc(const void *a_e4m3, const float *a_scales,
                                  const void *w_e4m3, const float *w_scales, void *c,
                                  int out_dtype, int64_t M, int64_t N, int64_t K,
                                  void *hip_stream);

/*
 * Dgrad on the forward layout of the weights, read transposed inside the
 * GEMM (page "why-be.co.kr as_center 36949", passage recommending that
 * matrices be read transposed from shared memory before the MMA; gfx950's
 * ds_read_b64_tr_b8 does that): no transposed copy of W is needed.
 *   dX[m][k] = sum_nb dy_scales[m][nb] * w_scales[nb][k/128]
 *                    * sum_{n in block nb} dy[m][n] * w[n][k]
 *   dy_e4m3 [M][N] E4M3 with dy_scales [M][N/128] (fp8_quant_act_1x128 of dY)
 *   w_e4m3  [N][K] E4M3 with w_scales [N/128][K/128]: the forward weights as
 *           fp8_quant_weight_128x128 wrote them (row n = output channel of
 *           the forward layer); a 128x128 block's scale serves both
 *           orientations
 *   dx      [M][K] fp32 or bf16 (RNE)
 * N % 128 == 0, K % 128 == 0, N < 2^24 and N * K < 2^32 are required
 * (FP8_ERR_SHAPE); dy_e4m3, w_e4m3 and dx 16-byte aligned (FP8_ERR_ALIGN).
 * workspace: as fp8_block_gemm for an M x K output over N, i.e. of
 * fp8_gemm_workspace_bytes(M, K, N, out_dtype) bytes for the split-K path.
 * Results equal fp8_block_gemm(dy, W^T) with W^T from
 * fp8_transpose_weight_128x128 up to the FP32 summation order.
 */
fp8_status fp8_block_gemm_dgrad(const void *dy_e4m3, const float *dy_scales,
                                const void *w_e4m3, const float *w_scales, void *dx,
                                int out_dtype, int64_t M, int64_t N, int64_t K,
                                void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * fp8_block_gemm_dgrad with every scale a power of two (dY from
 * fp8_quant_act_1x128_pow2, W from fp8_quant_weight_128x128_pow2): the
 * block-scaled MFMA applies the scales' E8M0 codes and accumulates each K
 * block itself, as in fp8_block_gemm_pow2.  Only the scales' exponent fields
 * are read.  Arguments, layouts, workspace and errors are those of
 * fp8_block_gemm_dgrad; results equal fp8_block_gemm_pow2(dy, W^T) bit for
 * bit where both run the same K splits.
 */
fp8_status fp8_block_gemm_dgrad_pow2(const void *dy_e4m3, const float *dy_scales,
                                     const void *w_e4m3, const float *w_scales, void *dx,
                                     int out_dtype, int64_t M, int64_t N, int64_t K,
                                     void *workspace, size_t workspace_bytes,
                                     void *hip_stream);

/* Workspace bytes that let fp8_block_gemm use its split-K path for this
 * shape (0 when the shape does not use it). */
size_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int out_dtype);

/* Workspace bytes with which fp8_block_gemm_fused_quant takes the faster
 * plan for this shape: the fused kernel's split-K partials (0 if it does not
 * split), or for the staged plan the E4M3 activations, their scales and
 * fp8_block_gemm's partials, each part rounded up to 256 bytes. */
size_t fp8_fused_quant_workspace_bytes(int64_t M, int64_t N, int64_t K, int out_dtype);

/* Workspace bytes that let the fused kernel itself split K for this shape
 * whenever fp8_block_gemm_fused_quant runs it (its 64 x 256 tiles, and so
 * its splits, differ from fp8_block_gemm's; 0 when it does not split).  On
 * shapes that prefer the staged plan the call runs the fused kernel only
 * with fewer than fp8_fused_quant_workspace_bytes() bytes, which may or may
 * not leave room for these partials. */
size_t fp8_fused_quant_kernel_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                              int out_dtype);

/* Static, human-readable name of a status code. */
const char *fp8_status_string(fp8_status s);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H_ */
