// Host-side launchers behind the C ABI (argument checking happens in abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8blk {

// pow2: scales are the smallest powers of two >= amax / 448 (at least
// 2^-126) instead of amax / 448 itself.
hipError_t launch_quant_act_1x128(const void *x, int64_t M, int64_t K, void *q, float *scales,
                                  bool pow2, hipStream_t stream);

hipError_t launch_quant_weight_128x128(const void *w, int64_t N, int64_t K, void *q,
                                       float *scales, bool pow2, hipStream_t stream);

// 128x1 tiles (128 rows of one column) of x [M][K], written transposed:
// q_t [K][M], scales_t [K][ceil(M/128)].
hipError_t launch_quant_act_128x1_t(const void *x, int64_t M, int64_t K, void *q_t,
                                    float *scales_t, bool pow2, hipStream_t stream);

// E4M3 weights [N][K] with 128x128 block scales [ceil(N/128)][ceil(K/128)],
// transposed: q_t [K][N], scales_t [ceil(K/128)][ceil(N/128)].
hipError_t launch_transpose_weight(const void *q, const float *s, int64_t N, int64_t K,
                                   void *q_t, float *s_t, hipStream_t stream);

// Bytes of fp32 split-K partials the dense GEMM would use for this shape
// (0 when it runs without splitting K).
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

// C[M][N] = sum_kb sa[m][kb] sb[n][kb] sum_{k in kb} a[m][k] b[n][k]: one
// scale per row and K block on both operands (the Wgrad GEMM).
// pow2: every scale is a power of two, applied by the block-scaled MFMA.
hipError_t launch_block_gemm_wgrad(const void *a, const float *sa, const void *b,
                                   const float *sb, void *c, bool bf16_out, int64_t M, int64_t N,
                                   int64_t K, bool pow2, hipStream_t stream);

// pow2: every scale is a power of two, applied by the block-scaled MFMA.
hipError_t launch_block_gemm(const void *a, const float *sa, const void *w, const float *sw,
                             void *c, bool bf16_out, int64_t M, int64_t N, int64_t K,
                             void *workspace, size_t workspace_bytes, bool pow2,
                             hipStream_t stream);

// fp8_block_gemm with its split-K partials in the library's static device
// scratch array (noalloc_scratch_bytes() of it) instead of a workspace.
size_t noalloc_scratch_bytes();
hipError_t launch_block_gemm_noalloc(const void *a, const float *sa, const void *w,
                                     const float *sw, void *c, bool bf16_out, int64_t M,
                                     int64_t N, int64_t K, hipStream_t stream);

// The block-scaled GEMM on bf16 activations x [M][K], quantized 1x128 inside
// the GEMM; q_out / sa_out (both or neither) receive the E4M3 bytes and
// scales the standalone quantizer would write.  K is split over workgroups
// (partials in the workspace) when the workspace holds
// fused_quant_workspace_bytes(M, N, K).
size_t fused_quant_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_block_gemm_fused_quant(const void *x, const void *w, const float *sw, void *c,
                                         bool bf16_out, int64_t M, int64_t N, int64_t K,
                                         void *q_out, float *sa_out, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

// Dgrad dX [M][Kx] = dY [M][N] W [N][Kx], W E4M3 with 128x128 block scales
// [N/128][Kx/128] in its forward layout, read transposed in LDS.
// pow2: every scale is a power of two, applied by the block-scaled MFMA.
hipError_t launch_block_gemm_dgrad(const void *dy, const float *sdy, const void *w,
                                   const float *sw, void *dx, bool bf16_out, int64_t M,
                                   int64_t N, int64_t Kx, void *workspace, size_t workspace_bytes,
                                   bool pow2, hipStream_t stream);

hipError_t launch_grouped_gemm(const void *a, const float *sa, const void *w, const float *sw,
                               const int32_t *offsets, int64_t E, int64_t T, void *c,
                               bool bf16_out, int64_t N, int64_t K, bool pow2,
                               hipStream_t stream);

}  // namespace fp8blk
