// C ABI of fp8blk: argument validation, then dispatch to the launchers.
// Every check runs before anything is enqueued; on error nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8blk.h"
#include "launch.hpp"

namespace {

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline fp8_status from_hip(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_HIP; }

inline hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// Limits of the kernels' grid arithmetic: any one size below 2^31, a tensor
// below 2^40 elements, a GEMM below 2^30 output tiles of 128 x 128.
constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int64_t kMaxTiles = (int64_t)1 << 30;
// GEMM inner dimension: a tile's 256 operand rows of K bytes are addressed
// through one buffer resource, whose byte range and offsets are 32-bit, so
// 256 K < 2^32.
constexpr int64_t kMaxInner = (int64_t)1 << 24;

fp8_status check_quant(const void *x, int64_t R, int64_t K, const void *q, const float *s) {
    if (R < 0 || K < 0) return FP8_ERR_SHAPE;
    if (R == 0 || K == 0) return FP8_OK;
    if (!x || !q || !s) return FP8_ERR_NULL;
    if (R >= kMaxDim || K >= kMaxDim || R * K >= kMaxElems) return FP8_ERR_SHAPE;
    return FP8_OK;
}

fp8_status check_gemm_common(const void *a, const float *sa, const void *w, const float *sw,
                             const void *c, int out_dtype, int64_t rows, int64_t N, int64_t K,
                             const void *ws, size_t ws_bytes) {
    if (out_dtype != FP8_OUT_F32 && out_dtype != FP8_OUT_BF16) return FP8_ERR_DTYPE;
    if (rows < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
    if (N % 128 != 0 || K % 128 != 0) return FP8_ERR_SHAPE;
    if (rows >= kMaxDim || N >= kMaxDim || K >= kMaxInner) return FP8_ERR_SHAPE;
    if (rows * K >= kMaxElems || rows * N >= kMaxElems) return FP8_ERR_SHAPE;
    if (((rows + 127) / 128 + 1) * (N / 128) >= kMaxTiles) return FP8_ERR_SHAPE;
    if ((ws == nullptr) != (ws_bytes == 0)) return FP8_ERR_WORKSPACE;
    if (ws && !aligned(ws, 256)) return FP8_ERR_WORKSPACE;
    if (rows == 0 || N == 0) return FP8_OK;
    if (!a || !sa || !w || !sw || !c) return FP8_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(c, 16)) return FP8_ERR_ALIGN;
    if (!aligned(sa, 4) || !aligned(sw, 4)) return FP8_ERR_ALIGN;
    return FP8_OK;
}

fp8_status quant_act(const void *x_bf16, int64_t M, int64_t K, void *q_e4m3, float *scales,
                     bool pow2, void *hip_stream) {
    fp8_status st = check_quant(x_bf16, M, K, q_e4m3, scales);
    if (st != FP8_OK || M == 0 || K == 0) return st;
    if (!aligned(x_bf16, 2) || !aligned(scales, 4)) return FP8_ERR_ALIGN;
    return from_hip(fp8blk::launch_quant_act_1x128(x_bf16, M, K, q_e4m3, scales, pow2,
                                                   as_stream(hip_stream)));
}

fp8_status quant_weight(const void *w_bf16, int64_t N, int64_t K, void *q_e4m3, float *scales,
                        bool pow2, void *hip_stream) {
    fp8_status st = check_quant(w_bf16, N, K, q_e4m3, scales);
    if (st != FP8_OK || N == 0 || K == 0) return st;
    if (!aligned(w_bf16, 2) || !aligned(scales, 4)) return FP8_ERR_ALIGN;
    return from_hip(fp8blk::launch_quant_weight_128x128(w_bf16, N, K, q_e4m3, scales, pow2,
                                                        as_stream(hip_stream)));
}

fp8_status block_gemm(const void *a_e4m3, const float *a_scales, const void *w_e4m3,
                      const float *w_scales, void *c, int out_dtype, int64_t M, int64_t N,
                      int64_t K, void *workspace, size_t workspace_bytes, bool pow2,
                      void *hip_stream) {
    fp8_status st = check_gemm_common(a_e4m3, a_scales, w_e4m3, w_scales, c, out_dtype, M, N, K,
                                      workspace, workspace_bytes);
    if (st != FP8_OK || M == 0 || N == 0) return st;
    if (K == 0) return FP8_ERR_SHAPE;
    return from_hip(fp8blk::launch_block_gemm(a_e4m3, a_scales, w_e4m3, w_scales, c,
                                              out_dtype == FP8_OUT_BF16, M, N, K, workspace,
                                              workspace_bytes, pow2, as_stream(hip_stream)));
}

fp8_status grouped_gemm(const void *a_e4m3, const float *a_scales, const void *w_e4m3,
                        const float *w_scales, const int32_t *group_offsets, int64_t E,
                        int64_t T, void *c, int out_dtype, int64_t N, int64_t K, void *workspace,
                        size_t workspace_bytes, bool pow2, void *hip_stream) {
    fp8_status st = check_gemm_common(a_e4m3, a_scales, w_e4m3, w_scales, c, out_dtype, T, N, K,
                                      workspace, workspace_bytes);
    if (st != FP8_OK) return st;
    if (E < 0 || E >= (int64_t)1 << 20) return FP8_ERR_SHAPE;
    if (E * N * K >= kMaxElems * 64) return FP8_ERR_SHAPE;
    if (((T + 127) / 128 + E) * (N / 128) >= kMaxTiles) return FP8_ERR_SHAPE;
    if (T == 0 || N == 0) return FP8_OK;
    if (E == 0 || K == 0) return FP8_ERR_SHAPE;
    if (!group_offsets) return FP8_ERR_NULL;
    if (!aligned(group_offsets, 4)) return FP8_ERR_ALIGN;
    return from_hip(fp8blk::launch_grouped_gemm(a_e4m3, a_scales, w_e4m3, w_scales, group_offsets,
                                                E, T, c, out_dtype == FP8_OUT_BF16, N, K, pow2,
                                                as_stream(hip_stream)));
}

}  // namespace

extern "C" {

fp8_status fp8_quant_act_1x128(const void *x_bf16, int64_t M, int64_t K, void *q_e4m3,
                               float *scales, void *hip_stream) {
    return quant_act(x_bf16, M, K, q_e4m3, scales, false, hip_stream);
}

fp8_status fp8_quant_weight_128x128(const void *w_bf16, int64_t N, int64_t K, void *q_e4m3,
                                    float *scales, void *hip_stream) {
    return quant_weight(w_bf16, N, K, q_e4m3, scales, false, hip_stream);
}

fp8_status fp8_quant_act_1x128_pow2(const void *x_bf16, int64_t M, int64_t K, void *q_e4m3,
                                    float *scales, void *hip_stream) {
    return quant_act(x_bf16, M, K, q_e4m3, scales, true, hip_stream);
}

fp8_status fp8_quant_weight_128x128_pow2(const void *w_bf16, int64_t N, int64_t K,
                                         void *q_e4m3, float *scales, void *hip_stream) {
    return quant_weight(w_bf16, N, K, q_e4m3, scales, true, hip_stream);
}

fp8_status fp8_block_gemm(const void *a_e4m3, const float *a_scales, const void *w_e4m3,
                          const float *w_scales, void *c, int out_dtype, int64_t M, int64_t N,
                          int64_t K, void *workspace, size_t workspace_bytes, void *hip_stream) {
    return block_gemm(a_e4m3, a_scales, w_e4m3, w_scales, c, out_dtype, M, N, K, workspace,
                      workspace_bytes, false, hip_stream);
}

fp8_status fp8_block_gemm_pow2(const void *a_e4m3, const float *a_scales, const void *w_e4m3,
                               const float *w_scales, void *c, int out_dtype, int64_t M,
                               int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                               void *hip_stream) {
    return block_gemm(a_e4m3, a_scales, w_e4m3, w_scales, c, out_dtype, M, N, K, workspace,
                      workspace_bytes, true, hip_stream);
}

fp8_status fp8_block_grouped_gemm(const void *a_e4m3, const float *a_scales,
                                  const void *w_e4m3, const float *w_scales,
                                  const int32_t *group_offsets, int64_t E, int64_t T, void *c,
                                  int out_dtype, int64_t N, int64_t K, void *workspace,
                                  size_t workspace_bytes, void *hip_stream) {
    return grouped_gemm(a_e4m3, a_scales, w_e4m3, w_scales, group_offsets, E, T, c, out_dtype,
                        N, K, workspace, workspace_bytes, false, hip_stream);
}

fp8_status fp8_block_grouped_gemm_pow2(const void *a_e4m3, const float *a_scales,
                                       const void *w_e4m3, const float *w_scales,
                                       const int32_t *group_offsets, int64_t E, int64_t T,
                                       void *c, int out_dtype, int64_t N, int64_t K,
                                       void *workspace, size_t workspace_bytes,
                                       void *hip_stream) {
    return grouped_gemm(a_e4m3, a_scales, w_e4m3, w_scales, group_offsets, E, T, c, out_dtype,
                        N, K, workspace, workspace_bytes, true, hip_stream);
}

fp8_status fp8_quant_act_128x1_t(const void *x_bf16, int64_t M, int64_t K, void *q_t,
                                 float *scales_t, void *hip_stream) {
    fp8_status st = check_quant(x_bf16, M, K, q_t, scales_t);
    if (st != FP8_OK || M == 0 || K == 0) return st;
    if (!aligned(x_bf16, 2) || !aligned(scales_t, 4)) return FP8_ERR_ALIGN;
    return from_hip(
        fp8blk::launch_quant_act_128x1_t(x_bf16, M, K, q_t, scales_t, as_stream(hip_stream)));
}

fp8_status fp8_transpose_weight_128x128(const void *q_e4m3, const float *scales, int64_t N,
                                        int64_t K, void *q_t, float *scales_t,
                                        void *hip_stream) {
    if (N < 0 || K < 0) return FP8_ERR_SHAPE;
    if (N == 0 || K == 0) return FP8_OK;
    if (!q_e4m3 || !scales || !q_t || !scales_t) return FP8_ERR_NULL;
    if (N >= kMaxDim || K >= kMaxDim || N * K >= kMaxElems) return FP8_ERR_SHAPE;
    if (!aligned(scales, 4) || !aligned(scales_t, 4)) return FP8_ERR_ALIGN;
    return from_hip(fp8blk::launch_transpose_weight(q_e4m3, scales, N, K, q_t, scales_t,
                                                    as_stream(hip_stream)));
}

fp8_status fp8_block_gemm_wgrad(const void *dy_t, const float *dy_t_scales, const void *x_t,
                                const float *x_t_scales, void *dw, int out_dtype, int64_t N,
                                int64_t K, int64_t T, void *hip_stream) {
    // rows N, columns K, inner dimension T (tokens)
    fp8_status st = check_gemm_common(dy_t, dy_t_scales, x_t, x_t_scales, dw, out_dtype, N, K, T,
                                      nullptr, 0);
    if (st != FP8_OK || N == 0 || K == 0) return st;
    if (T == 0) return FP8_ERR_SHAPE;
    return from_hip(fp8blk::launch_block_gemm_wgrad(dy_t, dy_t_scales, x_t, x_t_scales, dw,
                                                    out_dtype == FP8_OUT_BF16, N, K, T,
                                                    as_stream(hip_stream)));
}

size_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int out_dtype) {
    if (out_dtype != FP8_OUT_F32 && out_dtype != FP8_OUT_BF16) return 0;
    if (M <= 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return 0;
    return fp8blk::gemm_workspace_bytes(M, N, K);
}

const char *fp8_status_string(fp8_status s) {
    switch (s) {
        case FP8_OK: return "FP8_OK";
        case FP8_ERR_NULL: return "FP8_ERR_NULL: a required pointer is NULL";
        case FP8_ERR_SHAPE: return "FP8_ERR_SHAPE: invalid size (negative, too large, or a GEMM N/K not a multiple of 128)";
        case FP8_ERR_ALIGN: return "FP8_ERR_ALIGN: pointer not aligned (GEMM operands and output need 16 bytes)";
        case FP8_ERR_DTYPE: return "FP8_ERR_DTYPE: out_dtype must be FP8_OUT_F32 or FP8_OUT_BF16";
        case FP8_ERR_WORKSPACE: return "FP8_ERR_WORKSPACE: workspace NULL with nonzero size, or not 256-byte aligned";
        case FP8_ERR_HIP: return "FP8_ERR_HIP: a HIP kernel launch failed";
    }
    return "unknown fp8_status";
}

}  // extern "C"
