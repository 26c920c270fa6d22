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

// Bytes of fp32 split-K partials the dense GEMM would use for this shape
// (0 when it runs without splitting K).
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

// pow2: every scale is a power of two, applied by the block-scaled MFMA.
hipError_t launch_block_gemm(const void *a, const float *sa, const void *w, const float *sw,
                             void *c, bool bf16_out, int64_t M, int64_t N, int64_t K,
                             void *workspace, size_t workspace_bytes, bool pow2,
                             hipStream_t stream);

hipError_t launch_grouped_gemm(const void *a, const float *sa, const void *w, const float *sw,
                               const int32_t *offsets, int64_t E, int64_t T, void *c,
                               bool bf16_out, int64_t N, int64_t K, bool pow2,
                               hipStream_t stream);

}  // namespace fp8blk
