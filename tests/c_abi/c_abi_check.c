/*
 * The C ABI used from plain C99, with no Python in the process: seeded bf16
 * activations and weights go through fp8_quant_act_1x128,
 * fp8_quant_weight_128x128 and fp8_block_gemm (FP32 output, split-K
 * workspace from fp8_gemm_workspace_bytes) on a HIP stream of this program,
 * and are checked against the CPU oracle's C functions (test
 * infrastructure, linked here only): E4M3 bytes and scale bits equal, and a
 * relative Frobenius error of at most 1e-3 against the binary64 GEMM.  The
 * argument checks are exercised too (a K that is not a multiple of 128,
 * NULL pointers, an unknown output type).
 *
 * Usage: c_abi_check [M N K]   (defaults 200 384 2688: two M tiles, the
 * second ragged, and K split four ways through the workspace).  Prints one
 * line; exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8blk.h"

/* oracle/oracle.c */
void orc_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *scales);
void orc_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q,
                              float *scales);
void orc_block_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qw,
                         const float *sw, int64_t M, int64_t N, int64_t K,
                         const int64_t *rows, int64_t nrows, double *R);

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            printf("c-abi FAIL: %s -> %s\n", #call, hipGetErrorString(e_));      \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

/* xorshift64* stream for the inputs */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void *dev_alloc(size_t n) {
    void *p = NULL;
    HIP_OK(hipMalloc(&p, n ? n : 1));
    return p;
}

int main(int argc, char **argv) {
    int64_t M = 200, N = 384, K = 2688;
    if (argc == 4) {
        M = atoll(argv[1]);
        N = atoll(argv[2]);
        K = atoll(argv[3]);
    }
    const int64_t G = (K + 127) / 128, NB = (N + 127) / 128;
    int fails = 0;

    /* activations: uniform(-1, 1) with every 37th channel x 50 (outliers);
     * weights: uniform(-0.02, 0.02) */
    uint16_t *x = malloc(sizeof(uint16_t) * M * K), *w = malloc(sizeof(uint16_t) * N * K);
    for (int64_t i = 0; i < M * K; ++i) {
        const double v = 2.0 * uniform01() - 1.0;
        x[i] = to_bf16((float)(((i % K) % 37 == 0) ? 50.0 * v : v));
    }
    for (int64_t i = 0; i < N * K; ++i) w[i] = to_bf16((float)(0.04 * uniform01() - 0.02));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void *dx = dev_alloc(2 * M * K), *dw = dev_alloc(2 * N * K);
    void *dqa = dev_alloc(M * K), *dqw = dev_alloc(N * K);
    float *dsa = dev_alloc(4 * M * G), *dsw = dev_alloc(4 * NB * G);
    float *dc = dev_alloc(4 * M * N);
    HIP_OK(hipMemcpy(dx, x, 2 * M * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw, w, 2 * N * K, hipMemcpyHostToDevice));

    fp8_status st = fp8_quant_act_1x128(dx, M, K, dqa, dsa, stream);
    if (st == FP8_OK) st = fp8_quant_weight_128x128(dw, N, K, dqw, dsw, stream);
    const size_t ws_bytes = fp8_gemm_workspace_bytes(M, N, K, FP8_OUT_F32);
    void *ws = ws_bytes ? dev_alloc(ws_bytes) : NULL;
    if (st == FP8_OK)
        st = fp8_block_gemm(dqa, dsa, dqw, dsw, dc, FP8_OUT_F32, M, N, K, ws, ws_bytes, stream);
    if (st != FP8_OK) {
        printf("c-abi FAIL: %s\n", fp8_status_string(st));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));

    uint8_t *qa = malloc(M * K), *qw = malloc(N * K), *qa_o = malloc(M * K), *qw_o = malloc(N * K);
    float *sa = malloc(4 * M * G), *sw = malloc(4 * NB * G), *sa_o = malloc(4 * M * G),
          *sw_o = malloc(4 * NB * G), *c = malloc(4 * M * N);
    HIP_OK(hipMemcpy(qa, dqa, M * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(qw, dqw, N * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sa, dsa, 4 * M * G, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sw, dsw, 4 * NB * G, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(c, dc, 4 * M * N, hipMemcpyDeviceToHost));

    orc_quant_act_1x128(x, M, K, qa_o, sa_o);
    orc_quant_weight_128x128(w, N, K, qw_o, sw_o);
    const int bytes_equal = !memcmp(qa, qa_o, M * K) && !memcmp(qw, qw_o, N * K);
    const int scales_equal = !memcmp(sa, sa_o, 4 * M * G) && !memcmp(sw, sw_o, 4 * NB * G);
    fails += !bytes_equal + !scales_equal;

    int64_t *rows = malloc(sizeof(int64_t) * M);
    double *R = malloc(sizeof(double) * M * N);
    for (int64_t m = 0; m < M; ++m) rows[m] = m;
    orc_block_gemm_rows(qa_o, sa_o, qw_o, sw_o, M, N, K, rows, M, R);
    double num = 0.0, den = 0.0;
    for (int64_t i = 0; i < M * N; ++i) {
        const double d = (double)c[i] - R[i];
        num += d * d;
        den += R[i] * R[i];
    }
    const double rel_fro = sqrt(num / den);
    fails += !(rel_fro <= 1e-3);

    /* argument checks: nothing enqueued, the documented status returned */
    const int err_shape = fp8_block_gemm(dqa, dsa, dqw, dsw, dc, FP8_OUT_F32, M, N, 100, NULL,
                                         0, stream) == FP8_ERR_SHAPE;
    const int err_null = fp8_quant_act_1x128(NULL, M, K, dqa, dsa, stream) == FP8_ERR_NULL;
    const int err_dtype = fp8_block_gemm(dqa, dsa, dqw, dsw, dc, 7, M, N, K, NULL, 0,
                                         stream) == FP8_ERR_DTYPE;
    fails += !err_shape + !err_null + !err_dtype;

    printf("c-abi %s: M=%lld N=%lld K=%lld workspace=%zu bytes_equal=%d scales_equal=%d "
           "rel_fro=%.3e error_codes=%d%d%d\n",
           fails ? "FAIL" : "ok", (long long)M, (long long)N, (long long)K, ws_bytes, bytes_equal,
           scales_equal, rel_fro, err_shape, err_null, err_dtype);

    HIP_OK(hipStreamDestroy(stream));
    hipFree(dx); hipFree(dw); hipFree(dqa); hipFree(dqw); hipFree(dsa); hipFree(dsw);
    hipFree(dc); if (ws) hipFree(ws);
    free(x); free(w); free(qa); free(qw); free(qa_o); free(qw_o); free(sa); free(sw);
    free(sa_o); free(sw_o); free(c); free(rows); free(R);
    return fails ? 1 : 0;
}
