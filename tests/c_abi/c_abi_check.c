/*
 * The C ABI used from plain C99, with no Python in the process: seeded bf16
 * activations and weights go through fp8_quant_act_1x128,
 * fp8_quant_weight_128x128 and fp8_block_gemm (FP32 output, split-K
 * workspace from fp8_gemm_workspace_bytes) on a HIP stream of this program,
 * and are checked against the CPU oracle's C functions (test
 * infrastructure, linked here only): E4M3 bytes and scale bits equal, and a
 * relative Frobenius error of at most 1e-3 against the binary64 GEMM.  Then
 * the other entry points on the same activations:
 *   - fp8_block_grouped_gemm over three experts (the middle one empty, BF16
 *     output; every row against the binary64 reference, at most 8e-3);
 *   - fp8_quant_act_128x1_t (bytes and scale bits equal);
 *   - fp8_transpose_weight_128x128 (equal to the transposed oracle bytes and
 *     scales);
 *   - fp8_block_gemm_wgrad, dW = X^T X over the whole 128-token blocks of
 *     the activations (sampled rows, at most 1e-3);
 *   - fp8_block_gemm_fused_quant on the bf16 activations (its E4M3 bytes and
 *     scales equal the oracle's, C within 1e-3);
 *   - fp8_block_gemm_noalloc (bitwise equal to fp8_block_gemm's C);
 *   - fp8_block_gemm_dgrad, dX = dY W for a seeded dY [M][N] on the forward
 *     weights (within 1e-3 of the oracle on the transposed weights).
 * The argument checks are exercised too (a K that is not a multiple of 128,
 * NULL pointers, an unknown output type, a token count that is not a
 * multiple of 128 for Wgrad, no experts for routed tokens, fused bytes out
 * without scales out, a Dgrad inner size that is not a multiple of 128).
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
void orc_quant_act_128x1_t(const uint16_t *x, int64_t M, int64_t K, uint8_t *q_t,
                           float *scales_t);
void orc_rowscaled_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qb,
                             const float *sb, int64_t M, int64_t N, int64_t K,
                             const int64_t *rows, int64_t nrows, double *R);
void orc_grouped_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qw,
                           const float *sw, const int32_t *off, int64_t E, int64_t T,
                           int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                           double *R, int32_t *found);

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

/* relative Frobenius error of got (n values) against the binary64 ref */
static double rel_fro_of(const float *got, const double *ref, int64_t n) {
    double num = 0.0, den = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double d = (double)got[i] - ref[i];
        num += d * d;
        den += ref[i] * ref[i];
    }
    return den > 0.0 ? sqrt(num / den) : sqrt(num);
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

    /* ---- grouped GEMM: three experts over the M tokens, expert 1 empty ---- */
    const int64_t E = 3;
    const int32_t off[4] = {0, (int32_t)(M / 2), (int32_t)(M / 2), (int32_t)M};
    uint16_t *we = malloc(sizeof(uint16_t) * E * N * K);
    for (int64_t i = 0; i < E * N * K; ++i) we[i] = to_bf16((float)(0.04 * uniform01() - 0.02));
    void *dwe = dev_alloc(2 * E * N * K), *dqwe = dev_alloc(E * N * K);
    float *dswe = dev_alloc(4 * E * NB * G);
    int32_t *doff = dev_alloc(sizeof(off));
    uint16_t *dcg = dev_alloc(2 * M * N);
    HIP_OK(hipMemcpy(dwe, we, 2 * E * N * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(doff, off, sizeof(off), hipMemcpyHostToDevice));
    st = fp8_quant_weight_128x128(dwe, E * N, K, dqwe, dswe, stream);
    if (st == FP8_OK)
        st = fp8_block_grouped_gemm(dqa, dsa, dqwe, dswe, doff, E, M, dcg, FP8_OUT_BF16, N, K,
                                    NULL, 0, stream);
    if (st != FP8_OK) {
        printf("c-abi FAIL (grouped): %s\n", fp8_status_string(st));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));
    uint8_t *qwe_o = malloc(E * N * K);
    float *swe_o = malloc(4 * E * NB * G);
    uint16_t *cg16 = malloc(2 * M * N);
    float *cg = malloc(4 * M * N);
    double *Rg = malloc(sizeof(double) * M * N);
    int32_t *found = malloc(sizeof(int32_t) * M);
    HIP_OK(hipMemcpy(cg16, dcg, 2 * M * N, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < M * N; ++i) {
        const uint32_t u = (uint32_t)cg16[i] << 16;
        memcpy(&cg[i], &u, 4);
    }
    orc_quant_weight_128x128(we, E * N, K, qwe_o, swe_o);
    orc_grouped_gemm_rows(qa_o, sa_o, qwe_o, swe_o, off, E, M, N, K, rows, M, Rg, found);
    int all_found = 1;
    for (int64_t m = 0; m < M; ++m) all_found &= found[m] != 0;
    const double grouped_rel_fro = rel_fro_of(cg, Rg, M * N);
    fails += !all_found + !(grouped_rel_fro <= 8e-3);

    /* ---- backward pieces ---- */
    const int64_t GM = (M + 127) / 128, T = (M / 128) * 128;
    void *dqt = dev_alloc(K * M), *dqwt = dev_alloc(K * N);
    float *dst = dev_alloc(4 * K * GM), *dswt = dev_alloc(4 * G * NB);
    st = fp8_quant_act_128x1_t(dx, M, K, dqt, dst, stream);
    if (st == FP8_OK) st = fp8_transpose_weight_128x128(dqw, dsw, N, K, dqwt, dswt, stream);
    if (st != FP8_OK) {
        printf("c-abi FAIL (backward): %s\n", fp8_status_string(st));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));
    uint8_t *qt = malloc(K * M), *qt_o = malloc(K * M), *qwt = malloc(K * N);
    float *st_ = malloc(4 * K * GM), *st_o = malloc(4 * K * GM), *swt = malloc(4 * G * NB);
    HIP_OK(hipMemcpy(qt, dqt, K * M, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(st_, dst, 4 * K * GM, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(qwt, dqwt, K * N, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(swt, dswt, 4 * G * NB, hipMemcpyDeviceToHost));
    orc_quant_act_128x1_t(x, M, K, qt_o, st_o);
    const int t_equal = !memcmp(qt, qt_o, K * M) && !memcmp(st_, st_o, 4 * K * GM);
    int tr_equal = 1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) tr_equal &= qwt[k * N + n] == qw_o[n * K + k];
    for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t g = 0; g < G; ++g) tr_equal &= swt[g * NB + nb] == sw_o[nb * G + g];
    fails += !t_equal + !tr_equal;

    /* Wgrad dW = X^T X over the first T tokens (their 128x1 groups), if any */
    double wgrad_rel_fro = 0.0;
    if (T > 0) {
        void *dq2 = dev_alloc(K * T);
        float *ds2 = dev_alloc(4 * K * (T / 128)), *ddw = dev_alloc(4 * K * K);
        st = fp8_quant_act_128x1_t(dx, T, K, dq2, ds2, stream);
        if (st == FP8_OK) st = fp8_block_gemm_wgrad(dq2, ds2, dq2, ds2, ddw, FP8_OUT_F32, K, K, T, stream);
        if (st != FP8_OK) {
            printf("c-abi FAIL (wgrad): %s\n", fp8_status_string(st));
            return 1;
        }
        HIP_OK(hipStreamSynchronize(stream));
        int64_t wrows[8], nw = 0;
        const int64_t cand[8] = {0, 1, 127, 128, K / 2, K - 129, K - 128, K - 1};
        for (int i = 0; i < 8; ++i)
            if (cand[i] >= 0 && cand[i] < K && (nw == 0 || cand[i] > wrows[nw - 1])) wrows[nw++] = cand[i];
        uint8_t *q2 = malloc(K * T);
        float *s2 = malloc(4 * K * (T / 128)), *dwr = malloc(4 * nw * K);
        double *Rw = malloc(sizeof(double) * nw * K);
        for (int64_t i = 0; i < nw; ++i)
            HIP_OK(hipMemcpy(dwr + i * K, ddw + wrows[i] * K, 4 * K, hipMemcpyDeviceToHost));
        orc_quant_act_128x1_t(x, T, K, q2, s2);
        orc_rowscaled_gemm_rows(q2, s2, q2, s2, K, K, T, wrows, nw, Rw);
        wgrad_rel_fro = rel_fro_of(dwr, Rw, nw * K);
        fails += !(wgrad_rel_fro <= 1e-3);
        hipFree(dq2); hipFree(ds2); hipFree(ddw);
        free(q2); free(s2); free(dwr); free(Rw);
    }
    const int err_tokens = fp8_block_gemm_wgrad(dqt, dst, dqt, dst, dc, FP8_OUT_F32, K, K, 200,
                                                stream) == FP8_ERR_SHAPE;
    const int err_experts = fp8_block_grouped_gemm(dqa, dsa, dqwe, dswe, doff, 0, M, dcg,
                                                   FP8_OUT_BF16, N, K, NULL, 0,
                                                   stream) == FP8_ERR_SHAPE;
    fails += !err_tokens + !err_experts;

    /* ---- quantization fused into the GEMM, on the bf16 activations ---- */
    void *dqf = dev_alloc(M * K);
    float *dsf = dev_alloc(4 * M * G), *dcf = dev_alloc(4 * M * N), *dcn = dev_alloc(4 * M * N);
    st = fp8_block_gemm_fused_quant(dx, dqw, dsw, dcf, FP8_OUT_F32, M, N, K, dqf, dsf, NULL, 0,
                                    stream);
    /* ---- the no-allocation GEMM: its own static scratch for split-K ---- */
    if (st == FP8_OK)
        st = fp8_block_gemm_noalloc(dqa, dsa, dqw, dsw, dcn, FP8_OUT_F32, M, N, K, stream);
    if (st != FP8_OK) {
        printf("c-abi FAIL (fused / noalloc): %s\n", fp8_status_string(st));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));
    uint8_t *qf = malloc(M * K);
    float *sf = malloc(4 * M * G), *cf = malloc(4 * M * N), *cn = malloc(4 * M * N);
    HIP_OK(hipMemcpy(qf, dqf, M * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sf, dsf, 4 * M * G, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(cf, dcf, 4 * M * N, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(cn, dcn, 4 * M * N, hipMemcpyDeviceToHost));
    const int fused_q_equal = !memcmp(qf, qa_o, M * K) && !memcmp(sf, sa_o, 4 * M * G);
    const double fused_rel_fro = rel_fro_of(cf, R, M * N);
    const int noalloc_equal = !memcmp(cn, c, 4 * M * N);
    fails += !fused_q_equal + !(fused_rel_fro <= 1e-3) + !noalloc_equal;

    /* ---- Dgrad on the forward weights: dX [M][K] = dY [M][N] W [N][K] ---- */
    uint16_t *dyb = malloc(sizeof(uint16_t) * M * N);
    for (int64_t i = 0; i < M * N; ++i) dyb[i] = to_bf16((float)(2.0 * uniform01() - 1.0));
    void *ddy = dev_alloc(2 * M * N), *dqdy = dev_alloc(M * N);
    float *dsdy = dev_alloc(4 * M * NB), *ddx = dev_alloc(4 * M * K);
    HIP_OK(hipMemcpy(ddy, dyb, 2 * M * N, hipMemcpyHostToDevice));
    const size_t ws_dg = fp8_gemm_workspace_bytes(M, K, N, FP8_OUT_F32);
    void *wsd = ws_dg ? dev_alloc(ws_dg) : NULL;
    st = fp8_quant_act_1x128(ddy, M, N, dqdy, dsdy, stream);
    if (st == FP8_OK)
        st = fp8_block_gemm_dgrad(dqdy, dsdy, dqw, dsw, ddx, FP8_OUT_F32, M, N, K, wsd, ws_dg,
                                  stream);
    if (st != FP8_OK) {
        printf("c-abi FAIL (dgrad): %s\n", fp8_status_string(st));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));
    uint8_t *qdy_o = malloc(M * N), *qwt_o = malloc(K * N);
    float *sdy_o = malloc(4 * M * NB), *swt_o = malloc(4 * G * NB), *dxh = malloc(4 * M * K);
    double *Rd = malloc(sizeof(double) * M * K);
    HIP_OK(hipMemcpy(dxh, ddx, 4 * M * K, hipMemcpyDeviceToHost));
    orc_quant_act_1x128(dyb, M, N, qdy_o, sdy_o);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) qwt_o[k * N + n] = qw_o[n * K + k];
    for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t g = 0; g < G; ++g) swt_o[g * NB + nb] = sw_o[nb * G + g];
    orc_block_gemm_rows(qdy_o, sdy_o, qwt_o, swt_o, M, K, N, rows, M, Rd);
    const double dgrad_rel_fro = rel_fro_of(dxh, Rd, M * K);
    fails += !(dgrad_rel_fro <= 1e-3);
    const int err_fused = fp8_block_gemm_fused_quant(dx, dqw, dsw, dcf, FP8_OUT_F32, M, N, K, dqf,
                                                     NULL, NULL, 0, stream) == FP8_ERR_NULL;
    const int err_dgrad = fp8_block_gemm_dgrad(dqdy, dsdy, dqw, dsw, ddx, FP8_OUT_F32, M, 200, K,
                                               NULL, 0, stream) == FP8_ERR_SHAPE;
    fails += !err_fused + !err_dgrad;

    printf("c-abi %s: M=%lld N=%lld K=%lld workspace=%zu bytes_equal=%d scales_equal=%d "
           "rel_fro=%.3e grouped_rel_fro=%.3e q128x1_t_equal=%d transpose_equal=%d "
           "wgrad_tokens=%lld wgrad_rel_fro=%.3e fused_q_equal=%d fused_rel_fro=%.3e "
           "noalloc_equal=%d dgrad_rel_fro=%.3e error_codes=%d%d%d%d%d%d%d\n",
           fails ? "FAIL" : "ok", (long long)M, (long long)N, (long long)K, ws_bytes, bytes_equal,
           scales_equal, rel_fro, grouped_rel_fro, t_equal, tr_equal, (long long)T, wgrad_rel_fro,
           fused_q_equal, fused_rel_fro, noalloc_equal, dgrad_rel_fro, err_shape, err_null,
           err_dtype, err_tokens, err_experts, err_fused, err_dgrad);
    hipFree(dqf); hipFree(dsf); hipFree(dcf); hipFree(dcn); hipFree(ddy); hipFree(dqdy);
    hipFree(dsdy); hipFree(ddx); if (wsd) hipFree(wsd);
    free(qf); free(sf); free(cf); free(cn); free(dyb); free(qdy_o); free(qwt_o); free(sdy_o);
    free(swt_o); free(dxh); free(Rd);
    hipFree(dwe); hipFree(dqwe); hipFree(dswe); hipFree(doff); hipFree(dcg);
    hipFree(dqt); hipFree(dqwt); hipFree(dst); hipFree(dswt);
    free(we); free(qwe_o); free(swe_o); free(cg16); free(cg); free(Rg); free(found);
    free(qt); free(qt_o); free(qwt); free(st_); free(st_o); free(swt);

    HIP_OK(hipStreamDestroy(stream));
    hipFree(dx); hipFree(dw); hipFree(dqa); hipFree(dqw); hipFree(dsa); hipFree(dsw);
    hipFree(dc); if (ws) hipFree(ws);
    free(x); free(w); free(qa); free(qw); free(qa_o); free(qw_o); free(sa); free(sw);
    free(sa_o); free(sw_o); free(c); free(rows); free(R);
    return fails ? 1 : 0;
}
