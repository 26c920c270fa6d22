/*
 * CPU oracle for fine-grained FP8 quantization and block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library; it is built with gcc, plain C99, IEEE
 * binary32/binary64 arithmetic (-O2 -ffp-contract=off, no fast-math), and
 * OpenMP only across independent rows.
 *
 * Sources (the pages are cited by site and post, then by figure/passage):
 *   [dssusan 93378]  page "dssusan.co.kr qna 93378", passage on Figure 7 (a):
 *                    activations are grouped and scaled per token per 128
 *                    channels (1x128 tiles), weights per 128 input x 128
 *                    output channels (128x128 blocks); E4M3 on all tensors;
 *                    per-group scaling factors run along the inner dimension K
 *                    and are multiplied in as the dequantization step; the
 *                    GEMMs take FP8 inputs and produce BF16 or FP32.
 *   [kailasan 147436] page "kailasan.com recruit 147436", passage on
 *                    promotion (Figure 7 (b)): partial results are scaled and
 *                    added into FP32 registers at a fixed K interval.
 *   [why-be 36949]   page "why-be.co.kr as_center 36949", passage on the
 *                    quantization round trip: 128 BF16 activation values are
 *                    read, quantized and written back as FP8.
 * The pages name E4M3 (4-bit exponent, 3-bit mantissa) but not its variant,
 * the scale formula or the rounding.  The readings used here: OCP E4M3FN
 * (bias 7, largest finite 448, S.1111.111 is NaN, no infinity), per-group
 * scale s = amax / 448 computed in binary32, quotient x / s in binary32, then
 * round-to-nearest-even into E4M3 (two roundings, in that order), an all-zero
 * group gives s = 0 and zero bytes, and the GEMM reference is the exact sum of
 * dequantized products evaluated in binary64.
 *
 * Power-of-two variant (the *_pow2 quantizers), after [kailasan 147436],
 * passage recommending that matrix units take the scaling factors and do
 * the group-scaled MMA themselves (block-scaled matrix instructions take
 * power-of-two scales).  The pages give no rule for such scales; the reading
 * used: s = the smallest power of two with 448 s >= amax, but at least
 * 2^-126 (so s is a normal binary32); then the same quotient and rounding as
 * above (x / s is exact); an all-zero group keeps s = 2^-126 and gets zero
 * bytes.  The GEMM reference needs no variant: it takes the scales as
 * inputs.
 *
 * Backward GEMMs [dssusan 93378, passages on FP8 in Fprop, Dgrad and Wgrad
 * (E4M3 on every tensor; Wgrad lets activations be kept in FP8) and on
 * per-group scaling along the inner dimension]; the grouping along the
 * transposed axis is a reading.  Dgrad (dX = dY W) keeps the forward
 * groupings: dY in 1x128 tiles along its inner dimension N, W in its
 * 128x128 blocks, used transposed.  Wgrad (dW = dY^T X) sums over tokens, so
 * both operands are grouped in 128x1 tiles (128 tokens of one channel),
 * stored transposed with the token axis contiguous; its reference is the
 * GEMM with one scale per row on both operands.
 *
 * Parity pins: every function here is pinned by tests that do not reuse this
 * code (format facts and an independent library cast for the E4M3 codec,
 * closed forms, invariants and exact-rational brute force for the rest).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FP8_MAX 448.0f
#define ORC_GROUP 128

/* ---- bf16 and E4M3 value definitions -------------------------------- */

/* bf16 is the top half of a binary32: widening is a 16-bit left shift. */
static float orc_bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Value of one E4M3FN code from the format definition: sign bit, 4-bit
 * exponent field E (bias 7), 3-bit mantissa m; E = 0 is subnormal
 * (m * 2^-9); E = 15, m = 7 is NaN; there is no infinity. */
double orc_e4m3_value(int code) {
    int s = (code >> 7) & 1;
    int E = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (E == 15 && m == 7) return NAN;
    if (E == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, E - 7);
    return s ? -mag : mag;
}

/* Table of the 127 finite non-negative magnitudes, ascending (code c has
 * value orc_mag[c] for c = 0..126). */
static double orc_mag[127];
static int orc_mag_ready = 0;

static void orc_init_table(void) {
    int c;
    if (orc_mag_ready) return;
    for (c = 0; c < 127; ++c) orc_mag[c] = orc_e4m3_value(c);
    orc_mag_ready = 1;
}

/* Encode a binary32 value into E4M3FN: round to nearest, ties to the code
 * with an even mantissa (LSB 0), magnitudes at or above the largest finite
 * value give that value, and the sign bit of the input is kept (so -0.0 and
 * negative values that round to zero give 0x80).  A plain bisection over
 * the sorted table of finite magnitudes; no bit manipulation of the float. */
uint8_t orc_e4m3_encode(float y) {
    double a = fabs((double)y);
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    int lo, code;
    double mid;
    orc_init_table();
    if (a >= (double)ORC_FP8_MAX) return (uint8_t)(sign | 0x7E);
    /* Bisection for the largest code lo with orc_mag[lo] <= a; the
     * invariant is orc_mag[lo] <= a < orc_mag[hi] (orc_mag[126] = 448 > a). */
    lo = 0;
    {
        int hi = 126;
        while (hi - lo > 1) {
            int m = (lo + hi) / 2;
            if (orc_mag[m] <= a)
                lo = m;
            else
                hi = m;
        }
    }
    /* a < 448 here, so lo <= 125 and lo + 1 is a finite code. */
    mid = (orc_mag[lo] + orc_mag[lo + 1]) * 0.5; /* exact in binary64 */
    if (a < mid)
        code = lo;
    else if (a > mid)
        code = lo + 1;
    else
        code = (lo % 2 == 0) ? lo : lo + 1;
    return (uint8_t)(sign | code);
}

/* Element-wise encode of n binary32 values (same rule as above). */
void orc_e4m3_encode_array(const float *y, int64_t n, uint8_t *out) {
    int64_t i;
    orc_init_table();
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_e4m3_encode(y[i]);
}

/* ---- one quantization group ------------------------------------------- */

/* Quantize the elements x[r*ld + c] for r < rows, c < cols as ONE group:
 *   amax = max |x|            (exact, order-free)
 *   s    = fl32(amax / 448)   (binary32 divide, RNE, gradual underflow),
 *          or with pow2 the smallest power of two >= amax / 448 and >= 2^-126
 *   q    = E4M3_RNE(fl32(x / s)), or all 0x00 when amax == 0 (with s = +0,
 *          or 2^-126 with pow2).
 * The bytes go to q[r*ld + c]; the scale is returned. */
static float orc_quant_group(const uint16_t *x, int64_t ld, int64_t rows,
                             int64_t cols, int pow2, uint8_t *q) {
    int64_t r, c;
    float amax = 0.0f, s;
    for (r = 0; r < rows; ++r)
        for (c = 0; c < cols; ++c) {
            float v = fabsf(orc_bf16_to_float(x[r * ld + c]));
            if (v > amax) amax = v;
        }
    if (pow2) {
        /* Start at the floor 2^-126 and double until 448 s reaches amax;
         * every step is exact in binary64. */
        double sd = ldexp(1.0, -126);
        while (448.0 * sd < (double)amax) sd *= 2.0;
        s = (float)sd; /* a power of two in binary32's normal range: exact */
    } else {
        s = amax / ORC_FP8_MAX;
    }
    if (amax == 0.0f) {
        for (r = 0; r < rows; ++r)
            for (c = 0; c < cols; ++c) q[r * ld + c] = 0x00;
        return s;
    }
    for (r = 0; r < rows; ++r)
        for (c = 0; c < cols; ++c) {
            float y = orc_bf16_to_float(x[r * ld + c]) / s;
            q[r * ld + c] = orc_e4m3_encode(y);
        }
    return s;
}

/* ---- the two quantizers ------------------------------------------------ */

/* 1x128 activation tiles [dssusan 93378, Figure 7 (a)]: x is bf16 [M][K]
 * row-major, q is E4M3 [M][K], scales is fp32 [M][ceil(K/128)] row-major;
 * the last group of a row holds the K % 128 remaining channels. */
static void orc_quant_act(const uint16_t *x, int64_t M, int64_t K, int pow2,
                          uint8_t *q, float *scales) {
    int64_t G = (K + ORC_GROUP - 1) / ORC_GROUP;
    int64_t m;
    orc_init_table();
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t g;
        for (g = 0; g < G; ++g) {
            int64_t k0 = g * ORC_GROUP;
            int64_t w = (K - k0 < ORC_GROUP) ? K - k0 : ORC_GROUP;
            scales[m * G + g] =
                orc_quant_group(x + m * K + k0, K, 1, w, pow2, q + m * K + k0);
        }
    }
}

/* 128x128 weight blocks [dssusan 93378, Figure 7 (a)]: w is bf16 [N][K]
 * (output channel n, input channel k), q is E4M3 [N][K], scales is fp32
 * [ceil(N/128)][ceil(K/128)]; edge blocks hold what remains. */
static void orc_quant_weight(const uint16_t *w, int64_t N, int64_t K, int pow2,
                             uint8_t *q, float *scales) {
    int64_t NB = (N + ORC_GROUP - 1) / ORC_GROUP;
    int64_t G = (K + ORC_GROUP - 1) / ORC_GROUP;
    int64_t blk;
    orc_init_table();
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < NB * G; ++blk) {
        int64_t nb = blk / G, g = blk % G;
        int64_t n0 = nb * ORC_GROUP, k0 = g * ORC_GROUP;
        int64_t h = (N - n0 < ORC_GROUP) ? N - n0 : ORC_GROUP;
        int64_t wd = (K - k0 < ORC_GROUP) ? K - k0 : ORC_GROUP;
        scales[nb * G + g] =
            orc_quant_group(w + n0 * K + k0, K, h, wd, pow2, q + n0 * K + k0);
    }
}

void orc_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q,
                         float *scales) {
    orc_quant_act(x, M, K, 0, q, scales);
}

void orc_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K,
                              uint8_t *q, float *scales) {
    orc_quant_weight(w, N, K, 0, q, scales);
}

/* Power-of-two-scale variants (same layouts). */
void orc_quant_act_1x128_pow2(const uint16_t *x, int64_t M, int64_t K,
                              uint8_t *q, float *scales) {
    orc_quant_act(x, M, K, 1, q, scales);
}

void orc_quant_weight_128x128_pow2(const uint16_t *w, int64_t N, int64_t K,
                                   uint8_t *q, float *scales) {
    orc_quant_weight(w, N, K, 1, q, scales);
}

/* 128x1 tiles, written transposed [backward reading above]: group (mb, k)
 * holds x[m][k] for m in [128 mb, min(128 mb + 128, M)), quantized as one
 * group (as orc_quant_group: amax / 448 scale, or with pow2 the power-of-two
 * scale).  q_t is E4M3 [K][M] with q_t[k][m] the code of x[m][k]; scales_t
 * is fp32 [K][ceil(M/128)]. */
static void orc_quant_128x1_t(const uint16_t *x, int64_t M, int64_t K, int pow2,
                              uint8_t *q_t, float *scales_t) {
    int64_t GM = (M + ORC_GROUP - 1) / ORC_GROUP;
    int64_t k;
    uint8_t *q = (uint8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    orc_init_table();
#pragma omp parallel for schedule(static)
    for (k = 0; k < K; ++k) {
        int64_t mb;
        for (mb = 0; mb < GM; ++mb) {
            int64_t m0 = mb * ORC_GROUP;
            int64_t h = (M - m0 < ORC_GROUP) ? M - m0 : ORC_GROUP;
            scales_t[k * GM + mb] =
                orc_quant_group(x + m0 * K + k, K, h, 1, pow2, q + m0 * K + k);
        }
    }
#pragma omp parallel for schedule(static)
    for (k = 0; k < K; ++k) {
        int64_t m;
        for (m = 0; m < M; ++m) q_t[k * M + m] = q[m * K + k];
    }
    free(q);
}

void orc_quant_act_128x1_t(const uint16_t *x, int64_t M, int64_t K,
                           uint8_t *q_t, float *scales_t) {
    orc_quant_128x1_t(x, M, K, 0, q_t, scales_t);
}

void orc_quant_act_128x1_t_pow2(const uint16_t *x, int64_t M, int64_t K,
                                uint8_t *q_t, float *scales_t) {
    orc_quant_128x1_t(x, M, K, 1, q_t, scales_t);
}

/* ---- GEMM reference ----------------------------------------------------- */

/* Dequantized operand element: the E4M3 value times its group's scale.
 * Both factors are exact in binary64 and so is their product (4 + 24
 * significant bits). */
static double orc_deq(uint8_t code, float scale) {
    return orc_e4m3_value(code) * (double)scale;
}

/* One output row of C = A_deq * W_deq^T with the per-group scales running
 * along K [dssusan 93378, passage on scaling along the inner dimension]:
 *   R[n] = sum_{k=0}^{K-1} (qa[k] * sa[k/128]) * (qw[n][k] * sw[n/128][k/128])
 * summed in ascending k in binary64.  qa_row / sa_row are one activation row
 * and its ceil(K/128) scales; qw is [N][K], sw is [ceil(N/128)][ceil(K/128)].
 */
/* w_rows_per_scale: 128 when sw holds one scale row per 128 W rows (128x128
 * blocks), 1 when every W row has its own scales (1x128 tiles, Wgrad). */
static void orc_gemm_row(const uint8_t *qa_row, const float *sa_row,
                         const uint8_t *qw, const float *sw, int64_t N,
                         int64_t K, int64_t w_rows_per_scale, double *R) {
    int64_t G = (K + ORC_GROUP - 1) / ORC_GROUP;
    int64_t n, k;
    double *a_deq = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    for (k = 0; k < K; ++k) a_deq[k] = orc_deq(qa_row[k], sa_row[k / ORC_GROUP]);
    for (n = 0; n < N; ++n) {
        const uint8_t *wrow = qw + n * K;
        const float *swrow = sw + (n / w_rows_per_scale) * G;
        double acc = 0.0;
        for (k = 0; k < K; ++k)
            acc += a_deq[k] * orc_deq(wrow[k], swrow[k / ORC_GROUP]);
        R[n] = acc;
    }
    free(a_deq);
}

/* Dense block-scaled GEMM reference for a chosen set of rows.
 * qa: E4M3 [M][K], sa: fp32 [M][ceil(K/128)], qw: E4M3 [N][K],
 * sw: fp32 [ceil(N/128)][ceil(K/128)], rows: nrows indices into [0, M),
 * R: binary64 [nrows][N]. */
void orc_block_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qw,
                         const float *sw, int64_t M, int64_t N, int64_t K,
                         const int64_t *rows, int64_t nrows, double *R) {
    int64_t G = (K + ORC_GROUP - 1) / ORC_GROUP;
    int64_t r;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nrows; ++r) {
        int64_t m = rows[r];
        orc_gemm_row(qa + m * K, sa + m * G, qw, sw, N, K, ORC_GROUP, R + r * N);
    }
}

/* GEMM with one scale row per row of both operands (Wgrad on 128x1-grouped
 * operands stored transposed): R[r][n] = sum_k (qa[m][k] sa[m][k/128])
 * (qb[n][k] sb[n][k/128]) for m = rows[r]; qb is [N][K], sb [N][ceil(K/128)]. */
void orc_rowscaled_gemm_rows(const uint8_t *qa, const float *sa,
                             const uint8_t *qb, const float *sb, int64_t M,
                             int64_t N, int64_t K, const int64_t *rows,
                             int64_t nrows, double *R) {
    int64_t G = (K + ORC_GROUP - 1) / ORC_GROUP;
    int64_t r;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nrows; ++r) {
        int64_t m = rows[r];
        orc_gemm_row(qa + m * K, sa + m * G, qb, sb, N, K, 1, R + r * N);
    }
}

/* Grouped (MoE) reference: rows t in [off[e], off[e+1]) belong to expert e
 * and use W[e] = qw + e*N*K with its scales sw + e*ceil(N/128)*ceil(K/128).
 * Offsets are read as given (the caller passes a valid non-decreasing
 * array).  For each requested row the expert is found by a linear scan;
 * found[r] = 1 and R[r][:] holds the row, or found[r] = 0 (row outside every
 * expert) and R[r][:] is left untouched. */
void orc_grouped_gemm_rows(const uint8_t *qa, const float *sa,
                           const uint8_t *qw, const float *sw,
                           const int32_t *off, int64_t E, int64_t T, int64_t N,
                           int64_t K, const int64_t *rows, int64_t nrows,
                           double *R, int32_t *found) {
    int64_t G = (K + ORC_GROUP - 1) / ORC_GROUP;
    int64_t NB = (N + ORC_GROUP - 1) / ORC_GROUP;
    int64_t r;
    (void)T;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nrows; ++r) {
        int64_t t = rows[r], e, hit = -1;
        for (e = 0; e < E; ++e)
            if (t >= off[e] && t < off[e + 1]) { hit = e; break; }
        found[r] = hit >= 0;
        if (hit < 0) continue;
        orc_gemm_row(qa + t * K, sa + t * G, qw + hit * N * K,
                     sw + hit * NB * G, N, K, ORC_GROUP, R + r * N);
    }
}

int orc_max_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the OpenMP loops above (the benchmark times the quantizer
 * single-threaded as well); n <= 0 leaves it unchanged. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
