/* Drives every exported routine of the CPU oracle (oracle/oracle.c) once on
 * small ragged shapes, with exact-size heap buffers, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer reports any out-of-bounds
 * access or undefined operation.  Test infrastructure only: built and run by
 * tests/test_oracle_sanitize_cpu.py.  Prints one checksum line. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e4m3_value(int code);
uint8_t orc_e4m3_encode(float y);
void orc_e4m3_encode_array(const float *y, int64_t n, uint8_t *out);
void orc_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s);
void orc_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s);
void orc_quant_act_1x128_pow2(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s);
void orc_quant_weight_128x128_pow2(const uint16_t *w, int64_t N, int64_t K, uint8_t *q,
                                   float *s);
void orc_quant_act_128x1_t(const uint16_t *x, int64_t M, int64_t K, uint8_t *q_t,
                           float *scales_t);
void orc_block_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qw,
                         const float *sw, int64_t M, int64_t N, int64_t K,
                         const int64_t *rows, int64_t nrows, double *R);
void orc_rowscaled_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qb,
                             const float *sb, int64_t M, int64_t N, int64_t K,
                             const int64_t *rows, int64_t nrows, double *R);
void orc_grouped_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qw,
                           const float *sw, const int32_t *off, int64_t E, int64_t T,
                           int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                           double *R, int32_t *found);
int orc_max_threads(void);
void orc_set_threads(int n);

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state;
}

/* bf16 bit patterns: mostly moderate normals of either sign, with zeros,
 * negative zeros, subnormals and the largest finite values mixed in */
static uint16_t *bf16_buffer(int64_t n) {
    uint16_t *p = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint16_t));
    int64_t i;
    for (i = 0; i < n; ++i) {
        uint32_t r = next_u32();
        switch (r % 16) {
            case 0: p[i] = 0x0000; break;
            case 1: p[i] = 0x8000; break;
            case 2: p[i] = (uint16_t)(0x0001 + (r >> 8) % 0x7F); break;
            case 3: p[i] = (r & 0x100) ? 0x7F7F : 0xFF7F; break;
            default:
                p[i] = (uint16_t)(((r >> 16) & 0x8000) | (0x3C00 + ((r >> 4) % 0x0600)));
        }
    }
    return p;
}

static double checksum_u8(const uint8_t *p, int64_t n) {
    double s = 0;
    int64_t i;
    for (i = 0; i < n; ++i) s += (double)p[i] * (double)(i % 7 + 1);
    return s;
}

static double checksum_f(const float *p, int64_t n) {
    double s = 0;
    int64_t i;
    for (i = 0; i < n; ++i) s += (double)p[i];
    return s;
}

static double checksum_d(const double *p, int64_t n) {
    double s = 0;
    int64_t i;
    for (i = 0; i < n; ++i) s += p[i];
    return s;
}

int main(void) {
    const int64_t M = 3, K = 200, N = 130, G = 2, NB = 2;
    const int64_t E = 3, T = 7;
    double total = 0;
    int c;
    int64_t i;

    orc_set_threads(1);
    total += orc_max_threads();

    for (c = 0; c < 256; ++c) {
        double v = orc_e4m3_value(c);
        if (v == v) total += v;  /* NaN codes are skipped */
    }
    {
        const int64_t n = 1000;
        float *y = (float *)malloc((size_t)n * sizeof(float));
        uint8_t *o = (uint8_t *)malloc((size_t)n);
        for (i = 0; i < n; ++i) y[i] = ((float)(int32_t)(next_u32() % 2001) - 1000.0f) * 0.448f;
        orc_e4m3_encode_array(y, n, o);
        total += checksum_u8(o, n) + orc_e4m3_encode(-0.0f) + orc_e4m3_encode(448.0f);
        free(y);
        free(o);
    }

    {
        uint16_t *x = bf16_buffer(M * K);
        uint16_t *w = bf16_buffer(N * K);
        uint8_t *qa = (uint8_t *)malloc((size_t)(M * K));
        float *sa = (float *)malloc((size_t)(M * G) * sizeof(float));
        uint8_t *qw = (uint8_t *)malloc((size_t)(N * K));
        float *sw = (float *)malloc((size_t)(NB * G) * sizeof(float));
        uint8_t *qb = (uint8_t *)malloc((size_t)(N * K));
        float *sb = (float *)malloc((size_t)(N * G) * sizeof(float));
        int64_t rows[2] = {0, M - 1};
        double *R = (double *)malloc((size_t)(2 * N) * sizeof(double));

        orc_quant_act_1x128_pow2(x, M, K, qa, sa);
        orc_quant_weight_128x128_pow2(w, N, K, qw, sw);
        total += checksum_u8(qa, M * K) + checksum_f(sa, M * G);
        total += checksum_u8(qw, N * K) + checksum_f(sw, NB * G);

        orc_quant_act_1x128(x, M, K, qa, sa);
        orc_quant_weight_128x128(w, N, K, qw, sw);
        total += checksum_u8(qa, M * K) + checksum_f(sa, M * G);
        total += checksum_u8(qw, N * K) + checksum_f(sw, NB * G);

        orc_block_gemm_rows(qa, sa, qw, sw, M, N, K, rows, 2, R);
        total += checksum_d(R, 2 * N) * 1e-30;

        orc_quant_act_1x128(w, N, K, qb, sb);  /* W rows with per-row scales */
        orc_rowscaled_gemm_rows(qa, sa, qb, sb, M, N, K, rows, 2, R);
        total += checksum_d(R, 2 * N) * 1e-30;
        free(x); free(w); free(qa); free(sa); free(qw); free(sw); free(qb); free(sb); free(R);
    }

    {
        const int64_t Mt = 130, Kt = 5, GM = 2;
        uint16_t *x = bf16_buffer(Mt * Kt);
        uint8_t *qt = (uint8_t *)malloc((size_t)(Kt * Mt));
        float *st = (float *)malloc((size_t)(Kt * GM) * sizeof(float));
        orc_quant_act_128x1_t(x, Mt, Kt, qt, st);
        total += checksum_u8(qt, Kt * Mt) + checksum_f(st, Kt * GM);
        free(x); free(qt); free(st);
    }

    {
        int32_t off[4] = {0, 2, 2, 7};  /* expert 1 empty */
        uint16_t *x = bf16_buffer(T * K);
        uint16_t *w = bf16_buffer(E * N * K);
        uint8_t *qa = (uint8_t *)malloc((size_t)(T * K));
        float *sa = (float *)malloc((size_t)(T * G) * sizeof(float));
        uint8_t *qw = (uint8_t *)malloc((size_t)(E * N * K));
        float *sw = (float *)malloc((size_t)(E * NB * G) * sizeof(float));
        int64_t rows[T];
        double *R = (double *)malloc((size_t)(T * N) * sizeof(double));
        int32_t found[T];
        orc_quant_act_1x128(x, T, K, qa, sa);
        for (i = 0; i < E; ++i)
            orc_quant_weight_128x128(w + i * N * K, N, K, qw + i * N * K, sw + i * NB * G);
        for (i = 0; i < T; ++i) rows[i] = i;
        memset(R, 0, (size_t)(T * N) * sizeof(double));
        orc_grouped_gemm_rows(qa, sa, qw, sw, off, E, T, N, K, rows, T, R, found);
        for (i = 0; i < T; ++i) total += found[i];
        total += checksum_d(R, T * N) * 1e-30;
        free(x); free(w); free(qa); free(sa); free(qw); free(sw); free(R);
    }

    printf("oracle sanitize driver ok: checksum %.17g\n", total);
    return 0;
}
