/*
 * Drives every entry point of oracle/oracle.c once on small inputs (including
 * the data-error paths: invalid expert ids, all-zero blocks, empty batches), so
 * that a build of the oracle with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitize.py) checks its memory accesses and integer
 * arithmetic.  Exits 0 when every call returned as documented.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_half_to_double(uint16_t h);
double oracle_bf16_to_double(uint16_t b);
double oracle_e4m3_to_double(uint8_t c);
double oracle_e2m1_to_double(uint8_t c);
double oracle_ue8m0_to_double(uint8_t s);
int64_t oracle_row_bytes(int fmt, int64_t K);
int64_t oracle_matrix_bytes(int fmt, int64_t N, int64_t K);
int oracle_dequant(int fmt, const uint8_t *W, int64_t N, int64_t K, double *out);
void oracle_quantize_act_q8(const float *x, int64_t M, int64_t K, int8_t *qx, float *dx, int32_t *sx);
int oracle_gemv(int fmt, const uint8_t *W, int64_t N, int64_t K, const int8_t *qx, const float *dx, int64_t M,
                double *y, double *bound, int nthreads);
int oracle_gemv_fx(int fmt, const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M, double *y,
                   double *bound, int nthreads);
int oracle_block_isums(int fmt, const uint8_t *W, int64_t N, int64_t K, const int8_t *qx, int64_t M, int32_t *isum);
int oracle_moe_table(const int32_t *ids, int64_t T, int64_t topk, int64_t E, int32_t *uniq, int32_t *n_uniq,
                     int32_t *slot, int32_t *pair_off, int32_t *pairs, int32_t *status);
double oracle_silu(double z);
int oracle_moe_routed_fmt(int fmt, const int8_t *qx, const float *dx, int64_t T, int64_t D, int64_t F, int64_t E,
                          int64_t topk, const int32_t *ids, const float *rw, const uint8_t *const *gate,
                          const uint8_t *const *up, const uint8_t *const *down, double *y, double *bound,
                          int32_t *status, int nthreads);
int oracle_prefill(int fmt, const uint8_t *W, int64_t N, int64_t K, const uint16_t *xbf16, int64_t M, double *Y,
                   double *bound, int nthreads);
int oracle_max_threads(void);

static uint64_t s_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    s_state ^= s_state << 13;
    s_state ^= s_state >> 7;
    s_state ^= s_state << 17;
    return (uint32_t)(s_state >> 32);
}

/* random bytes for a matrix; every fp16 / UE8M0 scale field made finite */
static uint8_t *matrix(int fmt, int64_t N, int64_t K) {
    const int64_t nb = oracle_matrix_bytes(fmt, N, K);
    uint8_t *w = (uint8_t *)malloc((size_t)nb);
    for (int64_t i = 0; i < nb; ++i) w[i] = (uint8_t)rnd();
    if (fmt == 0) { /* Q8_0: fp16 scale at the head of each 34-byte block */
        for (int64_t b = 0; b < N * K / 32; ++b) w[34 * b + 1] = (uint8_t)(0x18 | (w[34 * b + 1] & 0x03));
    } else if (fmt == 1) { /* Q4_K: fp16 d, dmin at the head of each 144-byte superblock */
        for (int64_t s = 0; s < N * K / 256; ++s) {
            w[144 * s + 1] = (uint8_t)(0x18 | (w[144 * s + 1] & 0x03));
            w[144 * s + 3] = (uint8_t)(0x18 | (w[144 * s + 3] & 0x03));
        }
    } else { /* FP8 / FP4: no NaN code (E4M3 S.1111.111); scales after the codes in 118..125 */
        const int64_t codes = fmt == 2 ? N * K : N * K / 2;
        if (fmt == 2)
            for (int64_t i = 0; i < codes; ++i)
                if ((w[i] & 0x7F) == 0x7F) w[i] ^= 1;
        for (int64_t i = (codes + 255) / 256 * 256; i < nb; ++i) w[i] = (uint8_t)(118 + (w[i] & 7));
    }
    return w;
}

static int fails = 0;
#define EXPECT(c)                                                      \
    do {                                                               \
        if (!(c)) {                                                    \
            fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #c); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

int main(void) {
    for (uint32_t h = 0; h < 65536; ++h) {
        (void)oracle_half_to_double((uint16_t)h);
        (void)oracle_bf16_to_double((uint16_t)h);
    }
    for (int c = 0; c < 256; ++c) {
        (void)oracle_e4m3_to_double((uint8_t)c);
        (void)oracle_e2m1_to_double((uint8_t)(c & 15));
        (void)oracle_ue8m0_to_double((uint8_t)c);
    }
    EXPECT(oracle_max_threads() >= 1);
    const int64_t M = 3, N = 5, K = 512;
    float *x = (float *)malloc(sizeof(float) * M * K);
    for (int64_t i = 0; i < M * K; ++i) x[i] = ((float)(int32_t)rnd() / 2147483648.0f) * 3.0f;
    for (int64_t i = 0; i < 32; ++i) x[K + i] = 0.0f;      /* an all-zero block */
    x[2 * K + 40] = 1e-40f;                                 /* a subnormal */
    int8_t *qx = (int8_t *)malloc((size_t)(M * K));
    float *dx = (float *)malloc(sizeof(float) * M * K / 32);
    int32_t *sx = (int32_t *)malloc(sizeof(int32_t) * M * K / 32);
    oracle_quantize_act_q8(x, M, K, qx, dx, sx);
    oracle_quantize_act_q8(x, 0, K, qx, dx, sx);
    double *y = (double *)malloc(sizeof(double) * M * 4096);
    double *bound = (double *)malloc(sizeof(double) * M * 4096);
    for (int fmt = 0; fmt < 4; ++fmt) {
        uint8_t *W = matrix(fmt, N, K);
        double *deq = (double *)malloc(sizeof(double) * N * K);
        EXPECT(oracle_dequant(fmt, W, N, K, deq) == 0);
        EXPECT(oracle_gemv(fmt, W, N, K, qx, dx, M, y, bound, 2) == 0);
        EXPECT(oracle_gemv(fmt, W, N, K, qx, dx, 0, y, NULL, 2) == 0);
        EXPECT(oracle_gemv_fx(fmt, W, N, K, x, M, y, bound, 2) == 0);
        if (fmt < 2) {
            int32_t *is = (int32_t *)malloc(sizeof(int32_t) * M * N * K / 32);
            EXPECT(oracle_block_isums(fmt, W, N, K, qx, M, is) == 0);
            free(is);
            uint16_t *xb = (uint16_t *)malloc(sizeof(uint16_t) * M * K);
            for (int64_t i = 0; i < M * K; ++i) {
                uint32_t u;
                memcpy(&u, &x[i], 4);
                xb[i] = (uint16_t)(u >> 16);
            }
            EXPECT(oracle_prefill(fmt, W, N, K, xb, M, y, bound, 2) == 0);
            free(xb);
        }
        EXPECT(oracle_gemv(fmt, W, N, 300, qx, dx, M, y, bound, 1) != 0); /* K not a multiple of 256 */
        free(deq);
        free(W);
    }
    /* routed MoE: E experts, ids with duplicates and invalid entries */
    const int64_t T = 3, topk = 3, E = 5, D = 256, F = 256;
    const int32_t ids[9] = {4, 1, 4, -1, 2, 0, 7, 1, 3};
    int32_t uniq[9], nuniq = 0, slot[9], off[10], pairs[9], status = 0;
    EXPECT(oracle_moe_table(ids, T, topk, E, uniq, &nuniq, slot, off, pairs, &status) == 0);
    EXPECT(status != 0 && nuniq == 5);
    float rw[9];
    for (int i = 0; i < 9; ++i) rw[i] = 1.0f / 3.0f;
    float *xm = (float *)malloc(sizeof(float) * T * D);
    for (int64_t i = 0; i < T * D; ++i) xm[i] = (float)(int32_t)rnd() / 2147483648.0f;
    int8_t *mq = (int8_t *)malloc((size_t)(T * D));
    float *md = (float *)malloc(sizeof(float) * T * D / 32);
    int32_t *ms = (int32_t *)malloc(sizeof(int32_t) * T * D / 32);
    oracle_quantize_act_q8(xm, T, D, mq, md, ms);
    for (int fmt = 1; fmt < 4; ++fmt) {
        const uint8_t *gate[5], *up[5], *down[5];
        uint8_t *own[15];
        for (int e = 0; e < E; ++e) {
            gate[e] = own[3 * e] = matrix(fmt, F, D);
            up[e] = own[3 * e + 1] = matrix(fmt, F, D);
            down[e] = own[3 * e + 2] = matrix(fmt, D, F);
        }
        status = 0;
        EXPECT(oracle_moe_routed_fmt(fmt, mq, md, T, D, F, E, topk, ids, rw, gate, up, down, y, bound, &status, 2) ==
               0);
        EXPECT(status != 0);
        for (int i = 0; i < 15; ++i) free(own[i]);
    }
    EXPECT(oracle_silu(-800.0) == -0.0 || oracle_silu(-800.0) == 0.0);
    free(x), free(qx), free(dx), free(sx), free(y), free(bound), free(xm), free(mq), free(md), free(ms);
    if (fails) return 1;
    printf("ORACLE_SANITIZE_OK\n");
    return 0;
}
