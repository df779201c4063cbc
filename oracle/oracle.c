/*
 * oracle.c -- plain, slow CPU oracle for the block-quantized decode mat-vec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under routed_moe_matvec_amd/) never calls it, and the two
 * share no code, headers, tables or helpers.
 *
 * What it computes, and where that is defined:
 *
 *   - Prequantized Q8 decode: the decode activation is quantized to 8-bit
 *     blocks once and every Q8_0 projection consumes those blocks
 *     ("ROCm: restore DeepSeek V4 Flash decode performance and Q4 SSD
 *     streaming", antirez/ds4 pull request 623, Summary; the per-stage table in
 *     the review comments names the Q8_0 entry points).
 *   - Q4_K dense projections ("Support AProjQ4 GGUFs: Q4_K dense attention
 *     projections ...", antirez/ds4 pull request 621, section 1 and the
 *     executive summary) and the Q4_K routed experts of the distributed model
 *     in pull request 623 (Tested models; 13.50 MiB per expert in the SSD
 *     streaming log of the review comments).
 *   - Routed MoE with a compact selected-expert table staged before the
 *     pointer-backed launch (pull request 623, Summary and Correctness), with
 *     sigmoid-normalized top-6 routing (ROCm/ATOM "DeepSeek-V4 Usage Guide",
 *     opening paragraph and MoE tips).
 *   - The dequantize-then-GEMM prefill path (pull request 621, the CUDA / GB10
 *     prefill discussion).
 *
 * Every floating-point result is the plain definition written out: each
 * weight block is dequantized on its own and products are accumulated in
 * double precision, row by row, in index order.  The one exception is the
 * activation quantizer, whose output is *defined* by fp32 rounding (scale =
 * absmax/127 on an fp32 activation, round half to even), so it is written in
 * fp32 exactly as that definition reads.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off (no fast-math), x86-64
 * SSE arithmetic, so every float operation is a single IEEE-754 rounding.
 *
 * Formats (the pages name them but print no byte layout; the layout below is
 * this library's own, see the header of the public C interface for the same
 * statement from the product side):
 *
 *   Q8_0 block, 34 bytes, 32 weights:
 *     bytes 0..1   fp16 scale d (little endian)
 *     bytes 2..33  int8 quants q[0..31]
 *     weight i = d * q[i]
 *   A row of K weights is K/32 consecutive blocks; rows are consecutive.
 *
 *   Q4_K-style superblock, 144 bytes, 256 weights in 8 sub-blocks of 32:
 *     bytes 0..1    fp16 d
 *     bytes 2..3    fp16 dmin
 *     bytes 4..15   sixteen 6-bit fields read as one little-endian 96-bit
 *                   string; field f occupies bits [6f, 6f+6).  Fields 0..7
 *                   are the sub-block scales sc[j], fields 8..15 the sub-block
 *                   mins m[j].
 *     bytes 16..143 4-bit quants.  Sub-blocks 2p and 2p+1 (p = 0..3) share the
 *                   32 bytes 16+32p .. 16+32p+31: element i of sub-block 2p is
 *                   the low nibble of byte 16+32p+i, element i of sub-block
 *                   2p+1 is the high nibble of the same byte.
 *     weight (j, i) = d * sc[j] * q - dmin * m[j]
 *   A row of K weights is K/256 consecutive superblocks.
 *
 *   FP8 E4M3 with 128 x 128 block scales, and FP4 E2M1 with 1 x 32
 *   microscaling, both with UE8M0 scales (the routed-expert formats of
 *   ROCm/ATOM "DeepSeek-V4 Usage Guide", section "FP8 on MI308 / gfx942":
 *   its quantization-config table and the V4-Pro MoE backend note).  One
 *   matrix of N rows and K columns is one buffer: the codes, then, from the
 *   first multiple of 256 bytes after them, the scale bytes, then zeros up to
 *   a multiple of 16 bytes (matrices stored back to back stay 16-byte aligned).
 *     FP8: codes uint8 [N][K]; scales [ceil(N/128)][K/128];
 *          weight (n, k) = e4m3(code) * 2^(S[n/128][k/128] - 127).
 *     FP4: codes uint8 [N][K/2], element 2i in the low nibble of byte i and
 *          element 2i+1 in the high nibble; scales [N][K/32];
 *          weight (n, k) = e2m1(nibble) * 2^(S[n][k/32] - 127).
 *   E4M3 (OCP 8-bit float, no infinities): sign, 4 exponent bits (bias 7),
 *   3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN.  E2M1 (OCP
 *   4-bit float): sign, 2 exponent bits (bias 1), 1 mantissa bit.  UE8M0:
 *   an unsigned 8-bit exponent, 2^(s - 127), 255 being NaN.
 *
 *   Q8 activation (per row of K fp32 values, per block b of 32):
 *     qx int8[K], dx fp32[K/32] (the block scale), sx int32[K/32] (sum of
 *     the block's quants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_FMT_Q8_0 0
#define ORACLE_FMT_Q4K 1
#define ORACLE_FMT_FP8_B128 2
#define ORACLE_FMT_FP4_MX 3

#define ORACLE_OK 0
#define ORACLE_ERR_ARG -1
#define ORACLE_ERR_NOMEM -2

/* device-status style codes for data errors found in the expert ids */
#define ORACLE_BAD_EXPERT 1

/* ------------------------------------------------------------------ */
/* scalar decoders                                                      */
/* ------------------------------------------------------------------ */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: (f / 2^10) * 2^-14 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE-754 binary32. */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3: sign, exponent e (4 bits, bias 7), mantissa m (3 bits).
 * e == 0: (m / 8) * 2^-6;  otherwise (1 + m / 8) * 2^(e - 7);  e == 15 with
 * m == 7 is NaN (the format has no infinities). */
double oracle_e4m3_to_double(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* OCP FP4 E2M1 (the low 4 bits of c): sign, exponent e (2 bits, bias 1),
 * mantissa m (1 bit).  e == 0: m / 2;  otherwise (1 + m / 2) * 2^(e - 1). */
double oracle_e2m1_to_double(uint8_t c) {
    int sign = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * (double)m : ldexp((double)(2 + m), e - 2);
    return sign ? -v : v;
}

/* UE8M0 scale: 2^(s - 127); s == 255 is NaN. */
double oracle_ue8m0_to_double(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

static uint16_t load_u16_le(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* field f (0..15) of the 96-bit little-endian string held in bytes[0..11] */
static int q4k_field(const uint8_t *bytes, int f) {
    int v = 0;
    for (int bit = 0; bit < 6; ++bit) {
        int pos = 6 * f + bit;
        int b = (bytes[pos / 8] >> (pos % 8)) & 1;
        v |= b << bit;
    }
    return v;
}

int64_t oracle_row_bytes(int fmt, int64_t K) {
    if (fmt == ORACLE_FMT_Q8_0) return (K / 32) * 34;
    if (fmt == ORACLE_FMT_Q4K) return (K / 256) * 144;
    if (fmt == ORACLE_FMT_FP8_B128) return K; /* codes only */
    if (fmt == ORACLE_FMT_FP4_MX) return K / 2;
    return -1;
}

static int is_scaled_fmt(int fmt) { return fmt == ORACLE_FMT_FP8_B128 || fmt == ORACLE_FMT_FP4_MX; }

/* Byte offset of the scales of an FP8 / FP4 matrix: the codes rounded up to 256. */
static int64_t scale_offset(int fmt, int64_t N, int64_t K) {
    int64_t codes = N * oracle_row_bytes(fmt, K);
    return (codes + 255) / 256 * 256;
}

/* Bytes of a whole N x K matrix in format fmt (codes and, for FP8 / FP4,
 * scales, the buffer rounded up to a multiple of 16 bytes). */
int64_t oracle_matrix_bytes(int fmt, int64_t N, int64_t K) {
    int64_t end;
    if (fmt == ORACLE_FMT_FP8_B128) end = scale_offset(fmt, N, K) + (N + 127) / 128 * (K / 128);
    else if (fmt == ORACLE_FMT_FP4_MX) end = scale_offset(fmt, N, K) + N * (K / 32);
    else return N * oracle_row_bytes(fmt, K);
    return (end + 15) / 16 * 16;
}

/* Dequantize the 32 weights of block b (0 .. K/32-1) of one row into w[32]. */
static void dequant_block(int fmt, const uint8_t *row, int64_t b, double *w) {
    if (fmt == ORACLE_FMT_Q8_0) {
        const uint8_t *blk = row + 34 * b;
        double d = oracle_half_to_double(load_u16_le(blk));
        for (int i = 0; i < 32; ++i) w[i] = d * (double)(int8_t)blk[2 + i];
    } else {
        int64_t s = b / 8; /* superblock */
        int j = (int)(b % 8); /* sub-block within it */
        const uint8_t *sb = row + 144 * s;
        double d = oracle_half_to_double(load_u16_le(sb));
        double dmin = oracle_half_to_double(load_u16_le(sb + 2));
        int sc = q4k_field(sb + 4, j);
        int m = q4k_field(sb + 4, 8 + j);
        const uint8_t *qs = sb + 16 + 32 * (j / 2);
        for (int i = 0; i < 32; ++i) {
            int q = (j % 2 == 0) ? (qs[i] & 0x0f) : (qs[i] >> 4);
            w[i] = d * (double)sc * (double)q - dmin * (double)m;
        }
    }
}

/* Block b (32 weights) of row n of matrix W (N x K), any format, into w[32]. */
static void dequant_row_block(int fmt, const uint8_t *W, int64_t N, int64_t K, int64_t n, int64_t b, double *w) {
    if (fmt == ORACLE_FMT_FP8_B128) {
        const uint8_t *codes = W + n * K + 32 * b;
        double scale = oracle_ue8m0_to_double(W[scale_offset(fmt, N, K) + (n / 128) * (K / 128) + (32 * b) / 128]);
        for (int i = 0; i < 32; ++i) w[i] = oracle_e4m3_to_double(codes[i]) * scale;
    } else if (fmt == ORACLE_FMT_FP4_MX) {
        const uint8_t *codes = W + n * (K / 2) + 16 * b;
        double scale = oracle_ue8m0_to_double(W[scale_offset(fmt, N, K) + n * (K / 32) + b]);
        for (int i = 0; i < 32; ++i) {
            uint8_t byte = codes[i / 2];
            uint8_t nib = (i % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
            w[i] = oracle_e2m1_to_double(nib) * scale;
        }
    } else {
        dequant_block(fmt, W + n * oracle_row_bytes(fmt, K), b, w);
    }
}

/* Raw integer quant of block b, element i (int8 for Q8_0, nibble 0..15 for Q4_K). */
static int raw_quant(int fmt, const uint8_t *row, int64_t b, int i) {
    if (fmt == ORACLE_FMT_Q8_0) return (int8_t)row[34 * b + 2 + i];
    int64_t s = b / 8;
    int j = (int)(b % 8);
    const uint8_t *qs = row + 144 * s + 16 + 32 * (j / 2);
    return (j % 2 == 0) ? (qs[i] & 0x0f) : (qs[i] >> 4);
}

static int fmt_ok(int fmt, int64_t K) {
    if (fmt == ORACLE_FMT_Q8_0) return K > 0 && K % 32 == 0;
    if (fmt == ORACLE_FMT_Q4K) return K > 0 && K % 256 == 0;
    if (fmt == ORACLE_FMT_FP8_B128) return K > 0 && K % 128 == 0;
    if (fmt == ORACLE_FMT_FP4_MX) return K > 0 && K % 32 == 0;
    return 0;
}

/* Full dequantized matrix, out[N*K] row-major. */
int oracle_dequant(int fmt, const uint8_t *W, int64_t N, int64_t K, double *out) {
    if (!fmt_ok(fmt, K) || N < 0) return ORACLE_ERR_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < K / 32; ++b) dequant_row_block(fmt, W, N, K, n, b, out + n * K + 32 * b);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* activation quantization (fp32 by definition)                          */
/* ------------------------------------------------------------------ */

/*
 * Per block of 32 fp32 values: amax = max |x|; d = amax / 127 (one fp32
 * division, round to nearest even); q = round-half-to-even(fl32(x / d)),
 * clamped to [-127, 127]; d == 0 gives q = 0.  s = sum of q.
 */
void oracle_quantize_act_q8(const float *x, int64_t M, int64_t K, int8_t *qx, float *dx, int32_t *sx) {
    int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + m * K + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            int32_t s = 0;
            for (int i = 0; i < 32; ++i) {
                int q = 0;
                if (d != 0.0f) {
                    float r = xb[i] / d;
                    float qr = rintf(r); /* default rounding mode: half to even */
                    if (qr > 127.0f) qr = 127.0f;
                    if (qr < -127.0f) qr = -127.0f;
                    q = (int)qr;
                }
                qx[m * K + 32 * b + i] = (int8_t)q;
                s += q;
            }
            dx[m * nb + b] = d;
            sx[m * nb + b] = s;
        }
    }
}

/* ------------------------------------------------------------------ */
/* mat-vec                                                              */
/* ------------------------------------------------------------------ */

/*
 * y[m, n] = sum_k w[n, k] * (dx[m, k/32] * qx[m, k])   in fp64,
 * bound[m, n] = sum_k |w[n, k] * dx[m, k/32] * qx[m, k]|.
 * Weights are dequantized one 32-block at a time.  bound may be NULL.
 */
int oracle_gemv(int fmt, const uint8_t *W, int64_t N, int64_t K, const int8_t *qx, const float *dx, int64_t M,
                double *y, double *bound, int nthreads) {
    if (!fmt_ok(fmt, K) || N < 0 || M < 0) return ORACLE_ERR_ARG;
    int64_t nb = K / 32;
    int err = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        double *acc = (double *)calloc((size_t)(M > 0 ? M : 1) * 2, sizeof(double));
        if (!acc) {
#pragma omp atomic write
            err = 1;
        } else {
            double *bnd = acc + (M > 0 ? M : 1);
#pragma omp for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                double w[32];
                for (int64_t m = 0; m < M; ++m) acc[m] = bnd[m] = 0.0;
                for (int64_t b = 0; b < nb; ++b) {
                    dequant_row_block(fmt, W, N, K, n, b, w);
                    for (int64_t m = 0; m < M; ++m) {
                        double scale = (double)dx[m * nb + b];
                        const int8_t *q = qx + m * K + 32 * b;
                        for (int i = 0; i < 32; ++i) {
                            double t = w[i] * (scale * (double)q[i]);
                            acc[m] += t;
                            bnd[m] += fabs(t);
                        }
                    }
                }
                for (int64_t m = 0; m < M; ++m) {
                    y[m * N + n] = acc[m];
                    if (bound) bound[m * N + n] = bnd[m];
                }
            }
            free(acc);
        }
    }
    return err ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * The fp32-activation product kept as the exact-activation ("quality")
 * comparator of the prequantized path (pull request 623, Summary: the shared-x
 * fp32 path that prequantization replaced):
 * y[m, n] = sum_k w[n, k] * x[m, k]   in fp64, x taken as the given fp32 values,
 * bound[m, n] = sum_k |w[n, k] * x[m, k]|.  bound may be NULL.
 */
int oracle_gemv_fx(int fmt, const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M, double *y,
                   double *bound, int nthreads) {
    if (!fmt_ok(fmt, K) || N < 0 || M < 0) return ORACLE_ERR_ARG;
    int64_t nb = K / 32;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, bnd = 0.0;
            double w[32];
            for (int64_t b = 0; b < nb; ++b) {
                dequant_row_block(fmt, W, N, K, n, b, w);
                for (int i = 0; i < 32; ++i) {
                    double t = w[i] * (double)x[m * K + 32 * b + i];
                    acc += t;
                    bnd += fabs(t);
                }
            }
            y[m * N + n] = acc;
            if (bound) bound[m * N + n] = bnd;
        }
    }
    return ORACLE_OK;
}

/*
 * Per-block integer dot products of the raw quants with the activation quants:
 * isum[m, n, b] = sum_{i<32} q_w[n, b, i] * qx[m, 32b + i]
 * (Q8_0: q_w is the int8 quant; Q4_K: q_w is the 4-bit quant 0..15 of
 * sub-block b).  Exact in int32: |isum| <= 32*127*127 (Q8_0), 32*15*127 (Q4_K).
 */
int oracle_block_isums(int fmt, const uint8_t *W, int64_t N, int64_t K, const int8_t *qx, int64_t M, int32_t *isum) {
    if (!fmt_ok(fmt, K) || is_scaled_fmt(fmt) || N < 0 || M < 0) return ORACLE_ERR_ARG;
    int64_t rb = oracle_row_bytes(fmt, K);
    int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i) s += raw_quant(fmt, W + n * rb, b, i) * (int32_t)qx[m * K + 32 * b + i];
                isum[(m * N + n) * nb + b] = s;
            }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* routed MoE                                                           */
/* ------------------------------------------------------------------ */

/*
 * Compact selected-expert table for P = T*topk (token, slot) pairs,
 * pair p = t*topk + k:
 *   uniq[0..U)      distinct valid expert ids, ascending
 *   *n_uniq         U
 *   slot[p]         index of ids[p] in uniq, or -1 for an invalid id
 *   pair_off[0..U]  CSR offsets: pairs of uniq[u] are pairs[pair_off[u] .. pair_off[u+1])
 *   pairs[]         pair indices grouped by expert, ascending p within a group
 *   *status         0, or ORACLE_BAD_EXPERT if any id is outside [0, E)
 * An id outside [0, E) is a data error (the pages show a decode that fails on
 * an expert id of -1, out of the range 0..256); such a pair belongs to no expert.
 */
int oracle_moe_table(const int32_t *ids, int64_t T, int64_t topk, int64_t E, int32_t *uniq, int32_t *n_uniq,
                     int32_t *slot, int32_t *pair_off, int32_t *pairs, int32_t *status) {
    if (T < 0 || topk < 1 || E < 1) return ORACLE_ERR_ARG;
    int64_t P = T * topk;
    int32_t *rank = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!rank || !fill) {
        free(rank);
        free(fill);
        return ORACLE_ERR_NOMEM;
    }
    *status = 0;
    for (int64_t e = 0; e < E; ++e) rank[e] = -1;
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = ids[p];
        if (e < 0 || e >= E)
            *status = ORACLE_BAD_EXPERT;
        else
            rank[e] = 0; /* mark present */
    }
    int32_t U = 0;
    for (int64_t e = 0; e < E; ++e)
        if (rank[e] >= 0) {
            rank[e] = U;
            uniq[U++] = (int32_t)e;
        }
    *n_uniq = U;
    for (int32_t u = 0; u <= U; ++u) pair_off[u] = 0;
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = ids[p];
        slot[p] = (e < 0 || e >= E) ? -1 : rank[e];
        if (slot[p] >= 0) pair_off[slot[p] + 1] += 1;
    }
    for (int32_t u = 0; u < U; ++u) pair_off[u + 1] += pair_off[u];
    for (int32_t u = 0; u < U; ++u) fill[u] = pair_off[u];
    for (int64_t p = 0; p < P; ++p)
        if (slot[p] >= 0) pairs[fill[slot[p]]++] = (int32_t)p;
    free(rank);
    free(fill);
    return ORACLE_OK;
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * End-to-end routed MoE for T tokens, from scratch:
 *   for every valid pair (t, k) with e = ids[t, k]:
 *     g = gate_e . x_t, v = up_e . x_t            (fp64, on the Q8 activation)
 *     h = silu(g) * v                              (fp64)
 *     (hq, hd, hs) = Q8-quantize(fl32(h))          (the down projection consumes
 *                                                   a Q8 activation, like every
 *                                                   other projection)
 *     o = down_e . h_q                             (fp64)
 *     y_t += rw[t, k] * o,  bound_t += |rw[t, k]| * bound(o)
 * Gate/up are F x D, down is D x F, all in format fmt (Q4_K for the
 * distributed model; FP8 E4M3 128 x 128 or FP4 E2M1 1 x 32 for the ATOM
 * expert formats).  Pairs with an invalid id add nothing and set *status.
 * y, bound are [T, D].
 */
int oracle_moe_routed_fmt(int fmt, const int8_t *qx, const float *dx, int64_t T, int64_t D, int64_t F, int64_t E,
                          int64_t topk, const int32_t *ids, const float *rw, const uint8_t *const *gate,
                          const uint8_t *const *up, const uint8_t *const *down, double *y, double *bound,
                          int32_t *status, int nthreads) {
    if (T < 0 || D % 256 || F % 256 || D <= 0 || F <= 0 || E < 1 || topk < 1) return ORACLE_ERR_ARG;
    if (fmt != ORACLE_FMT_Q4K && !is_scaled_fmt(fmt)) return ORACLE_ERR_ARG;
    double *g = (double *)malloc(sizeof(double) * (size_t)F);
    double *v = (double *)malloc(sizeof(double) * (size_t)F);
    float *hf = (float *)malloc(sizeof(float) * (size_t)F);
    int8_t *hq = (int8_t *)malloc((size_t)F);
    float *hd = (float *)malloc(sizeof(float) * (size_t)(F / 32));
    int32_t *hs = (int32_t *)malloc(sizeof(int32_t) * (size_t)(F / 32));
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    double *ob = (double *)malloc(sizeof(double) * (size_t)D);
    int rc = ORACLE_OK;
    if (!g || !v || !hf || !hq || !hd || !hs || !o || !ob) {
        rc = ORACLE_ERR_NOMEM;
        goto done;
    }
    *status = 0;
    for (int64_t i = 0; i < T * D; ++i) y[i] = bound[i] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < topk; ++k) {
            int32_t e = ids[t * topk + k];
            if (e < 0 || e >= E) {
                *status = ORACLE_BAD_EXPERT;
                continue;
            }
            oracle_gemv(fmt, gate[e], F, D, qx + t * D, dx + t * (D / 32), 1, g, NULL, nthreads);
            oracle_gemv(fmt, up[e], F, D, qx + t * D, dx + t * (D / 32), 1, v, NULL, nthreads);
            for (int64_t f = 0; f < F; ++f) hf[f] = (float)(oracle_silu(g[f]) * v[f]);
            oracle_quantize_act_q8(hf, 1, F, hq, hd, hs);
            oracle_gemv(fmt, down[e], D, F, hq, hd, 1, o, ob, nthreads);
            double r = (double)rw[t * topk + k];
            for (int64_t n = 0; n < D; ++n) {
                y[t * D + n] += r * o[n];
                bound[t * D + n] += fabs(r) * ob[n];
            }
        }
    }
done:
    free(g);
    free(v);
    free(hf);
    free(hq);
    free(hd);
    free(hs);
    free(o);
    free(ob);
    return rc;
}

/* The distributed model's routed MoE: every expert matrix Q4_K. */
int oracle_moe_routed(const int8_t *qx, const float *dx, int64_t T, int64_t D, int64_t F, int64_t E, int64_t topk,
                      const int32_t *ids, const float *rw, const uint8_t *const *gate, const uint8_t *const *up,
                      const uint8_t *const *down, double *y, double *bound, int32_t *status, int nthreads) {
    return oracle_moe_routed_fmt(ORACLE_FMT_Q4K, qx, dx, T, D, F, E, topk, ids, rw, gate, up, down, y, bound, status,
                                 nthreads);
}

/* ------------------------------------------------------------------ */
/* prefill                                                              */
/* ------------------------------------------------------------------ */

/*
 * Y[m, n] = sum_k w[n, k] * x[m, k], x given as bfloat16 bits, fp64 accumulate;
 * bound[m, n] = sum_k |w[n, k] * x[m, k]|.  bound may be NULL.
 */
int oracle_prefill(int fmt, const uint8_t *W, int64_t N, int64_t K, const uint16_t *xbf16, int64_t M, double *Y,
                   double *bound, int nthreads) {
    if (!fmt_ok(fmt, K) || is_scaled_fmt(fmt) || N < 0 || M < 0) return ORACLE_ERR_ARG;
    int64_t rb = oracle_row_bytes(fmt, K);
    int64_t nb = K / 32;
    if (nthreads < 1) nthreads = 1;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xd) return ORACLE_ERR_NOMEM;
    for (int64_t i = 0; i < M * K; ++i) xd[i] = oracle_bf16_to_double(xbf16[i]);
    int err = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                /* the row, dequantized one 32-block at a time */
                for (int64_t b = 0; b < nb; ++b) dequant_block(fmt, W + n * rb, b, w + 32 * b);
                for (int64_t m = 0; m < M; ++m) {
                    double acc = 0.0, bnd = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        double t = w[k] * xd[m * K + k];
                        acc += t;
                        bnd += fabs(t);
                    }
                    Y[m * N + n] = acc;
                    if (bound) bound[m * N + n] = bnd;
                }
            }
            free(w);
        }
    }
    free(xd);
    return err ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
