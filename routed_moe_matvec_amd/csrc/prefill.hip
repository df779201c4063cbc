// Prefill: Q4_K weights x bf16 activations, dequantize then GEMM on the
// matrix cores ("Support AProjQ4 GGUFs: Q4_K dense attention projections ...",
// antirez/ds4 PR 621: the dequant + GEMM prefill path whose ~16x regression
// and recovery that page reports).
//
//   Y[m, n] = sum_k w[n, k] x[m, k],  w = d*sc_j*q - dmin*m_j  (Q4_K)
//
// Numerics: written per superblock s and sub-block j,
//   Y = sum_s ( d_s * sum_k (sc*q)_k x_k  -  dmin_s * sum_j m_j S_j ),
//   S_j = sum of the 32 activations of sub-block j.
// sc*q <= 63*15 = 945 is an integer, exact in fp16, and a bf16 activation is
// exact in fp16 once its row is scaled by a power of two 2^e that puts the
// row's largest |x| in [2^15, 2^16) (values more than 2^32 below it lose low
// bits).  So the main product runs on the fp16 MFMA with exact inputs and fp32
// accumulation, and d_s is applied per superblock in fp32.  The min term is a
// second, 32x smaller product over the sub-block sums: dmin*m (17 significant
// bits) scaled per weight row and 4-superblock window by a power of two 2^E
// into [0, 2^16), and S*2^(e-6), are each split into two fp16 halves; three
// hi/lo MFMA products give the term to ~2^-21 relative.  Every scaling is by a
// power of two and is undone exactly.  Plain bf16 or fp16 dequantization of w
// would not meet 1e-5 * sum |w x|.
//
// Two forms.
//   qgemm_prefill: 128 tokens x 128 weight rows per workgroup, four waves of
//   64 x 64, v_mfma_f32_16x16x32_f16 (A: lane l holds row l%16, k 8*(l/16)..+8;
//   B: column l%16, same k; C: rows 4*(l/16)+i, column l%16), K steps of 128.
//   Each step the workgroup dequantizes its 128 x 128 weight slice once into
//   LDS as fp16 sc*q (nibbles are widened with byte permutes into fp16 1024+q,
//   and one packed fp16 fma per pair, (1024+q)*sc - 1024*sc, gives sc*q
//   exactly) and converts the activations bf16 -> fp16 into LDS (e = 0, so it
//   needs |x| <= 65504 and loses low bits of |x| < 2^-17), with padded rows.
//   qgemm_prefill_ws: a pre-pass (one workgroup per token) finds e and writes
//   x * 2^e as fp16, and the sums of its 32-input blocks as fp16 hi + lo
//   pairs, to a caller workspace; the GEMM (eight waves, operands through
//   pipelined global -> LDS copies, weights dequantized in registers;
//   described at the kernel) reads them from there.
#include <type_traits>

#include "common.h"

namespace qg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4p __attribute__((ext_vector_type(4)));

constexpr int kPfBM = 128;         // tokens per workgroup
constexpr int kPfBN = 128;         // weight rows per workgroup
constexpr int kPfKS = 128;         // K per step: half a superblock (four sub-blocks)
constexpr int kPfLd = kPfKS + 8;   // padded LDS row, halves (68 dwords: conflict-free 16-byte reads)
constexpr int kPfWin = 4;          // superblocks per min-term window (32 sub-block sums)
constexpr int kPfSLd = 32 + 8;     // padded LDS row of the in-kernel sub-block sums, halves
constexpr int kPfSumShift = 6;     // sub-block sums are kept as S * 2^(e-6): |S| <= 32 |x|max
constexpr int kPfPreThreads = 256;

struct __attribute__((aligned(16))) PrefillLds {
    _Float16 a[kPfBM * kPfLd];      // activations, fp16
    _Float16 b[kPfBN * kPfLd];      // sc*q, fp16
    _Float16 s_hi[kPfBM * kPfSLd];  // sub-block sums of x, high half (in-kernel conversion only)
    _Float16 s_lo[kPfBM * kPfSLd];  // and the remainder
    float d[kPfBN];                 // d of the current superblock per row
};

__device__ __forceinline__ uint32_t field6(uint32_t s0, uint32_t s1, uint32_t s2, int f) {
    const int bit = 6 * f, word = bit >> 5, off = bit & 31;
    const uint32_t lo = word == 0 ? s0 : (word == 1 ? s1 : s2);
    const uint32_t hi = word == 0 ? s1 : (word == 1 ? s2 : 0u);
    return (off == 0 ? lo : ((lo >> off) | (hi << (32 - off)))) & 63u;
}

__device__ __forceinline__ float half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void split_half(float v, _Float16 &hi, _Float16 &lo) {
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);
}

// Sum of the 32 values of one sub-block in a fixed order: four consecutive
// values at a time, then a pairwise tree over the eight partial sums.
__device__ __forceinline__ float sub_block_sum(const float t[8]) {
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}
__device__ __forceinline__ float quad_sum(float a, float b, float c, float d) { return ((a + b) + c) + d; }

// Four nibble bytes (0..15 each, one per byte of nb) times sc -> two half2
// holding sc*q exactly: bytes are widened to fp16 1024+q with byte permutes
// (0x64 is the high byte of fp16 1024), then one packed fma per pair.
__device__ __forceinline__ void nibbles_to_half(uint32_t nb, half2v sc2, half2v off2, uint32_t &o0, uint32_t &o1) {
    const uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, nb, 0x04010400u);  // 1024+b0, 1024+b1
    const uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, nb, 0x04030402u);  // 1024+b2, 1024+b3
    o0 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2v, p0), sc2, off2));
    o1 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2v, p1), sc2, off2));
}

__device__ __forceinline__ uint32_t bf16x2_to_half2(uint32_t w) {
    const half2v h = {(_Float16)bf_lo(w), (_Float16)bf_hi(w)};
    return __builtin_bit_cast(uint32_t, h);
}

// Exponent e with max|x| * 2^e in [2^15, 2^16); 0 for an all-zero row.
__device__ __forceinline__ int row_exponent(float amax) {
    if (!(amax > 0.f)) return 0;
    int x;
    (void)frexpf(amax, &x);  // amax = f * 2^x, f in [0.5, 1)
    return 16 - x;
}

// ------------------------------------------------------------------ pre-pass

// One workgroup per token m: e[m], X16[m] = x * 2^e (fp16), and for every
// 32-input block b the sum S of its 32 fp16 values, stored as S * 2^-6 split
// into fp16 hi + lo: the four blocks of each 128-input step as one 16-byte
// record SS[m][b / 4] = {hi of blocks 0..3, lo of blocks 0..3}, so that the
// GEMM copies a token's step with one 16-byte read.  Each thread reads its 8-value
// chunks once (16-byte loads) and keeps them in registers for the conversion
// after the row's maximum is known; a block's four chunks sit in four
// neighbouring lanes, each chunk summed as a pairwise tree, then the four
// chunk sums as (c0 + c1) + (c2 + c3).
constexpr int kPfPreChunks = QG_MAX_K / (8 * kPfPreThreads);  // chunks per thread at most
__global__ __launch_bounds__(kPfPreThreads) void prefill_prepass_kernel(const uint16_t *__restrict__ X, int K,
                                                                        _Float16 *__restrict__ X16,
                                                                        int32_t *__restrict__ e_out,
                                                                        _Float16 *__restrict__ SS) {
    __shared__ float red[kPfPreThreads / kWave];
    const int m = blockIdx.x, tid = threadIdx.x;
    const uint16_t *xr = X + (size_t)m * K;
    uint4 v[kPfPreChunks];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kPfPreChunks; ++c) {
        const int k = 8 * (tid + c * kPfPreThreads);
        if (k < K) {
            v[c] = *reinterpret_cast<const uint4 *>(xr + k);
            const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(w[j])), fabsf(bf_hi(w[j]))));
        }
    }
    for (int o = 1; o < kWave; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < kPfPreThreads / kWave; ++i) amax = fmaxf(amax, red[i]);
    const int e = row_exponent(amax);
    if (tid == 0) e_out[m] = e;
#pragma unroll
    for (int c = 0; c < kPfPreChunks; ++c) {
        const int k = 8 * (tid + c * kPfPreThreads);
        float p = 0.0f;  // this chunk's sum (0 past the row: K / 8 chunks come in whole blocks)
        if (k < K) {
            const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
            uint32_t o[4];
            float f[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const half2v h = {(_Float16)ldexpf(bf_lo(w[j]), e), (_Float16)ldexpf(bf_hi(w[j]), e)};
                o[j] = __builtin_bit_cast(uint32_t, h);
                f[2 * j] = (float)h.x;
                f[2 * j + 1] = (float)h.y;
            }
            *reinterpret_cast<uint4 *>(X16 + (size_t)m * K + k) = make_uint4(o[0], o[1], o[2], o[3]);
            p = ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
        }
        // lanes 4i .. 4i+3 hold the block's chunks (k / 8 = tid + 256 c)
        p = p + __shfl_xor(p, 1, kWave);
        p = p + __shfl_xor(p, 2, kWave);
        if (k < K && (tid & 3) == 0) {
            const int b = k / 32;
            _Float16 *rec = SS + ((size_t)m * (K / 128) + b / 4) * 8 + b % 4;
            split_half(ldexpf(p, -kPfSumShift), rec[0], rec[4]);
        }
    }
}

// ------------------------------------------------------------------ GEMM

// Prefetch registers of one K step for one thread.
struct PfRegs {
    u32x4p x[8];  // 64 activations (fp16 or bf16)
    u32x4p hdr;   // the row's superblock header
    u32x4p q[2];  // 32 bytes of nibbles
};

__global__ __launch_bounds__(256) void qgemm_prefill_q4k_kernel(const uint8_t *__restrict__ W, int N, int K,
                                                                const uint16_t *__restrict__ X, int M,
                                                                float *__restrict__ Y) {
    __shared__ PrefillLds L;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // the wave's 64 x 64 quadrant
    const int n0 = blockIdx.x * kPfBN, m0 = blockIdx.y * kPfBM;
    const int nsb = K / 256;
    const int nsteps = 2 * nsb;
    const size_t row_bytes = (size_t)nsb * 144;

    f32x4 acc[4][4], cs[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = cs[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging role of this thread: row r (token for activations, weight row for
    // weights), part = which 64 of the step's 128 inputs / which 32 nibble bytes
    const int r = tid >> 1, part = tid & 1;
    const bool wrow_ok = n0 + r < N;
    const bool xrow_ok = m0 + r < M;
    const uint8_t *wrow = W + (size_t)(wrow_ok ? n0 + r : 0) * row_bytes;

    auto load_step = [&](int g, PfRegs &pr) {
        const int s = g >> 1, h = g & 1;
        const size_t k0 = (size_t)s * 256 + 128 * h + 64 * part;
        if (xrow_ok) {
            const u32x4p *src = reinterpret_cast<const u32x4p *>(X + (size_t)(m0 + r) * K + k0);
#pragma unroll
            for (int c = 0; c < 8; ++c) pr.x[c] = src[c];
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) pr.x[c] = u32x4p{0, 0, 0, 0};
        }
        if (wrow_ok) {
            const u32x4p *sb = reinterpret_cast<const u32x4p *>(wrow + (size_t)s * 144);
            pr.hdr = sb[0];
            pr.q[0] = sb[1 + 4 * h + 2 * part];
            pr.q[1] = sb[2 + 4 * h + 2 * part];
        } else {
            pr.hdr = u32x4p{0, 0, 0, 0};
            pr.q[0] = pr.q[1] = u32x4p{0, 0, 0, 0};
        }
    };

    PfRegs pr;
    load_step(0, pr);

    for (int g = 0; g < nsteps; ++g) {
        const int s = g >> 1, h = g & 1;
        const int q = s % kPfWin;
        // ---- stage this step's weights (dequantized) and activations into LDS
        {
            // sub-block 4h+2part: low nibbles of the 32 bytes; 4h+2part+1: high nibbles
            const int sa = 4 * h + 2 * part;
            const _Float16 fa = (_Float16)(float)field6(pr.hdr.y, pr.hdr.z, pr.hdr.w, sa);
            const _Float16 fb = (_Float16)(float)field6(pr.hdr.y, pr.hdr.z, pr.hdr.w, sa + 1);
            const half2v sca = {fa, fa}, scb = {fb, fb};
            const _Float16 oa = (_Float16)(-1024.0f * (float)fa), ob = (_Float16)(-1024.0f * (float)fb);
            const half2v offa = {oa, oa}, offb = {ob, ob};
            const uint32_t qw[8] = {pr.q[0].x, pr.q[0].y, pr.q[0].z, pr.q[0].w, pr.q[1].x, pr.q[1].y, pr.q[1].z, pr.q[1].w};
            _Float16 *brow = L.b + r * kPfLd + 64 * part;
#pragma unroll
            for (int c = 0; c < 4; ++c) {  // elements 8c .. 8c+7 of both sub-blocks
                uint32_t lo[4], hi[4];
                nibbles_to_half(qw[2 * c] & 0x0F0F0F0Fu, sca, offa, lo[0], lo[1]);
                nibbles_to_half(qw[2 * c + 1] & 0x0F0F0F0Fu, sca, offa, lo[2], lo[3]);
                nibbles_to_half((qw[2 * c] >> 4) & 0x0F0F0F0Fu, scb, offb, hi[0], hi[1]);
                nibbles_to_half((qw[2 * c + 1] >> 4) & 0x0F0F0F0Fu, scb, offb, hi[2], hi[3]);
                *reinterpret_cast<u32x4p *>(brow + 8 * c) = u32x4p{lo[0], lo[1], lo[2], lo[3]};
                *reinterpret_cast<u32x4p *>(brow + 32 + 8 * c) = u32x4p{hi[0], hi[1], hi[2], hi[3]};
            }
            if (h == 0 && part == 0) L.d[r] = half_lo(pr.hdr.x);

            _Float16 *arow = L.a + r * kPfLd + 64 * part;
            // bf16 -> fp16, and the two sub-block sums (fixed order)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float t[8];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4p v = pr.x[4 * j + c];
                    *reinterpret_cast<u32x4p *>(arow + 32 * j + 8 * c) =
                        u32x4p{bf16x2_to_half2(v.x), bf16x2_to_half2(v.y), bf16x2_to_half2(v.z), bf16x2_to_half2(v.w)};
                    t[2 * c] = quad_sum(bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y));
                    t[2 * c + 1] = quad_sum(bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w));
                }
                const int idx = r * kPfSLd + 8 * q + 4 * h + 2 * part + j;
                split_half(ldexpf(sub_block_sum(t), -kPfSumShift), L.s_hi[idx], L.s_lo[idx]);
            }
        }
        __syncthreads();
        if (g + 1 < nsteps) load_step(g + 1, pr);  // overlaps the MFMAs below

        // ---- 64 x 64 per wave: 4 x 4 tiles, four k-steps of 32
#pragma unroll
        for (int kk = 0; kk < kPfKS; kk += 32) {
            half8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const half8 *>(L.a + (64 * wm + 16 * i + (lane & 15)) * kPfLd + kk +
                                                          8 * (lane >> 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const half8 *>(L.b + (64 * wn + 16 * j + (lane & 15)) * kPfLd + kk +
                                                           8 * (lane >> 4));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    cs[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr[j], cs[i][j], 0, 0, 0);
        }

        if (h == 1) {
            // superblock done: acc += d * cs (d per weight row = column of C)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float d = L.d[64 * wn + 16 * j + (lane & 15)];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf_exact(d, cs[i][j][e], acc[i][j][e]);
                    cs[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            if (q == kPfWin - 1 || s == nsb - 1) {
                // min term over the window's superblocks sb0 .. s: the lane's k' range
                // is superblock sb0 + lane/16 (its 8 sub-blocks); later slots are zero
                const int slot = lane >> 4;
                const int sb0 = s - q;
                const bool live = slot <= q;
                const half8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
                half8 sh[4], sl[4], mh[4], ml[4];
                float fac[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int mr = 64 * wm + 16 * i + (lane & 15);
                    if (!live) {
                        sh[i] = sl[i] = zero;
                    } else {
                        sh[i] = *reinterpret_cast<const half8 *>(L.s_hi + mr * kPfSLd + 8 * slot);
                        sl[i] = *reinterpret_cast<const half8 *>(L.s_lo + mr * kPfSLd + 8 * slot);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + 64 * wn + 16 * j + (lane & 15);
                    u32x4p hd = u32x4p{0, 0, 0, 0};
                    if (live && n < N)
                        hd = *reinterpret_cast<const u32x4p *>(W + (size_t)n * row_bytes + (size_t)(sb0 + slot) * 144);
                    const float dmin = half_hi(hd.x);
                    // the window's largest dmin of row n (lanes n%16, +16, +32, +48)
                    float dmax = dmin;
                    dmax = fmaxf(dmax, __shfl_xor(dmax, 16, kWave));
                    dmax = fmaxf(dmax, __shfl_xor(dmax, 32, kWave));
                    const int E = row_exponent(dmax) - 6;  // dmin*m*2^E < 63 * 2^10
                    fac[j] = -ldexpf(1.0f, kPfSumShift - E);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float mv = ldexpf(dmin * (float)field6(hd.y, hd.z, hd.w, 8 + e), E);  // exact
                        _Float16 hi, lo;
                        split_half(mv, hi, lo);
                        mh[j][e] = hi;
                        ml[j][e] = lo;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
                        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(sh[i], mh[j], c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(sh[i], ml[j], c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(sl[i], mh[j], c, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf_exact(fac[j], c[e], acc[i][j][e]);
                    }
            }
        }
        __syncthreads();  // LDS is restaged next step
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + e;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + 64 * wn + 16 * j + (lane & 15);
                if (n < N) Y[(size_t)m * N + n] = acc[i][j][e];
            }
        }
}

// ------------------------------------------------------------------ GEMM, workspace form

// 128 tokens x 128 weight rows per workgroup of eight waves (two per SIMD, so
// one wave's copies and dequantization overlap the other's MFMAs), each wave
// the 128 tokens x 16 rows, so that every weight is dequantized by one wave
// (64 x 32 wave tiles dequantized each weight twice).  K advances 128 per step.
//
// Every global read of a step is a global -> LDS copy (global_load_lds), six
// or seven per thread, issued two steps ahead, into one of three rotating LDS
// stages:
//   * the 128 x 128 fp16 activations (from the pre-pass): rows of 16 chunks
//     of 16 bytes, chunk c of row r stored at r*16 + (c ^ (r & 15)), so the
//     16 lanes reading one operand column hit 16 different bank groups;
//   * the 128 weight rows' 64 nibble bytes of this half superblock: rows of
//     four 16-byte units, unit u of row r stored at r*4 + (u ^ ((r >> 2) & 3)),
//     so the 8-byte operand reads are conflict-free;
//   * the 128 superblock headers (d, dmin, scale fields);
// and one into the block sums of the min-term window (four superblocks, eight
// steps): the pre-pass's 16-byte records of the step's four 32-input blocks
// for the 128 tokens, stored [step in window][token], in one of two buffers by
// window parity, so the next window's copies never meet the current window's
// reads.  The headers are copied with the first half of each superblock only
// and kept in registers for the second; the header and block-sum copies take
// one 16-byte lane per row (rows sit 144 bytes or more apart: 4-byte lanes
// spread the same bytes over four times the lanes and twice the cache lines,
// 512x8192x4096 with the pre-pass: 61.5 -> 57.5 us).
// No vector register is the destination of a prefetch, so nothing makes the
// compiler wait early; the explicit waits below are the only ones on them.
// From LDS each lane takes the 8 nibble bytes of its B operand (column =
// lane % 16, k = 8 * (lane / 16) .. +8 of a sub-block: low nibbles give one
// sub-block, high nibbles the next) and dequantizes them in registers
// straight into the MFMA operand.  One barrier per step.
constexpr int kPf3Threads = 512;
constexpr int kPf3ChunkUnits = 16;    // 16-byte chunks per 128-half activation row
constexpr int kPf3Stages = 3;         // LDS stages: compute one, two in flight
// copies per thread and step: 4 activation + 1 nibble + 1 block-sum copy, and
// in the first half of a superblock (even steps) 1 header copy
constexpr int pf3_copies(int h) { return h == 0 ? 7 : 6; }
constexpr int kPfWinSteps = 2 * kPfWin;  // steps of a min-term window

struct __attribute__((aligned(16))) Prefill3Stage {
    _Float16 a[kPfBM * kPfKS];   // 32 KiB activations, swizzled
    uint8_t nib[kPfBN * 64];     // 8 KiB nibbles, swizzled
    uint32_t hdr[kPfBN * 4];     // 2 KiB headers
};

// The 8 weights of B operand (kk, lane) from 8 nibble bytes: low nibbles
// (even sub-block) when hi == 0, else high nibbles; times sc, exactly.
__device__ __forceinline__ half8 b_operand(uint2 nib, int hi, half2v sc2, half2v off2) {
    const uint32_t a = hi ? (nib.x >> 4) : nib.x;
    const uint32_t b = hi ? (nib.y >> 4) : nib.y;
    uint32_t o[4];
    nibbles_to_half(a & 0x0F0F0F0Fu, sc2, off2, o[0], o[1]);
    nibbles_to_half(b & 0x0F0F0F0Fu, sc2, off2, o[2], o[3]);
    return __builtin_bit_cast(half8, u32x4p{o[0], o[1], o[2], o[3]});
}

// s_waitcnt vmcnt(n), expcnt / lgkmcnt untouched (gfx9 encoding)
template <int n>
__device__ __forceinline__ void wait_vmem_at_most() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

__device__ __forceinline__ void global_to_lds4(const void *gsrc, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_base, 4, 0, 0);
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// would wait for every copy still in flight).  Every LDS write of the kernel
// that uses it is a global -> LDS copy waited for explicitly before the
// barrier, and every LDS read completes inside its own block; the empty asm
// statements keep the compiler from moving memory operations across it.
__device__ __forceinline__ void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// LDS reads issued together and completed inside one asm block, from base
// addresses and immediate offsets.  Written this way because the compiler,
// unable to place the global -> LDS copies in flight into the other stages,
// would otherwise wait for all of them before any LDS read; the copies are
// ordered against these reads by the explicit wait and barrier at the end of
// every step instead.
// two k-slices: for each, eight 16-byte A fragments (base a, rows 16 apart,
// +4096 bytes each) and one 8-byte nibble group (base n)
__device__ __forceinline__ void lds_read_slice2_t(uint32_t a, uint32_t n, uint32_t a2, uint32_t n2, u32x4p (&r)[16],
                                                  uint2 (&q)[2]) {
    asm volatile(
        "ds_read_b128 %0, %18\n\t"
        "ds_read_b128 %1, %18 offset:4096\n\t"
        "ds_read_b128 %2, %18 offset:8192\n\t"
        "ds_read_b128 %3, %18 offset:12288\n\t"
        "ds_read_b128 %4, %18 offset:16384\n\t"
        "ds_read_b128 %5, %18 offset:20480\n\t"
        "ds_read_b128 %6, %18 offset:24576\n\t"
        "ds_read_b128 %7, %18 offset:28672\n\t"
        "ds_read_b64 %16, %19\n\t"
        "ds_read_b128 %8, %20\n\t"
        "ds_read_b128 %9, %20 offset:4096\n\t"
        "ds_read_b128 %10, %20 offset:8192\n\t"
        "ds_read_b128 %11, %20 offset:12288\n\t"
        "ds_read_b128 %12, %20 offset:16384\n\t"
        "ds_read_b128 %13, %20 offset:20480\n\t"
        "ds_read_b128 %14, %20 offset:24576\n\t"
        "ds_read_b128 %15, %20 offset:28672\n\t"
        "ds_read_b64 %17, %21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
          "=&v"(r[15]), "=&v"(q[0]), "=&v"(q[1])
        : "v"(a), "v"(n), "v"(a2), "v"(n2)
        : "memory");
}

// sixteen 16-byte reads: base + 256 i and base + 2048 + 256 i (i < 8)
__device__ __forceinline__ void lds_read16_b128(uint32_t base, u32x4p (&r)[16]) {
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %16 offset:256\n\t"
        "ds_read_b128 %2, %16 offset:512\n\t"
        "ds_read_b128 %3, %16 offset:768\n\t"
        "ds_read_b128 %4, %16 offset:1024\n\t"
        "ds_read_b128 %5, %16 offset:1280\n\t"
        "ds_read_b128 %6, %16 offset:1536\n\t"
        "ds_read_b128 %7, %16 offset:1792\n\t"
        "ds_read_b128 %8, %16 offset:2048\n\t"
        "ds_read_b128 %9, %16 offset:2304\n\t"
        "ds_read_b128 %10, %16 offset:2560\n\t"
        "ds_read_b128 %11, %16 offset:2816\n\t"
        "ds_read_b128 %12, %16 offset:3072\n\t"
        "ds_read_b128 %13, %16 offset:3328\n\t"
        "ds_read_b128 %14, %16 offset:3584\n\t"
        "ds_read_b128 %15, %16 offset:3840\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
          "=&v"(r[15])
        : "v"(base)
        : "memory");
}

__device__ __forceinline__ void lds_read1_b128(uint32_t base, u32x4p &r0) {
    asm volatile(
        "ds_read_b128 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0)
        : "v"(base)
        : "memory");
}

// s_waitcnt vmcnt(n) lgkmcnt(0): also every LDS write of this wave is done
template <int n>
__device__ __forceinline__ void wait_vmem_lgkm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
}


// Steps run six at a time, so that a step's stage (g % 3) and half superblock
// (g % 2) are compile-time constants of the unrolled body: the compiler then
// sees that a step's LDS reads and the copies in flight into the other stages
// are disjoint and waits for nothing early.  Up to five remaining steps run
// in a guarded tail with the same property.  Copies past the last step
// re-read the last step's data, so every step of a parity issues the same
// copies (the waits count them: pf3_copies).
__global__ __launch_bounds__(kPf3Threads) void qgemm_prefill_q4k_ws_kernel(
    const uint8_t *__restrict__ W, int N, int K, int M, const _Float16 *__restrict__ X16,
    const int32_t *__restrict__ E_x, const _Float16 *__restrict__ SS, float *__restrict__ Y) {
    // three stages as three LDS objects: the compiler tells a stage's reads
    // from the copies in flight into another stage by object, not by offset
    __shared__ Prefill3Stage st0, st1, st2;
    // sums of the 32-input blocks of a min-term window, S * 2^(e-6) split into
    // fp16 hi + lo: [window parity][step in window][token] records of
    // {hi of the step's 4 blocks, lo of them}
    constexpr int kSumSlice = kPfBM * 8;  // halves of one step's records
    __shared__ __attribute__((aligned(16))) _Float16 wsum[2 * kPfWinSteps * kSumSlice];
    auto stage_ref = [&](auto sc) -> Prefill3Stage & {
        constexpr int i = decltype(sc)::value;
        if constexpr (i == 0)
            return st0;
        else if constexpr (i == 1)
            return st1;
        else
            return st2;
    };
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;  // wave: all 128 tokens x weight rows 16 wave ..
    const int n0 = blockIdx.x * kPfBN, m0 = blockIdx.y * kPfBM;
    const int nsb = K / 256;
    const int nsteps = 2 * nsb;
    const size_t row_bytes = (size_t)nsb * 144;
    const int quad = lane >> 4, l16 = lane & 15;

    // copy roles of this thread (fixed over the steps)
    const int nib_row = 16 * wave + (lane >> 2);                      // weight row whose nibbles it copies
    const int nib_unit = (lane & 3) ^ ((nib_row >> 2) & 3);           // logical 16-byte unit it fetches
    const uint8_t *nib_src = W + (size_t)min(n0 + nib_row, N - 1) * row_bytes + 16 + 16 * nib_unit;
    // lanes 0-15 of wave w copy the headers of weight rows 16 w .. (16 bytes
    // each) and the block-sum records of tokens 16 w ..; the other lanes idle
    const bool copy16 = lane < 16;
    const uint8_t *hdr_src = W + (size_t)min(n0 + 16 * wave + l16, N - 1) * row_bytes;
    const _Float16 *sum_src = SS + (size_t)min(m0 + 16 * wave + l16, M - 1) * (K / 128) * 8;

    auto issue = [&](int g, auto stage, auto hc) {
        const int gl = min(g, nsteps - 1);
        const int k0 = 128 * gl;
        Prefill3Stage &S = stage_ref(stage);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int seg = 4 * wave + i;
            const int r = 4 * seg + quad;
            const int c = l16 ^ (r & 15);  // logical chunk held by physical slot l16
            global_to_lds16(X16 + (size_t)min(m0 + r, M - 1) * K + k0 + 8 * c, S.a + seg * 64 * 8);
        }
        const int s = gl >> 1, h = gl & 1;
        global_to_lds16(nib_src + (size_t)s * 144 + 64 * h, S.nib + wave * 1024);
        if constexpr (decltype(hc)::value == 0) {
            if (copy16) global_to_lds16(hdr_src + (size_t)s * 144, S.hdr + wave * 64);
        }
        if (copy16)
            global_to_lds16(sum_src + 8 * gl,
                            wsum + (((gl / kPfWinSteps) & 1) * kPfWinSteps + gl % kPfWinSteps) * kSumSlice + wave * 128);
    };

    f32x4 acc[8], cs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = cs[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int brow = 16 * wave + l16;  // this lane's B row (weight row) inside the tile
    u32x4p mhd = u32x4p{0, 0, 0, 0};   // min-term header of this lane's slot
    u32x4p hd = u32x4p{0, 0, 0, 0};    // the current superblock's header of this lane's column

    // Step g = g6 + k (g6 a multiple of 6): issue step g+2 into stage
    // (k+2) % 3, compute step g from stage k % 3, wait for step g+1's copies,
    // barrier.  The min-term window closes after every fourth superblock and
    // after the last one.
    auto step = [&](auto kc, int g6) {
        constexpr int k = decltype(kc)::value;
        constexpr int h = k & 1;
        constexpr int stage = k % kPf3Stages;
        const int g = g6 + k;
        const int s = g >> 1;
        const bool window_end = h == 1 && ((s & (kPfWin - 1)) == kPfWin - 1 || s == nsb - 1);
        // min-term bookkeeping: superblocks sb_start .. s of the window; slot =
        // lane / 16 is the superblock whose header this lane keeps
        const int sb_start = s - (s & (kPfWin - 1));
        const bool mlive = sb_start + quad <= s;
        issue(g + 2, std::integral_constant<int, (k + 2) % kPf3Stages>{}, std::integral_constant<int, h>{});
        const Prefill3Stage &S = stage_ref(std::integral_constant<int, stage>{});
        // header of this lane's column (staged with the superblock's first
        // half); scales of this step's four sub-blocks (fields 4h .. 4h+3)
        if constexpr (h == 0) lds_read1_b128(lds_addr(S.hdr + 4 * brow), hd);
        const uint32_t bits = h ? ((hd.y >> 24) | (hd.z << 8)) : hd.y;  // the four 6-bit scale fields
#pragma unroll
        for (int kp = 0; kp < 4; kp += 2) {
            // A rows 16 i + l16 (i = 0..7 at +4096 bytes), chunk (4 kk + quad) ^ l16;
            // B row brow, 8 bytes at byte 32 * pair + 8 * quad of the row's 64:
            // unit 2 pair + quad / 2, swizzled by (row >> 2) & 3 = (l16 >> 2) & 3
            uint32_t aa[2], na[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int kk = kp + t;
                aa[t] = lds_addr(S.a + (l16 * kPf3ChunkUnits + ((4 * kk + quad) ^ l16)) * 8);
                const int u = (2 * (kk >> 1) + (quad >> 1)) ^ ((l16 >> 2) & 3);
                na[t] = lds_addr(S.nib + brow * 64 + 16 * u + 8 * (quad & 1));
            }
            u32x4p ar[16];
            uint2 nb[2];
            lds_read_slice2_t(aa[0], na[0], aa[1], na[1], ar, nb);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int kk = kp + t;
                const _Float16 v = (_Float16)(uint16_t)((bits >> (6 * kk)) & 63u);
                const _Float16 o = v * (_Float16)(-1024.0f);  // exact: |.| <= 64512
                const half8 bf = b_operand(nb[t], kk & 1, half2v{v, v}, half2v{o, o});
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    cs[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ar[8 * t + i]), bf, cs[i],
                                                                   0, 0, 0);
            }
        }
        if constexpr (h == 1) {
            // superblock done: acc += d * cs, d of this lane's column; the lanes
            // of this superblock's slot keep its header for the min term
            mhd = quad == (s & (kPfWin - 1)) ? hd : mhd;
            const float d = half_lo(hd.x);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] = fmaf_exact(d, cs[i][e], acc[i][e]);
                cs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (window_end) {
            // min term of the window; slot = lane / 16 is its superblock.  The
            // window's block sums came with its steps' copies, all waited for.
            // Slots past the window's last superblock hold finite leftovers
            // (the buffers start zeroed) and meet zero weights below.
            // Token rows 16 i + l16 (+256 bytes per i); the lane's 8 blocks are
            // those of steps 2 quad and 2 quad + 1 of the window (+2048 bytes).
            const int sl0 = (((g / kPfWinSteps) & 1) * kPfWinSteps + 2 * quad) * kSumSlice + 8 * l16;
            u32x4p rs[16];
            lds_read16_b128(lds_addr(wsum + sl0), rs);
            const float dmin = mlive ? half_hi(mhd.x) : 0.0f;
            float dmax = dmin;
            dmax = fmaxf(dmax, __shfl_xor(dmax, 16, kWave));
            dmax = fmaxf(dmax, __shfl_xor(dmax, 32, kWave));
            const int E = row_exponent(dmax) - 6;
            const float fac = -ldexpf(1.0f, kPfSumShift - E);
            half8 mh, ml;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float mv = ldexpf(dmin * (float)field6(mhd.y, mhd.z, mhd.w, 8 + e), E);
                _Float16 hi, lo;
                split_half(mv, hi, lo);
                mh[e] = hi;
                ml[e] = lo;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const half8 shi = __builtin_bit_cast(half8, u32x4p{rs[i].x, rs[i].y, rs[8 + i].x, rs[8 + i].y});
                const half8 slo = __builtin_bit_cast(half8, u32x4p{rs[i].z, rs[i].w, rs[8 + i].z, rs[8 + i].w});
                f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(shi, mh, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(shi, ml, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(slo, mh, c, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] = fmaf_exact(fac, c[e], acc[i][e]);
            }
        }
        // step g+1's copies have landed (this wave's; the barrier makes it every
        // wave's) while step g+2's stay in flight; after the barrier every wave
        // is also done with stage g % 3, which step g+3 refills
        wait_vmem_lgkm<pf3_copies(h)>();
        barrier_no_fence();
    };

    for (int i = tid; i < 2 * kPfWinSteps * kSumSlice / 8; i += kPf3Threads)
        reinterpret_cast<u32x4p *>(wsum)[i] = u32x4p{0, 0, 0, 0};
    __syncthreads();  // the zeros are written before any copy can land on them
    issue(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
    wait_vmem_lgkm<pf3_copies(1)>();  // step 0's copies are in LDS
    barrier_no_fence();
    const int nbody = nsteps - nsteps % 6;
    int g6 = 0;
    for (; g6 < nbody; g6 += 6) {
        step(std::integral_constant<int, 0>{}, g6);
        step(std::integral_constant<int, 1>{}, g6);
        step(std::integral_constant<int, 2>{}, g6);
        step(std::integral_constant<int, 3>{}, g6);
        step(std::integral_constant<int, 4>{}, g6);
        step(std::integral_constant<int, 5>{}, g6);
    }
    // tail: nsteps is even, so 0, 2 or 4 steps remain
    if (g6 < nsteps) {
        step(std::integral_constant<int, 0>{}, g6);
        step(std::integral_constant<int, 1>{}, g6);
    }
    if (g6 + 2 < nsteps) {
        step(std::integral_constant<int, 2>{}, g6);
        step(std::integral_constant<int, 3>{}, g6);
    }
    wait_vmem_at_most<0>();  // no copy into LDS may still be in flight when the workgroup ends

    const int n = n0 + brow;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + 16 * i + 4 * quad + e;
            if (m < M && n < N) Y[(size_t)m * N + n] = ldexpf(acc[i][e], -E_x[m]);
        }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// x * 2^e as fp16 [M][K], e [M], then the block-sum records [M][K / 128][8]
// (fp16), every region 256-byte aligned
struct PrefillWs {
    size_t off_e, off_s, total;
};

static PrefillWs prefill_ws_layout(int M, int K) {
    PrefillWs w;
    w.off_e = align256((size_t)M * K * 2);
    w.off_s = w.off_e + align256((size_t)M * 4);
    w.total = w.off_s + align256((size_t)M * (K / 128) * 16);
    return w;
}

static int prefill_check(int fmt, const void *W, int N, int K, const uint16_t *x, int M, float *y) {
    if (fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!W || !x || !y) return QG_ERR_NULL;
    if (M < 1 || N < 1 || K < 256 || K > QG_MAX_K || K % 256 != 0) return QG_ERR_SHAPE;
    if ((M + kPfBM - 1) / kPfBM > 65535) return QG_ERR_SHAPE;
    if (((uintptr_t)W | (uintptr_t)x | (uintptr_t)y) & 15) return QG_ERR_ALIGN;
    return QG_OK;
}

}  // namespace qg

extern "C" int qgemm_prefill(int fmt, const void *W, int N, int K, const uint16_t *x_bf16, int M, float *y,
                             void *stream) {
    const int rc = qg::prefill_check(fmt, W, N, K, x_bf16, M, y);
    if (rc) return rc;
    qg::clear_stale_error();
    dim3 grid((N + qg::kPfBN - 1) / qg::kPfBN, (M + qg::kPfBM - 1) / qg::kPfBM);
    hipLaunchKernelGGL(qg::qgemm_prefill_q4k_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t *>(W), N, K, x_bf16, M, y);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

extern "C" size_t qgemm_prefill_workspace_bytes(int M, int K) {
    if (M < 1 || K < 256 || K > QG_MAX_K || K % 256 != 0) return 0;
    return qg::prefill_ws_layout(M, K).total;
}

extern "C" int qgemm_prefill_ws(int fmt, const void *W, int N, int K, const uint16_t *x_bf16, int M, float *y,
                                void *ws, size_t ws_bytes, void *stream) {
    const int rc = qg::prefill_check(fmt, W, N, K, x_bf16, M, y);
    if (rc) return rc;
    if (!ws) return QG_ERR_NULL;
    if (((uintptr_t)ws) & 15) return QG_ERR_ALIGN;
    const qg::PrefillWs lay = qg::prefill_ws_layout(M, K);
    if (ws_bytes < lay.total) return QG_ERR_WORKSPACE;
    uint8_t *b = reinterpret_cast<uint8_t *>(ws);
    _Float16 *x16 = reinterpret_cast<_Float16 *>(b);
    int32_t *ex = reinterpret_cast<int32_t *>(b + lay.off_e);
    _Float16 *ss = reinterpret_cast<_Float16 *>(b + lay.off_s);
    qg::clear_stale_error();
    hipLaunchKernelGGL(qg::prefill_prepass_kernel, dim3(M), dim3(qg::kPfPreThreads), 0, (hipStream_t)stream, x_bf16,
                       K, x16, ex, ss);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;
    dim3 grid((N + qg::kPfBN - 1) / qg::kPfBN, (M + qg::kPfBM - 1) / qg::kPfBM);
    hipLaunchKernelGGL(qg::qgemm_prefill_q4k_ws_kernel, grid, dim3(qg::kPf3Threads), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t *>(W), N, K, M, x16, ex, ss, y);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}
