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
// Tiling (gfx950, wave64): 128 tokens x 128 weight rows per workgroup, four
// waves of 64 x 64, v_mfma_f32_16x16x32_f16 (A: lane l holds row l%16, k
// 8*(l/16)..+8; B: column l%16, same k; C: rows 4*(l/16)+i, column l%16).
// K advances 128 (half a superblock) per step.  Each step the workgroup
// dequantizes its 128 x 128 weight slice once into LDS as fp16 sc*q (nibbles
// are widened with byte permutes into fp16 1024+q, and one packed fp16 fma per
// pair, (1024+q)*sc - 1024*sc, gives sc*q exactly) and stages the activations
// as fp16, both with padded row strides so the 16-byte operand reads are
// bank-conflict free.  The global reads of the next step are issued before
// the current step's MFMAs, so they overlap.
//
// Two forms.  qgemm_prefill converts bf16 -> fp16 and forms the sub-block sums
// inside the GEMM, with e = 0 (so it needs |x| <= 65504 and loses low bits of
// |x| < 2^-17).  qgemm_prefill_ws first runs a pass, one workgroup per token,
// that finds e, writes x*2^e as fp16 and the hi/lo sums to a caller workspace;
// the GEMM then reads them instead of converting once per weight tile.
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

// One workgroup per token m: e[m], X16[m] = x*2^e (fp16), and the sums of each
// 32-block split as S*2^(e-6) = hi + lo (fp16).  Lane group of 8 per block,
// four values per lane.
__global__ __launch_bounds__(kPfPreThreads) void prefill_prepass_kernel(const uint16_t *__restrict__ X, int K,
                                                                        _Float16 *__restrict__ X16,
                                                                        _Float16 *__restrict__ s_hi,
                                                                        _Float16 *__restrict__ s_lo,
                                                                        int32_t *__restrict__ e_out) {
    __shared__ float red[kPfPreThreads / kWave];
    const int m = blockIdx.x, tid = threadIdx.x;
    const uint16_t *xr = X + (size_t)m * K;
    float amax = 0.f;
    for (int k = 4 * tid; k < K; k += 4 * kPfPreThreads) {
        const uint2 w = *reinterpret_cast<const uint2 *>(xr + k);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf_lo(w.x)), fabsf(bf_hi(w.x))), fmaxf(fabsf(bf_lo(w.y)), fabsf(bf_hi(w.y)))));
    }
    for (int o = 1; o < kWave; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = red[0];
    for (int i = 1; i < kPfPreThreads / kWave; ++i) amax = fmaxf(amax, red[i]);
    const int e = row_exponent(amax);
    if (tid == 0) e_out[m] = e;

    for (int k = 4 * tid; k < K; k += 4 * kPfPreThreads) {
        const uint2 w = *reinterpret_cast<const uint2 *>(xr + k);
        const float v0 = bf_lo(w.x), v1 = bf_hi(w.x), v2 = bf_lo(w.y), v3 = bf_hi(w.y);
        const half2v h0 = {(_Float16)ldexpf(v0, e), (_Float16)ldexpf(v1, e)};
        const half2v h1 = {(_Float16)ldexpf(v2, e), (_Float16)ldexpf(v3, e)};
        *reinterpret_cast<uint2 *>(X16 + (size_t)m * K + k) =
            make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
        // block sum: lanes 8b .. 8b+7 hold block b's four-value partial sums in order
        float s = quad_sum(v0, v1, v2, v3);
        s += __shfl_xor(s, 1, kWave);
        s += __shfl_xor(s, 2, kWave);
        s += __shfl_xor(s, 4, kWave);
        if ((tid & 7) == 0) {
            const size_t blk = (size_t)m * (K / 32) + (size_t)(k / 32);
            split_half(ldexpf(s, e - kPfSumShift), s_hi[blk], s_lo[blk]);
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

template <bool XPRE>
__global__ __launch_bounds__(256) void qgemm_prefill_q4k_kernel(const uint8_t *__restrict__ W, int N, int K,
                                                                const uint16_t *__restrict__ X, int M,
                                                                const _Float16 *__restrict__ X16,
                                                                const _Float16 *__restrict__ S_hi,
                                                                const _Float16 *__restrict__ S_lo,
                                                                const int32_t *__restrict__ E_x,
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
            const u32x4p *src = XPRE ? reinterpret_cast<const u32x4p *>(X16 + (size_t)(m0 + r) * K + k0)
                                     : reinterpret_cast<const u32x4p *>(X + (size_t)(m0 + r) * K + k0);
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
            if (XPRE) {
#pragma unroll
                for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4p *>(arow + 8 * c) = pr.x[c];
            } else {
                // bf16 -> fp16, and the two sub-block sums (the pre-pass's order)
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
                    } else if (XPRE) {
                        const size_t o = (size_t)min(m0 + mr, M - 1) * (K / 32) + (size_t)(sb0 + slot) * 8;
                        sh[i] = *reinterpret_cast<const half8 *>(S_hi + o);
                        sl[i] = *reinterpret_cast<const half8 *>(S_lo + o);
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
            const int ex = XPRE ? E_x[m] : 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + 64 * wn + 16 * j + (lane & 15);
                if (n < N) Y[(size_t)m * N + n] = XPRE ? ldexpf(acc[i][j][e], -ex) : acc[i][j][e];
            }
        }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PrefillWs {
    size_t off_shi, off_slo, off_e, total;
};

static PrefillWs prefill_ws_layout(int M, int K) {
    PrefillWs w;
    const size_t x16 = align256((size_t)M * K * 2);
    const size_t s = align256((size_t)M * (K / 32) * 2);
    w.off_shi = x16;
    w.off_slo = x16 + s;
    w.off_e = x16 + 2 * s;
    w.total = w.off_e + align256((size_t)M * 4);
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
    dim3 grid((N + qg::kPfBN - 1) / qg::kPfBN, (M + qg::kPfBM - 1) / qg::kPfBM);
    hipLaunchKernelGGL(qg::qgemm_prefill_q4k_kernel<false>, grid, dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t *>(W), N, K, x_bf16, M, nullptr, nullptr, nullptr, nullptr, y);
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
    _Float16 *s_hi = reinterpret_cast<_Float16 *>(b + lay.off_shi);
    _Float16 *s_lo = reinterpret_cast<_Float16 *>(b + lay.off_slo);
    int32_t *ex = reinterpret_cast<int32_t *>(b + lay.off_e);
    hipLaunchKernelGGL(qg::prefill_prepass_kernel, dim3(M), dim3(qg::kPfPreThreads), 0, (hipStream_t)stream, x_bf16,
                       K, x16, s_hi, s_lo, ex);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;
    dim3 grid((N + qg::kPfBN - 1) / qg::kPfBN, (M + qg::kPfBM - 1) / qg::kPfBM);
    hipLaunchKernelGGL(qg::qgemm_prefill_q4k_kernel<true>, grid, dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t *>(W), N, K, x_bf16, M, x16, s_hi, s_lo, ex, y);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}
