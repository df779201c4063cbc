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
// sc*q <= 63*15 = 945 is an integer, exact in fp16, and bf16 activations are
// exact in fp16 (apart from |x| < 2^-17, off by < 2^-25), so the main product
// runs on the fp16 MFMA with exact inputs and fp32 accumulation, and d_s is
// applied per superblock in fp32.  The min term is a second, 32x smaller
// product over the sub-block sums: dmin*m*2^12 (17 significant bits, scaled
// into fp16's normal range) and S are each split into two fp16 halves and
// three hi/lo MFMA products give it to ~2^-21 relative.  Plain bf16 or fp16
// dequantization of w would not meet 1e-5 * sum |w x|.
//
// Tiling (gfx950, wave64): 128 tokens x 128 weight rows per workgroup, four
// waves of 64 x 64, v_mfma_f32_16x16x32_f16 (A: lane l holds row l%16, k
// 8*(l/16)..+8; B: column l%16, same k; C: rows 4*(l/16)+i, column l%16).
// K advances 64 at a time: the workgroup dequantizes the 128 x 64 weight
// slice into LDS and converts the 128 x 64 activation slice, both with padded
// row strides (36 dwords) so the 16-byte operand reads are bank-conflict free.
#include "common.h"

namespace qg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfBM = 128;  // tokens per workgroup
constexpr int kPfBN = 128;  // weight rows per workgroup
constexpr int kPfKS = 64;   // K per step (two sub-blocks)
constexpr int kPfLd = kPfKS + 8;  // padded LDS row, halves
constexpr int kPfWin = 4;         // superblocks per min-term window (32 sub-blocks)
constexpr int kPfSLd = 32 + 8;    // padded LDS row of the min-term operands, halves
constexpr float kPfMinScale = 4096.0f;

struct PrefillLds {
    _Float16 a[kPfBM * kPfLd];        // activations, fp16
    _Float16 b[kPfBN * kPfLd];        // sc*q, fp16
    _Float16 s_hi[kPfBM * kPfSLd];    // sub-block sums of x, high half
    _Float16 s_lo[kPfBM * kPfSLd];    // and the remainder
    _Float16 mn_hi[kPfBN * kPfSLd];   // dmin*m*2^12, high half
    _Float16 mn_lo[kPfBN * kPfSLd];
    float d[kPfBN];                   // d of the current superblock per row
};

__device__ __forceinline__ uint32_t field6(uint32_t s0, uint32_t s1, uint32_t s2, int f) {
    const int bit = 6 * f, word = bit >> 5, off = bit & 31;
    const uint32_t lo = word == 0 ? s0 : (word == 1 ? s1 : s2);
    const uint32_t hi = word == 0 ? s1 : (word == 1 ? s2 : 0u);
    return (off == 0 ? lo : ((lo >> off) | (hi << (32 - off)))) & 63u;
}

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ void split_half(float v, _Float16 &hi, _Float16 &lo) {
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);
}

__global__ __launch_bounds__(256) void qgemm_prefill_q4k_kernel(const uint8_t *__restrict__ W, int N, int K,
                                                                const uint16_t *__restrict__ X, int M,
                                                                float *__restrict__ Y) {
    __shared__ PrefillLds L;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // wave's 64 x 64 quadrant
    const int n0 = blockIdx.x * kPfBN, m0 = blockIdx.y * kPfBM;
    const int nsb = K / 256;
    const size_t row_bytes = (size_t)nsb * 144;

    f32x4 acc[4][4], cs[4][4], cmin[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = cs[i][j] = cmin[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging roles: thread -> (row, half) for weights, (token, sub-block) for activations
    const int srow = tid >> 1, shalf = tid & 1;
    const bool wrow_ok = n0 + srow < N;
    const bool xrow_ok = m0 + srow < M;
    const uint8_t *wrow = W + (size_t)(n0 + srow) * row_bytes;
    const uint16_t *xrow = X + (size_t)(m0 + srow) * K;

    for (int s = 0; s < nsb; ++s) {
        const int q = s % kPfWin;  // superblock slot in the min-term window
        for (int p = 0; p < 4; ++p) {
            // ---- stage weights: 16 bytes of nibbles = 16 weights of sub-block 2p and 16 of 2p+1
            {
                uint4 hdr = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
                if (wrow_ok) {
                    hdr = *reinterpret_cast<const uint4 *>(wrow + (size_t)s * 144);
                    qv = *reinterpret_cast<const uint4 *>(wrow + (size_t)s * 144 + 16 + 32 * p + 16 * shalf);
                }
                const int sc_a = (int)field6(hdr.y, hdr.z, hdr.w, 2 * p);
                const int sc_b = (int)field6(hdr.y, hdr.z, hdr.w, 2 * p + 1);
                const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
                _Float16 *brow = L.b + srow * kPfLd;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
#pragma unroll
                    for (int by = 0; by < 4; ++by) {
                        const int i = 16 * shalf + 4 * w + by;  // element within the sub-block
                        const int byte = (int)((words[w] >> (8 * by)) & 0xffu);
                        brow[i] = (_Float16)(float)(sc_a * (byte & 15));
                        brow[32 + i] = (_Float16)(float)(sc_b * (byte >> 4));
                    }
                }
                if (p == 0 && shalf == 0) {
                    const float d = wrow_ok ? (float)__builtin_bit_cast(_Float16, (uint16_t)(hdr.x & 0xffffu)) : 0.f;
                    const float dmin = wrow_ok ? (float)__builtin_bit_cast(_Float16, (uint16_t)(hdr.x >> 16)) : 0.f;
                    L.d[srow] = d;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float mv = dmin * (float)field6(hdr.y, hdr.z, hdr.w, 8 + j) * kPfMinScale;  // exact
                        split_half(mv, L.mn_hi[srow * kPfSLd + 8 * q + j], L.mn_lo[srow * kPfSLd + 8 * q + j]);
                    }
                }
            }
            // ---- stage activations: 32 bf16 of one sub-block -> fp16, and their sum
            {
                const int j = shalf;  // sub-block 2p + j of superblock s
                float vals[32];
                if (xrow_ok) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(xrow + (size_t)s * 256 + 64 * p + 32 * j);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint4 v = src[c];
                        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            vals[8 * c + 2 * h] = bf16_to_float(wv[h] & 0xffffu);
                            vals[8 * c + 2 * h + 1] = bf16_to_float(wv[h] >> 16);
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 32; ++i) vals[i] = 0.f;
                }
                float ssum = 0.f;
                _Float16 *arow = L.a + srow * kPfLd + 32 * j;
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    arow[i] = (_Float16)vals[i];
                    ssum += vals[i];
                }
                split_half(ssum, L.s_hi[srow * kPfSLd + 8 * q + 2 * p + j], L.s_lo[srow * kPfSLd + 8 * q + 2 * p + j]);
            }
            __syncthreads();

            // ---- 64 x 64 per wave: 4 x 4 tiles, two k-steps of 32
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
                    for (int j = 0; j < 4; ++j) cs[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr[j], cs[i][j], 0, 0, 0);
            }

            if (p == 3) {
                // superblock done: acc += d * cs (d per weight row = column of C)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float d = L.d[64 * wn + 16 * j + (lane & 15)];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf_exact(d, cs[i][j][r], acc[i][j][r]);
                        cs[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
                if (q == kPfWin - 1 || s == nsb - 1) {
                    // min term over the window's sub-blocks (slots beyond the last superblock are masked)
                    const int valid_q = q + 1;
                    const bool live = (lane >> 4) < valid_q;  // this lane's k' range belongs to superblock lane>>4
                    half8 sh[4], sl[4], mh[4], ml[4];
                    const half8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = (64 * wm + 16 * i + (lane & 15)) * kPfSLd + 8 * (lane >> 4);
                        sh[i] = live ? *reinterpret_cast<const half8 *>(L.s_hi + r) : zero;
                        sl[i] = live ? *reinterpret_cast<const half8 *>(L.s_lo + r) : zero;
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = (64 * wn + 16 * j + (lane & 15)) * kPfSLd + 8 * (lane >> 4);
                        mh[j] = live ? *reinterpret_cast<const half8 *>(L.mn_hi + r) : zero;
                        ml[j] = live ? *reinterpret_cast<const half8 *>(L.mn_lo + r) : zero;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            cmin[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sh[i], mh[j], cmin[i][j], 0, 0, 0);
                            cmin[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sh[i], ml[j], cmin[i][j], 0, 0, 0);
                            cmin[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sl[i], mh[j], cmin[i][j], 0, 0, 0);
                        }
                }
            }
            __syncthreads();  // LDS is restaged next step
        }
    }

    // Y = acc - cmin / 2^12
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + 64 * wn + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + r;
                if (m < M && n < N) Y[(size_t)m * N + n] = fmaf_exact(-1.0f / kPfMinScale, cmin[i][j][r], acc[i][j][r]);
            }
        }
}

}  // namespace qg

extern "C" int qgemm_prefill(int fmt, const void *W, int N, int K, const uint16_t *x_bf16, int M, float *y,
                             void *stream) {
    if (fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!W || !x_bf16 || !y) return QG_ERR_NULL;
    if (M < 1 || N < 1 || K < 256 || K > QG_MAX_K || K % 256 != 0) return QG_ERR_SHAPE;
    if (((uintptr_t)W | (uintptr_t)x_bf16 | (uintptr_t)y) & 15) return QG_ERR_ALIGN;
    if ((long long)((M + qg::kPfBM - 1) / qg::kPfBM) > 65535) return QG_ERR_SHAPE;
    dim3 grid((N + qg::kPfBN - 1) / qg::kPfBN, (M + qg::kPfBM - 1) / qg::kPfBM);
    hipLaunchKernelGGL(qg::qgemm_prefill_q4k_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t *>(W), N, K, x_bf16, M, y);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}
