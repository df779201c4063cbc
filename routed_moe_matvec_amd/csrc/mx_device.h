// Mat-vec engine for the block-scaled low-precision expert formats: FP8 E4M3
// with one UE8M0 scale per 128 x 128 block and FP4 E2M1 with one UE8M0 scale
// per 1 x 32 block (ROCm/ATOM "DeepSeek-V4 Usage Guide", section "FP8 on
// MI308 / gfx942": the routed-expert quantization-config table, and the
// V4-Pro MoE backend note on FP4 e2m1 microscaling), against the Q8 activation
// every other projection consumes.
//
//   y[m, n] = sum_b  sum_{k in block b}  w[n, k] * (dx[m, b] * qx[m, k])
//
// Storage of one N x K matrix: the codes row-major (FP4: two per byte,
// element 2i in the low nibble), then from the next multiple of 256 bytes the
// scale bytes, [ceil(N/128)][K/128] for FP8 and [N][K/32] for FP4.
//
// A lane takes 16-byte chunks of a row (16 FP8 or 32 FP4 weights; one FP4
// chunk is one 32-block and one scale) with 64 consecutive chunks per wave
// instruction; a wave keeps kMxLoads chunks of R = kMxLoads / CPL rows in
// flight (CPL chunks per lane and row).  The tokens' Q8 activation is staged
// once per workgroup in LDS as fp16 (exact for int8), 64-byte block records
// padded to 80 bytes so that eight lanes reading consecutive blocks meet eight
// different bank groups.  Per chunk the hardware converts the codes to fp16
// pairs (v_cvt_scalef32_pk_f16_fp8 / _fp4, scale 1) and v_dot2_f32_f16
// accumulates them against the activation in fp32 (for FP4 every partial sum
// is a multiple of 1/2 below 2^15, so it is exact); then
// acc = fma(partial, ldexp(dx[m, b], s - 127), acc) in chunk order and the
// row's lanes meet in an xor butterfly.
#pragma once

#include "common.h"

namespace qg {

typedef _Float16 mx_half2 __attribute__((ext_vector_type(2)));
typedef unsigned int mx_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMxWaves = 4;
constexpr int kMxLoads = 16;             // 16-byte weight chunks a lane keeps in flight
constexpr int kMxActBudget = 64 * 1024;  // LDS for staged tokens
constexpr int kMxBlockRec = 80;          // LDS bytes of one 32-block of fp16 activation (64 + pad)

__host__ __device__ constexpr int mx_rows_per_wave(int cpl) { return kMxLoads / cpl > 0 ? kMxLoads / cpl : 1; }
__host__ __device__ inline size_t mx_align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int FMT>
struct MxFmt;
template <>
struct MxFmt<QG_FMT_FP8_E4M3_B128> {
    static constexpr int weights_per_chunk = 16;
    __host__ __device__ static size_t row_bytes(int K) { return (size_t)K; }
    __host__ __device__ static size_t scale_offset(int N, int K) { return mx_align256((size_t)N * K); }
    __device__ static size_t scale_index(int row, int chunk, int K) {
        return (size_t)(row >> 7) * (K >> 7) + (chunk >> 3);
    }
    __device__ static int act_offset(int chunk) { return kMxBlockRec * (chunk >> 1) + 32 * (chunk & 1); }
    __device__ static int act_block(int chunk) { return chunk >> 1; }
};
template <>
struct MxFmt<QG_FMT_FP4_E2M1_MX> {
    static constexpr int weights_per_chunk = 32;
    __host__ __device__ static size_t row_bytes(int K) { return (size_t)K / 2; }
    __host__ __device__ static size_t scale_offset(int N, int K) { return mx_align256((size_t)N * K / 2); }
    __device__ static size_t scale_index(int row, int chunk, int K) { return (size_t)row * (K >> 5) + chunk; }
    __device__ static int act_offset(int chunk) { return kMxBlockRec * chunk; }
    __device__ static int act_block(int chunk) { return chunk; }
};

// LDS bytes of one staged token: the fp16 block records, then the fp32 scales.
__host__ __device__ inline int mx_token_rec(int K) { return (K / 32) * (kMxBlockRec + 4); }

// Chunks per lane and row, as a power of two (K % 256 == 0).
template <int FMT>
inline int mx_chunks_per_lane(int K) {
    const int cpr = K / MxFmt<FMT>::weights_per_chunk;
    int cpl = 1;
    while (cpl * kWave < cpr) cpl <<= 1;
    return cpl;
}

// fp32 dot product of one 16-byte chunk with its fp16 activation in LDS.
template <int FMT>
__device__ __forceinline__ float mx_chunk_dot(const mx_u32x4 &w, const uint8_t *act) {
    float p = 0.0f;
    if constexpr (FMT == QG_FMT_FP4_E2M1_MX) {
        const mx_u32x4 a0 = reinterpret_cast<const mx_u32x4 *>(act)[0], a1 = reinterpret_cast<const mx_u32x4 *>(act)[1];
        const mx_u32x4 a2 = reinterpret_cast<const mx_u32x4 *>(act)[2], a3 = reinterpret_cast<const mx_u32x4 *>(act)[3];
        const uint32_t A[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                                a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
        const uint32_t Wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t word = Wd[k >> 2];
            mx_half2 h;
            switch (k & 3) {  // the byte selector is an immediate
                case 0: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0); break;
                case 1: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1); break;
                case 2: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2); break;
                default: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3); break;
            }
            const uint32_t ak = A[k];
            p = __builtin_amdgcn_fdot2(h, __builtin_bit_cast(mx_half2, ak), p, false);
        }
    } else {
        const mx_u32x4 a0 = reinterpret_cast<const mx_u32x4 *>(act)[0], a1 = reinterpret_cast<const mx_u32x4 *>(act)[1];
        const uint32_t A[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const uint32_t Wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t word = Wd[k >> 1];
            const mx_half2 h = (k & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true)
                                       : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
            const uint32_t ak = A[k];
            p = __builtin_amdgcn_fdot2(h, __builtin_bit_cast(mx_half2, ak), p, false);
        }
    }
    return p;
}

// One workgroup (kMxWaves waves) multiplies rows row_base .. row_base +
// kMxWaves * R - 1 of W (clipped to N) with M tokens; token m's activation is
// row token_row(m) of qx / dx; out(m, row, value) stores a result.  Tokens are
// staged mt at a time.  Every wave of the workgroup must call this.
template <int FMT, int CPL, class TokenRow, class Out>
__device__ __forceinline__ void mx_workgroup(const uint8_t *__restrict__ W, int N, int K, int row_base, int M, int mt,
                                             const int8_t *__restrict__ qx, const float *__restrict__ dx,
                                             TokenRow token_row, Out out, uint8_t *smem) {
    using F = MxFmt<FMT>;
    constexpr int R = mx_rows_per_wave(CPL);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int cpr = K / F::weights_per_chunk;
    const size_t rb = F::row_bytes(K);
    const uint8_t *scales = W + F::scale_offset(N, K);
    const int row0 = row_base + wave * R;
    const int nb = K / 32;
    const int rec = mx_token_rec(K);

    // the wave's weight chunks and their scales (rows past N and chunks past
    // the row's end re-read the last ones and are not used)
    mx_u32x4 w[R][CPL];
    int sc[R][CPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = min(lane + kWave * j, cpr - 1);
            w[r][j] = __builtin_nontemporal_load(reinterpret_cast<const mx_u32x4 *>(W + row * rb + 16 * (size_t)c));
            sc[r][j] = (int)scales[F::scale_index(row, c, K)] - 127;
        }
    }

    // tokens [m0, m0 + mtc) into LDS: int8 quants as fp16 block records, then the scales
    auto stage = [&](int m0, int mtc) {
        const int pieces = K / 16;
        for (int t = threadIdx.x; t < mtc * pieces; t += blockDim.x) {
            const int mm = t / pieces, pc = t - mm * pieces;
            const mx_u32x4 q = *reinterpret_cast<const mx_u32x4 *>(qx + (size_t)token_row(m0 + mm) * K + 16 * pc);
            const uint32_t Q[4] = {q.x, q.y, q.z, q.w};
            uint32_t H[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t word = Q[k >> 1] >> (16 * (k & 1));
                mx_half2 h;
                h.x = (_Float16)(float)(int8_t)(word & 0xffu);
                h.y = (_Float16)(float)(int8_t)((word >> 8) & 0xffu);
                H[k] = __builtin_bit_cast(uint32_t, h);
            }
            uint8_t *dst = smem + (size_t)mm * rec + kMxBlockRec * (pc >> 1) + 32 * (pc & 1);
            *reinterpret_cast<mx_u32x4 *>(dst) = mx_u32x4{H[0], H[1], H[2], H[3]};
            *reinterpret_cast<mx_u32x4 *>(dst + 16) = mx_u32x4{H[4], H[5], H[6], H[7]};
        }
        for (int t = threadIdx.x; t < mtc * nb; t += blockDim.x) {
            const int mm = t / nb, b = t - mm * nb;
            reinterpret_cast<float *>(smem + (size_t)mm * rec + kMxBlockRec * nb)[b] =
                dx[(size_t)token_row(m0 + mm) * nb + b];
        }
    };

    for (int m0 = 0; m0 < M; m0 += mt) {
        const int mtc = min(mt, M - m0);
        if (m0 > 0) __syncthreads();  // every wave is done with the previous tokens
        stage(m0, mtc);
        __syncthreads();
        for (int mm = 0; mm < mtc; ++mm) {
            const uint8_t *act = smem + (size_t)mm * rec;
            const float *dxs = reinterpret_cast<const float *>(act + kMxBlockRec * nb);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int c = lane + kWave * j;
                    if (c < cpr) {
                        const float p = mx_chunk_dot<FMT>(w[r][j], act + F::act_offset(c));
                        const float s = __builtin_ldexpf(dxs[F::act_block(c)], sc[r][j]);
                        acc = fmaf_exact(p, s, acc);
                    }
                }
                for (int off = 1; off < kWave; off <<= 1) acc += shfl_xor(acc, off);
                if (lane == 0 && row0 + r < N) out(m0 + mm, row0 + r, acc);
            }
        }
    }
}

// Tokens staged at once for K inputs (at least one).
inline int mx_tokens_per_chunk(int K, int M) {
    int mt = kMxActBudget / mx_token_rec(K);
    if (mt < 1) mt = 1;
    return mt < M ? mt : M;
}

}  // namespace qg
