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
// scale bytes, [ceil(N/128)][K/128] for FP8 and [N][K/32] for FP4, then
// padding to a multiple of 16 bytes (so the aligned 4-byte word holding any
// scale byte lies inside the buffer).
//
// A lane takes 16-byte chunks of a row (16 FP8 or 32 FP4 weights; one FP4
// chunk is one 32-block and one scale) with 64 consecutive chunks per wave
// instruction; a wave keeps L chunks of R = L / CPL rows in
// flight (CPL chunks per lane and row).  The tokens' Q8 activation is staged
// once per workgroup in LDS as fp16 (exact for int8), 64-byte block records
// padded to 80 bytes so that eight lanes reading consecutive blocks meet eight
// different bank groups.  Per chunk the hardware converts the codes to fp16
// pairs (v_cvt_scalef32_pk_f16_fp8 / _fp4, scale 1) and v_dot2_f32_f16
// accumulates them against the activation in fp32 (for FP4 every partial sum
// is a multiple of 1/2 below 2^15, so it is exact); then
// acc = fma(partial, ldexp(dx[m, b], s - 127), acc) in chunk order and the
// row's lanes meet in a fixed DPP reduction.
#pragma once

#include "common.h"
#include "quantize_device.h"

namespace qg {

typedef _Float16 mx_half2 __attribute__((ext_vector_type(2)));
typedef unsigned int mx_u32x4 __attribute__((ext_vector_type(4)));
typedef float mx_f32x4 __attribute__((ext_vector_type(4)));

// One token's activation given as the SwiGLU inputs instead of a Q8 vector:
// the staging forms h = silu(g) * v and its Q8 form itself (the activation
// quantizer, so the values equal a separate quantization bit for bit); when
// ph is set the workgroup also stores h, its quants, scales and block sums.
struct MxGlu {
    const float *g, *v;  // the token's rows (K values each)
    float *ph;
    int8_t *pqx;
    float *pdx;
    int32_t *psx;
};

constexpr int kMxWaves = 4;  // waves per workgroup of the dense calls (mx_workgroup's NW)
// 16-byte weight chunks a lane keeps in flight (L).  Dense mat-vecs: 4 for
// FP8, 8 for FP4 (its decode costs twice the instructions per byte); fewer
// rows per wave and more waves measured faster for both than 16.  Routed
// experts: 16, since each workgroup first waits for its expert's pointer and
// pair list and the staged tokens, a cost more rows amortize.
__host__ __device__ constexpr int mx_loads(int fmt) { return fmt == QG_FMT_FP4_E2M1_MX ? 8 : 4; }
constexpr int kMxLoadsRouted = 16;
// Waves per workgroup of the routed kernels: 8 for FP8 (each expert's rows in
// half as many workgroups, which share one staging of the tokens; measured
// faster at one token), 4 for FP4 (measured faster, as for the dense calls).
__host__ __device__ constexpr int mx_routed_waves(int fmt) { return fmt == QG_FMT_FP8_E4M3_B128 ? 8 : kMxWaves; }
constexpr int kMxActBudget = 64 * 1024;  // LDS for staged tokens
constexpr int kMxLdsMax = kMxActBudget + 4096;  // with a workgroup's weight scales
constexpr int kMxBlockRec = 80;          // LDS bytes of one 32-block of fp16 activation (64 + pad)
constexpr int kMxStageRegs = 1;          // activation pieces per thread requested before the weights

__host__ __device__ constexpr int mx_rows_per_wave(int loads, int cpl) { return loads / cpl > 0 ? loads / cpl : 1; }
__host__ __device__ inline size_t mx_align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline size_t mx_align16(size_t x) { return (x + 15) & ~(size_t)15; }

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

// LDS bytes of a workgroup's weight scales, after the staged tokens: FP4 the
// [rows][K/32] scales of its waves * R rows, FP8 the one [K/128] row of
// its 128-row block (a workgroup's rows never straddle one: their count
// divides 128).
template <int FMT>
__host__ __device__ inline int mx_scale_lds(int K, int cpl, int loads, int waves = kMxWaves) {
    const int rows = waves * mx_rows_per_wave(loads, cpl);
    const int bytes = FMT == QG_FMT_FP4_E2M1_MX ? rows * (K / 32) : K / 128;
    return (bytes + 15) / 16 * 16;
}

// Chunks per lane and row, as a power of two (K % 256 == 0).
template <int FMT>
inline int mx_chunks_per_lane(int K) {
    const int cpr = K / MxFmt<FMT>::weights_per_chunk;
    int cpl = 1;
    while (cpl * kWave < cpr) cpl <<= 1;
    return cpl;
}

// Sum over the wave in a fixed order: DPP adds within each row of 16 lanes
// (quad xor 1, quad xor 2, half-row mirror, row mirror: every lane then holds
// its row's sum), then the four rows in lane order.
template <int CTRL>
__device__ __forceinline__ float mx_dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float mx_wave_sum(float v) {
    v += mx_dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += mx_dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += mx_dpp<0x141>(v);  // row_half_mirror
    v += mx_dpp<0x140>(v);  // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
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

// One workgroup (NW waves) multiplies rows row_base .. row_base +
// NW * R - 1 of W (clipped to N), R = mx_rows_per_wave(L, CPL), with M tokens; token m's activation is
// row token_row(m) of qx / dx; out(m, row, value) stores a result.  Tokens are
// staged mt at a time.  Every wave of the workgroup must call this.
// GLU: one token (M = 1) whose activation is glu's SwiGLU inputs (MxGlu);
// qx, dx and token_row are then unused.
template <int FMT, int CPL, int L, int NW = kMxWaves, bool GLU = false, class TokenRow, class Out>
__device__ __forceinline__ void mx_workgroup(const uint8_t *__restrict__ W, int N, int K, int row_base, int M, int mt,
                                             const int8_t *__restrict__ qx, const float *__restrict__ dx,
                                             TokenRow token_row, Out out, uint8_t *smem, const MxGlu &glu = {}) {
    using F = MxFmt<FMT>;
    constexpr int R = mx_rows_per_wave(L, CPL);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int cpr = K / F::weights_per_chunk;
    const size_t rb = F::row_bytes(K);
    const uint8_t *scales = W + F::scale_offset(N, K);
    const int row0 = row_base + wave * R;
    const int nb = K / 32;
    const int rec = mx_token_rec(K);

    // tokens [m0, m0 + mtc) into LDS: int8 quants as fp16 block records, then the scales
    const int pieces = K / 16;
    auto put_piece = [&](int mm, int pc, const mx_u32x4 &q) __attribute__((always_inline)) {
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
    };
    auto piece_src = [&](int m0, int t) __attribute__((always_inline)) {
        const int mm = t / pieces, pc = t - mm * pieces;
        return reinterpret_cast<const mx_u32x4 *>(qx + (size_t)token_row(m0 + mm) * K + 16 * pc);
    };
    auto put_dx = [&](int m0, int t, float v) __attribute__((always_inline)) {
        const int mm = t / nb, b = t - mm * nb;
        reinterpret_cast<float *>(smem + (size_t)mm * rec + kMxBlockRec * nb)[b] = v;
    };
    auto dx_src = [&](int m0, int t) __attribute__((always_inline)) {
        const int mm = t / nb, b = t - mm * nb;
        return dx + (size_t)token_row(m0 + mm) * nb + b;
    };
    // staging after the first chunk of tokens: loads and stores together
    auto stage = [&](int m0, int mtc, int from) {
        for (int t = from + threadIdx.x; t < mtc * pieces; t += (NW * kWave)) {
            const int mm = t / pieces;
            put_piece(mm, t - mm * pieces, *piece_src(m0, t));
        }
        for (int t = from + threadIdx.x; t < mtc * nb; t += (NW * kWave)) put_dx(m0, t, *dx_src(m0, t));
    };

    // First chunk of tokens: its first kMxStageRegs pieces and scales per
    // thread are requested before the weights, so that storing them waits
    // for them alone and each row's weights are consumed as they arrive
    // (loads return in order).  Indexes past the end re-read a valid element.
    const int mt0 = min(mt, M);
    // the workgroup's weight scales, one load per thread at most, requested
    // first as well: FP4 the scales of its rows (contiguous; past the last
    // row the load stays inside the padded buffer and is not used), FP8 the
    // scale row of its 128-row block
    uint8_t *lsc = smem + (size_t)mt * rec;
    const size_t row_scale_bytes = FMT == QG_FMT_FP4_E2M1_MX ? (size_t)(K / 32) : 0;
    const size_t scale_total = FMT == QG_FMT_FP4_E2M1_MX ? (size_t)N * (K / 32) : (size_t)((N + 127) / 128) * (K / 128);
    const int scale_bytes = FMT == QG_FMT_FP4_E2M1_MX ? NW * R * (K / 32) : K / 128;
    const uint8_t *scale_src = FMT == QG_FMT_FP4_E2M1_MX ? scales + (size_t)row_base * row_scale_bytes
                                                          : scales + (size_t)(row_base >> 7) * (K / 128);
    mx_u32x4 sreg = {0u, 0u, 0u, 0u};
    uint32_t sbyte = 0;
    // every thread loads and stores (threads past the end repeat the last
    // piece: the same bytes to the same place), so that no load is moved
    // into a conditional store behind the weights
    const int lsc_off = FMT == QG_FMT_FP4_E2M1_MX ? min(16 * (int)threadIdx.x, scale_bytes - 16)
                                                   : min((int)threadIdx.x, scale_bytes - 1);
    if constexpr (FMT == QG_FMT_FP4_E2M1_MX) {
        // 16-byte pieces; rows past N read the last piece that starts inside the scales
        const size_t last = ((scale_total - 1) & ~(size_t)15) - (size_t)row_base * row_scale_bytes;
        sreg = *as_global<mx_u32x4>(scale_src + min((size_t)lsc_off, last));
    } else {
        sbyte = *as_global<uint8_t>(scale_src + lsc_off);
    }
    mx_u32x4 qreg[kMxStageRegs];
    float dreg[kMxStageRegs];
    // GLU: 16-byte chunks c of g and v (4 values; 8 lanes form a 32-block);
    // the first kMxGluRegs per thread are read before the weights.  A wave
    // past the end takes the last 64 chunks again (K / 4 is a multiple of 64):
    // identical values to the same places.
    constexpr int kMxGluRegs = 1;
    const int gchunks = K / 4;
    auto glu_chunk = [&](int t) __attribute__((always_inline)) {
        return t < gchunks ? t : gchunks - kWave + lane;
    };
    mx_f32x4 greg[GLU ? kMxGluRegs : 1], vreg[GLU ? kMxGluRegs : 1];
    if constexpr (GLU) {
#pragma unroll
        for (int i = 0; i < kMxGluRegs; ++i) {
            const int c = glu_chunk((int)threadIdx.x + i * (NW * kWave));
            greg[i] = as_global<mx_f32x4>(glu.g)[c];
            vreg[i] = as_global<mx_f32x4>(glu.v)[c];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMxStageRegs; ++i) {
            const int t = threadIdx.x + i * (NW * kWave);
            qreg[i] = *piece_src(0, min(t, mt0 * pieces - 1));
            dreg[i] = *dx_src(0, min(t, mt0 * nb - 1));
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // these loads are issued before the weights
    // chunk c's h = silu(g) * v, quantized with its 8-lane group: the fp16
    // quants and the scale into the token's record, h and the Q8 form to glu's
    // outputs when given
    auto glu_emit = [&](int c, mx_f32x4 g4, mx_f32x4 v4) __attribute__((always_inline)) {
        float h[4] = {silu(g4.x) * v4.x, silu(g4.y) * v4.y, silu(g4.z) * v4.z, silu(g4.w) * v4.w};
        int8_t q[4];
        float d;
        int32_t sum;
        quantize_block_8lanes(h, q, &d, &sum);  // every lane takes part (shuffles)
        const int blk = c >> 3, part = c & 7;
        mx_half2 h01, h23;
        h01.x = (_Float16)(float)q[0];
        h01.y = (_Float16)(float)q[1];
        h23.x = (_Float16)(float)q[2];
        h23.y = (_Float16)(float)q[3];
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2 *>(smem + kMxBlockRec * blk + 8 * part) =
            u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
        if (part == 0) put_dx(0, blk, d);
        if (glu.ph) {
            *reinterpret_cast<mx_f32x4 *>(glu.ph + 4 * c) = mx_f32x4{h[0], h[1], h[2], h[3]};
            *reinterpret_cast<uint32_t *>(glu.pqx + 4 * c) = (uint32_t)(uint8_t)q[0] | ((uint32_t)(uint8_t)q[1] << 8) |
                                                            ((uint32_t)(uint8_t)q[2] << 16) |
                                                            ((uint32_t)(uint8_t)q[3] << 24);
            if (part == 0) {
                glu.pdx[blk] = d;
                glu.psx[blk] = sum;
            }
        }
    };

    // the wave's weight chunks and their scales (rows past N and chunks past
    // the row's end re-read the last ones and are not used)
    mx_u32x4 w[R][CPL];

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = min(lane + kWave * j, cpr - 1);
            w[r][j] = __builtin_nontemporal_load(as_global<mx_u32x4>(W + row * rb + 16 * (size_t)c));
        }
    }

    // stored unconditionally (an index past the end stores the last element's
    // value again at its own place): a conditional store would let the
    // compiler move its load behind the weights
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FMT == QG_FMT_FP4_E2M1_MX)
        *reinterpret_cast<mx_u32x4 *>(lsc + lsc_off) = sreg;
    else
        lsc[lsc_off] = (uint8_t)sbyte;
    if constexpr (GLU) {
#pragma unroll
        for (int i = 0; i < kMxGluRegs; ++i)
            glu_emit(glu_chunk((int)threadIdx.x + i * (NW * kWave)), greg[i], vreg[i]);
        // chunks past the registers (rows longer than kMxGluRegs chunks per
        // thread), whole waves at a time
        for (int c0 = kMxGluRegs * (NW * kWave); c0 < gchunks; c0 += NW * kWave) {
            if (c0 + wave * kWave < gchunks) {
                const int c = c0 + (int)threadIdx.x;
                glu_emit(c, as_global<mx_f32x4>(glu.g)[c], as_global<mx_f32x4>(glu.v)[c]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMxStageRegs; ++i) {
            const int tq = min((int)threadIdx.x + i * (NW * kWave), mt0 * pieces - 1);
            put_piece(tq / pieces, tq - (tq / pieces) * pieces, qreg[i]);
            put_dx(0, min((int)threadIdx.x + i * (NW * kWave), mt0 * nb - 1), dreg[i]);
        }
        stage(0, mt0, kMxStageRegs * (NW * kWave));
    }

    // token mm of the chunk at m0 against every row of the wave
    auto token = [&](int m0, int mm) __attribute__((always_inline)) {
        const uint8_t *act = smem + (size_t)mm * rec;
        const float *dxs = reinterpret_cast<const float *>(act + kMxBlockRec * nb);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc = 0.0f;
            // row r's operands are used here, as they arrive: an empty asm that
            // rewrites them keeps work on them inside the token loop (hoisted,
            // it would wait for every load before the first row)
#pragma unroll
            for (int j = 0; j < CPL; ++j) asm volatile("" : "+v"(w[r][j]));
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + kWave * j;
                if (c < cpr) {
                    const float p = mx_chunk_dot<FMT>(w[r][j], act + F::act_offset(c));
                    const int e = (int)lsc[FMT == QG_FMT_FP4_E2M1_MX ? (wave * R + r) * (K / 32) + c : (c >> 3)] - 127;
                    const float s = __builtin_ldexpf(dxs[F::act_block(c)], e);
                    acc = fmaf_exact(p, s, acc);
                }
            }
            acc = mx_wave_sum(acc);
            if (lane == 0 && row0 + r < N) out(m0 + mm, row0 + r, acc);
        }
    };
    // The first token runs outside any loop: in a loop that only reads
    // registers loaded before it, every load would be waited for at its entry,
    // while here row r waits for its own chunks only.
    lds_barrier();
    token(0, 0);
    for (int mm = 1; mm < mt0; ++mm) token(0, mm);
    for (int m0 = mt; m0 < M; m0 += mt) {
        const int mtc = min(mt, M - m0);
        lds_barrier();  // every wave is done with the previous tokens
        stage(m0, mtc, 0);
        lds_barrier();
        for (int mm = 0; mm < mtc; ++mm) token(m0, mm);
    }
}

// Tokens staged at once for K inputs (at least one).
inline int mx_tokens_per_chunk(int K, int M) {
    int mt = kMxActBudget / mx_token_rec(K);
    if (mt < 1) mt = 1;
    return mt < M ? mt : M;
}

}  // namespace qg
