// Block-quantized weight x Q8 activation: the per-lane group decoders and the
// wave-level tile engine shared by the dense GEMV and the routed-MoE kernels.
//
// Work decomposition (MI355X-first, not taken from the pages' kernels):
//   * A "group" is 256 consecutive weights of one row: 8 Q8_0 blocks (272 B)
//     or one Q4_K superblock (144 B).  One lane decodes one group.
//   * A wave owns a "tile": R whole rows, R = 64 / lanes_per_row, where
//     lanes_per_row is K/256 rounded up to a power of two (<= 64).  The tile
//     is contiguous in memory, so the wave copies it HBM -> LDS with
//     16-byte direct-to-LDS loads: every load instruction moves 1 KiB of
//     consecutive bytes (fully coalesced), no VGPRs are used for staging.
//   * Each lane then reads its own group from LDS (16-byte reads; the 34-byte
//     Q8_0 blocks are re-aligned in registers with byte-align ops), forms the
//     per-block int32 sums with 4-way int8 dot products against the Q8
//     activation, scales them in fp32, and the lanes of a row combine their
//     partial sums with a fixed xor-butterfly (deterministic, the same order
//     for every token and every call).
#pragma once

#include "common.h"

namespace qg {

struct TileGeom {
    int gpr;  // groups per row = K / 256
    int lpr;  // lanes per row (power of two >= gpr, <= 64)
    int lsh;  // log2(lpr)
    int rpt;  // rows per tile = 64 / lpr
};

inline TileGeom make_tile_geom(int K) {
    TileGeom t;
    t.gpr = K / kGroupWeights;
    t.lpr = 1;
    t.lsh = 0;
    while (t.lpr < t.gpr) {
        t.lpr <<= 1;
        t.lsh += 1;
    }
    t.rpt = kWave / t.lpr;
    return t;
}

// ---------------------------------------------------------------- decoders

// One lane, one Q8_0 group (8 blocks, 68 dwords in w) against one token's
// activation for the same 256 inputs: qx8 = 64 dwords of int8 quants, dxg =
// the 8 block scales.  Returns sum_b (dw_b * dx_b) * isum_b in fp32 (blocks in
// order).  If isum_out is non-null the 8 exact block sums are stored there.
__device__ __forceinline__ float group_dot_q8_0(const uint32_t (&w)[68], const int8_t *__restrict__ qx8,
                                                const float *__restrict__ dxg, int32_t *isum_out) {
    const uint4 *qv = reinterpret_cast<const uint4 *>(qx8);
    const float4 dlo = reinterpret_cast<const float4 *>(dxg)[0];
    const float4 dhi = reinterpret_cast<const float4 *>(dxg)[1];
    const float dx[8] = {dlo.x, dlo.y, dlo.z, dlo.w, dhi.x, dhi.y, dhi.z, dhi.w};
    float acc = 0.0f;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int byte0 = 34 * b;   // block start inside the group
        const int dw0 = byte0 / 4;  // dword holding the fp16 scale
        const uint32_t sbits = (b & 1) ? (w[dw0] >> 16) : (w[dw0] & 0xffffu);
        const float dwt = half_bits_to_float(sbits);
        const uint4 q0 = qv[2 * b], q1 = qv[2 * b + 1];
        const uint32_t qa[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        int isum = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t wq;
            if (b & 1)
                wq = w[(byte0 + 2) / 4 + k];  // odd block: quants start dword-aligned
            else
                wq = align_bytes(w[dw0 + k + 1], w[dw0 + k], 2);  // even block: 2 bytes in
            isum = sdot4(wq, qa[k], isum);
        }
        if (isum_out) isum_out[b] = isum;
        acc = fmaf_exact((float)isum, dwt * dx[b], acc);
    }
    return acc;
}

// 6-bit field f (0..15) of the 96-bit little-endian string in s[0..2].
__device__ __forceinline__ uint32_t q4k_field(const uint32_t s0, const uint32_t s1, const uint32_t s2, int f) {
    const int bit = 6 * f;
    const int word = bit >> 5;
    const int off = bit & 31;
    const uint32_t lo = word == 0 ? s0 : (word == 1 ? s1 : s2);
    const uint32_t hi = word == 0 ? s1 : (word == 1 ? s2 : 0u);
    const uint32_t v = off == 0 ? lo : ((lo >> off) | (hi << (32 - off)));
    return v & 63u;
}

// One lane, one Q4_K superblock (36 dwords in w) against one token's
// activation for the same 256 inputs (qx8: 64 dwords, dxg/sxg: 8 scales and
// block sums).  Per sub-block j:
//   dx_j * (d*sc_j * isum_j - dmin*m_j * sx_j)
// with d*sc_j and dmin*m_j exact in fp32 (11-bit x 6-bit products).
__device__ __forceinline__ float group_dot_q4k(const uint32_t (&w)[36], const int8_t *__restrict__ qx8,
                                               const float *__restrict__ dxg, const int32_t *__restrict__ sxg,
                                               int32_t *isum_out) {
    const uint4 *qv = reinterpret_cast<const uint4 *>(qx8);
    const float4 dlo = reinterpret_cast<const float4 *>(dxg)[0];
    const float4 dhi = reinterpret_cast<const float4 *>(dxg)[1];
    const int4 slo = reinterpret_cast<const int4 *>(sxg)[0];
    const int4 shi = reinterpret_cast<const int4 *>(sxg)[1];
    const float dx[8] = {dlo.x, dlo.y, dlo.z, dlo.w, dhi.x, dhi.y, dhi.z, dhi.w};
    const int sx[8] = {slo.x, slo.y, slo.z, slo.w, shi.x, shi.y, shi.z, shi.w};
    const float d = half_bits_to_float(w[0]);
    const float dmin = half_bits_to_float(w[0] >> 16);
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint4 a0 = qv[4 * p], a1 = qv[4 * p + 1];  // sub-block 2p
        const uint4 b0 = qv[4 * p + 2], b1 = qv[4 * p + 3];  // sub-block 2p+1
        const uint32_t qa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const uint32_t qb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        int ia = 0, ib = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t v = w[4 + 8 * p + k];
            ia = sdot4(v & 0x0F0F0F0Fu, qa[k], ia);
            ib = sdot4((v >> 4) & 0x0F0F0F0Fu, qb[k], ib);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = 2 * p + h;
            const int isum = h ? ib : ia;
            if (isum_out) isum_out[j] = isum;
            const float a = d * (float)q4k_field(w[1], w[2], w[3], j);
            const float bm = dmin * (float)q4k_field(w[1], w[2], w[3], 8 + j);
            const float inner = fmaf_exact(a, (float)isum, -(bm * (float)sx[j]));
            acc = fmaf_exact(inner, dx[j], acc);
        }
    }
    return acc;
}

// ---------------------------------------------------------------- tile engine

// Start copying tile `tile` of matrix W (rows tile*rpt .. +rpt, clipped to N)
// into the wave's LDS buffer; the copy is left in flight (wait with
// wait_vmem_all before reading).  Returns the number of rows in the tile.
template <int FMT>
__device__ __forceinline__ int issue_tile_to_lds(const uint8_t *__restrict__ W, int N, const TileGeom &tg, int tile,
                                                 uint8_t *lds_wave) {
    constexpr int GB = GroupBytes<FMT>::value;
    const int lane = lane_id();
    const int row0 = tile * tg.rpt;
    const int nrows = min(tg.rpt, N - row0);
    const uint8_t *src = W + (size_t)row0 * tg.gpr * GB;
    const int nchunks = nrows * tg.gpr * (GB / 16);
    for (int i = 0; i * kWave < nchunks; ++i) {
        const int c = i * kWave + lane;
        if (c < nchunks) global_to_lds16(src + (size_t)c * 16, lds_wave + i * 1024);
    }
    return nrows;
}

template <int FMT>
struct GroupRegs;
template <>
struct GroupRegs<QG_FMT_Q8_0> {
    uint32_t w[68];
};
template <>
struct GroupRegs<QG_FMT_Q4K> {
    uint32_t w[36];
};

// Read this lane's group from the wave's LDS tile buffer.
template <int FMT>
__device__ __forceinline__ void read_group(const uint8_t *lds_group, GroupRegs<FMT> &g) {
    constexpr int NV = GroupBytes<FMT>::value / 16;
    const uint4 *p = reinterpret_cast<const uint4 *>(lds_group);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const uint4 v = p[i];
        g.w[4 * i + 0] = v.x;
        g.w[4 * i + 1] = v.y;
        g.w[4 * i + 2] = v.z;
        g.w[4 * i + 3] = v.w;
    }
}

template <int FMT>
__device__ __forceinline__ float group_dot(const GroupRegs<FMT> &g, const int8_t *qx8, const float *dxg,
                                           const int32_t *sxg, int32_t *isum_out);
template <>
__device__ __forceinline__ float group_dot<QG_FMT_Q8_0>(const GroupRegs<QG_FMT_Q8_0> &g, const int8_t *qx8,
                                                        const float *dxg, const int32_t *, int32_t *isum_out) {
    return group_dot_q8_0(g.w, qx8, dxg, isum_out);
}
template <>
__device__ __forceinline__ float group_dot<QG_FMT_Q4K>(const GroupRegs<QG_FMT_Q4K> &g, const int8_t *qx8,
                                                       const float *dxg, const int32_t *sxg, int32_t *isum_out) {
    return group_dot_q4k(g.w, qx8, dxg, sxg, isum_out);
}

// Sum over the lpr lanes of a row with a fixed xor butterfly; every lane of
// the row ends with the same value.
__device__ __forceinline__ float row_reduce(float p, int lpr) {
    for (int off = 1; off < lpr; off <<= 1) p += shfl_xor(p, off);
    return p;
}


// ---------------------------------------------------------------- activation staging

// LDS for staged activations per workgroup (the weight tiles take
// waves * 64 * group bytes on top; 4 waves: Q8_0 68 KiB, Q4_K 36 KiB).
constexpr int kActLdsBudget = 44 * 1024;

// Activations are staged in LDS as one record per 256-input group: 64 dwords
// of quants, 8 block scales (+ 8 block sums for Q4_K), padded so that the
// record stride is an odd multiple of 4 dwords.  Lanes of a wave read
// different groups at the same offset; with this stride their 16-byte reads
// fall in disjoint banks (a 256-byte stride would put them all in one).
template <int FMT>
struct ActRecord {
    static constexpr int dwords = FMT == QG_FMT_Q4K ? 84 : 76;  // 80 + 4 / 72 + 4
    static constexpr int bytes = dwords * 4;
};

template <int FMT>
__host__ __device__ inline int act_lds_bytes_per_token(int K) {
    return (K / kGroupWeights) * ActRecord<FMT>::bytes;
}

template <int FMT>
inline int tokens_per_chunk(int K, int M) {
    return max(1, min(min(M, kMaxChunkTokens), kActLdsBudget / act_lds_bytes_per_token<FMT>(K)));
}

template <int FMT>
inline size_t gemv_lds_bytes(int waves, int K, int mt) {
    return (size_t)waves * kWave * GroupBytes<FMT>::value + (size_t)mt * act_lds_bytes_per_token<FMT>(K) +
           (size_t)kMaxChunkTokens * sizeof(int);
}

// Stage tokens m0 .. m0+mt-1 (activation rows rows_lds[0..mt) of qx/dx/sx)
// into padded LDS records (whole workgroup; global -> VGPR -> LDS, 16 bytes
// per access).
template <int FMT, int WAVES>
__device__ __forceinline__ void stage_activations(const int8_t *__restrict__ qx, const float *__restrict__ dx,
                                                  const int32_t *__restrict__ sx, int K, int mt,
                                                  const int *rows_lds, uint8_t *lds) {
    constexpr int REC = ActRecord<FMT>::bytes;
    const int gpr = K / kGroupWeights;
    const int cpt = K / 16;  // 16-byte chunks of quants per token
    for (int c = threadIdx.x; c < mt * cpt; c += WAVES * kWave) {
        const int mm = c / cpt;
        const int w = c - mm * cpt;
        const uint4 *q = reinterpret_cast<const uint4 *>(qx + (size_t)rows_lds[mm] * K);
        *reinterpret_cast<uint4 *>(lds + (size_t)(mm * gpr + (w >> 4)) * REC + (w & 15) * 16) = q[w];
    }
    const int spt = gpr * 2;  // 16-byte chunks of scales per token
    for (int c = threadIdx.x; c < mt * spt; c += WAVES * kWave) {
        const int mm = c / spt;
        const int w = c - mm * spt;
        const size_t src = (size_t)rows_lds[mm] * (K / 32) / 4 + w;  // in uint4 units
        uint8_t *rec = lds + (size_t)(mm * gpr + (w >> 1)) * REC + 256 + (w & 1) * 16;
        *reinterpret_cast<uint4 *>(rec) = reinterpret_cast<const uint4 *>(dx)[src];
        if (FMT == QG_FMT_Q4K) *reinterpret_cast<uint4 *>(rec + 32) = reinterpret_cast<const uint4 *>(sx)[src];
    }
}

// ---------------------------------------------------------------- workgroup engine

// One workgroup of WAVES waves; each wave owns weight tile `tile` of W (if
// has_tile).  The tile is copied HBM -> LDS and kept; the M tokens are
// processed in chunks of mt_max, each chunk staged once in LDS for the whole
// workgroup.  token_row(m) gives the activation row of token m; out(m, row, v)
// stores one result; isum_out(m, row, g, sums8) receives the exact block sums
// when DEBUG_ISUM.  Every wave of the workgroup must call this (barriers).
template <int FMT, int WAVES, bool DEBUG_ISUM, class TokenRow, class Out, class IsumOut>
__device__ __forceinline__ void gemv_tiles_workgroup(const uint8_t *__restrict__ W, int N, int K, const TileGeom &tg,
                                                     int tile, bool has_tile, const int8_t *qx, const float *dx,
                                                     const int32_t *sx, int M, int mt_max, uint8_t *smem,
                                                     TokenRow token_row, Out out, IsumOut isum_out) {
    constexpr int GB = GroupBytes<FMT>::value;
    constexpr int REC = ActRecord<FMT>::bytes;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    uint8_t *lw = smem + wave * kWave * GB;
    uint8_t *lact = smem + WAVES * kWave * GB;
    int *lrows = reinterpret_cast<int *>(lact + (size_t)mt_max * act_lds_bytes_per_token<FMT>(K));

    // 1. this wave's weight tile: HBM -> LDS, left in flight
    int nrows = 0;
    if (has_tile) nrows = issue_tile_to_lds<FMT>(W, N, tg, tile, lw);
    const int r = lane >> tg.lsh;
    const int g = lane & (tg.lpr - 1);
    const bool valid = has_tile && g < tg.gpr && r < nrows;
    const int row = tile * tg.rpt + r;
    GroupRegs<FMT> regs;

    for (int m0 = 0; m0 < M; m0 += mt_max) {
        const int mt = min(mt_max, M - m0);
        if (m0 > 0) __syncthreads();  // every wave is done with the previous chunk
        for (int i = threadIdx.x; i < mt; i += WAVES * kWave) lrows[i] = token_row(m0 + i);
        __syncthreads();
        // 2. the chunk's activation quants, scales (and block sums), shared by the workgroup
        stage_activations<FMT, WAVES>(qx, dx, sx, K, mt, lrows, lact);
        wait_vmem_all();  // this wave's weight tile has landed in LDS
        __syncthreads();
        if (m0 == 0 && valid) read_group<FMT>(lw + (r * tg.gpr + g) * GB, regs);

        for (int mm = 0; mm < mt; ++mm) {
            float p = 0.0f;
            if (valid) {
                int32_t isum_tmp[8];
                const uint8_t *rec = lact + (size_t)(mm * tg.gpr + g) * REC;
                p = group_dot<FMT>(regs, reinterpret_cast<const int8_t *>(rec),
                                   reinterpret_cast<const float *>(rec + 256),
                                   reinterpret_cast<const int32_t *>(rec + 288), DEBUG_ISUM ? isum_tmp : nullptr);
                if (DEBUG_ISUM) isum_out(m0 + mm, row, g, isum_tmp);
            }
            p = row_reduce(p, tg.lpr);
            if (!DEBUG_ISUM && valid && g == 0) out(m0 + mm, row, p);
        }
    }
}

}  // namespace qg
