// Block-quantized weight x Q8 activation: per-lane unit decoders and the
// workgroup-level tile engine shared by the dense GEMV and the routed-MoE
// kernels.
//
// Work decomposition (MI355X-first, not taken from the pages' kernels):
//   * A "unit" is the run of one row's weights that one lane decodes:
//     4 Q8_0 blocks (128 weights, 136 B) when K <= 8192, 8 Q8_0 blocks (256
//     weights, 272 B) for larger K, or one Q4_K superblock (256 weights, 144 B).
//   * A wave owns a "tile" of whole rows, at most 64 units (8.5-17 KiB): rows
//     are contiguous in memory, so the wave reads the tile with 16-byte loads
//     in which every instruction moves 1 KiB of consecutive bytes.  Loads are
//     non-temporal (the weights are streamed once) and land in VGPRs, so the
//     compiler tracks their completion exactly; a wave keeps up to two tiles
//     in flight in two register sets and decodes one while the next arrives.
//   * To hand every lane its own unit, the wave writes the tile to a private
//     LDS buffer and reads its unit back (8/16-byte LDS reads; the 34-byte
//     Q8_0 blocks are re-aligned in registers with byte-align ops).
//   * The per-block int32 sums come from 4-way int8 dot products against the
//     Q8 activation, which the workgroup stages once in LDS as padded
//     per-unit records; they are scaled in fp32 with explicit fma, and the
//     lanes of a row combine their partial sums with a fixed xor butterfly
//     (deterministic, the same order for every token and every call).
#pragma once

#include "common.h"
#include "quantize_device.h"

namespace qg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- units

template <int FMT, int NB>
struct Unit;
// Q8_0, NB blocks of 34 bytes per lane
template <int NB>
struct Unit<QG_FMT_Q8_0, NB> {
    static constexpr int blocks = NB;
    static constexpr int weights = 32 * NB;
    static constexpr int bytes = 34 * NB;
    static constexpr int dwords = 17 * NB / 2;
    // activation record: quants, then NB scales; stride an odd multiple of 4 dwords
    static constexpr int rec_dwords = NB == 4 ? 36 : 76;
};
template <>
struct Unit<QG_FMT_Q4K, 8> {
    static constexpr int blocks = 8;
    static constexpr int weights = 256;
    static constexpr int bytes = 144;
    static constexpr int dwords = 36;
    static constexpr int rec_dwords = 84;  // 64 quants + 8 scales + 8 block sums + 4 pad
};

template <class U>
struct UnitRegs {
    uint32_t w[U::dwords];
};

// Q8_0 blocks of a unit against one token's record; returns
// sum_b (dw_b * dx_b) * isum_b in fp32 in block order.
template <int NB>
__device__ __forceinline__ float unit_dot_q8_0(const uint32_t (&w)[17 * NB / 2], const uint8_t *rec,
                                               int32_t *isum_out) {
    const u32x4 *qv = reinterpret_cast<const u32x4 *>(rec);
    const float *dxp = reinterpret_cast<const float *>(rec + 32 * NB);
    float acc = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int byte0 = 34 * b;   // block start inside the unit
        const int dw0 = byte0 / 4;  // dword holding the fp16 scale
        const uint32_t sbits = (b & 1) ? (w[dw0] >> 16) : (w[dw0] & 0xffffu);
        const float dwt = half_bits_to_float(sbits);
        const u32x4 q0 = qv[2 * b], q1 = qv[2 * b + 1];
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
        acc = fmaf_exact((float)isum, dwt * dxp[b], acc);
    }
    return acc;
}

// 6-bit field f (0..15) of the 96-bit little-endian string in s0..s2.
__device__ __forceinline__ uint32_t q4k_field(const uint32_t s0, const uint32_t s1, const uint32_t s2, int f) {
    const int bit = 6 * f;
    const int word = bit >> 5;
    const int off = bit & 31;
    const uint32_t lo = word == 0 ? s0 : (word == 1 ? s1 : s2);
    const uint32_t hi = word == 0 ? s1 : (word == 1 ? s2 : 0u);
    const uint32_t v = off == 0 ? lo : ((lo >> off) | (hi << (32 - off)));
    return v & 63u;
}

// One Q4_K superblock against one token's record (64 dwords of quants, 8
// scales, 8 block sums).  Per sub-block j:
//   dx_j * (d*sc_j * isum_j - dmin*m_j * sx_j)
// with d*sc_j and dmin*m_j exact in fp32 (11-bit x 6-bit products).
__device__ __forceinline__ float unit_dot_q4k(const uint32_t (&w)[36], const uint8_t *rec, int32_t *isum_out) {
    const u32x4 *qv = reinterpret_cast<const u32x4 *>(rec);
    const float *dxp = reinterpret_cast<const float *>(rec + 256);
    const int32_t *sxp = reinterpret_cast<const int32_t *>(rec + 288);
    const float d = half_bits_to_float(w[0]);
    const float dmin = half_bits_to_float(w[0] >> 16);
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4 a0 = qv[4 * p], a1 = qv[4 * p + 1];      // sub-block 2p
        const u32x4 b0 = qv[4 * p + 2], b1 = qv[4 * p + 3];  // sub-block 2p+1
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
            const float inner = fmaf_exact(a, (float)isum, -(bm * (float)sxp[j]));
            acc = fmaf_exact(inner, dxp[j], acc);
        }
    }
    return acc;
}

template <int FMT, int NB>
__device__ __forceinline__ float unit_dot(const UnitRegs<Unit<FMT, NB>> &u, const uint8_t *rec, int32_t *isum_out) {
    if constexpr (FMT == QG_FMT_Q8_0)
        return unit_dot_q8_0<NB>(u.w, rec, isum_out);
    else
        return unit_dot_q4k(u.w, rec, isum_out);
}

// Read this lane's unit from the wave's LDS tile buffer (16-byte reads when
// the unit is 16-byte aligned, else 8-byte reads).
template <class U>
__device__ __forceinline__ void read_unit(const uint8_t *p, UnitRegs<U> &u) {
    if constexpr (U::bytes % 16 == 0) {
#pragma unroll
        for (int i = 0; i < U::dwords / 4; ++i) {
            const u32x4 v = reinterpret_cast<const u32x4 *>(p)[i];
            u.w[4 * i] = v.x;
            u.w[4 * i + 1] = v.y;
            u.w[4 * i + 2] = v.z;
            u.w[4 * i + 3] = v.w;
        }
    } else {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < U::dwords / 2; ++i) {
            const u32x2 v = reinterpret_cast<const u32x2 *>(p)[i];
            u.w[2 * i] = v.x;
            u.w[2 * i + 1] = v.y;
        }
    }
}

// ---------------------------------------------------------------- geometry

struct TileGeom {
    int upr;  // units per row
    int lpr;  // lanes per row (power of two >= upr, <= 64)
    int lsh;  // log2(lpr)
    int rpt;  // rows per tile = 64 / lpr
    int row_bytes;
    // ceil(2^32 / d) for d = K / 16, K / 128 and K / 4: the token of a staging
    // chunk index c is then the high half of c times this, with no division in
    // the kernel (exact while c * d < 2^32: the product overshoots c / d by less
    // than c / 2^32 < 1 / d, and the fraction of c / d is at most 1 - 1 / d)
    uint32_t qdiv, sdiv, fdiv;
};

inline uint32_t recip32(uint32_t d) { return (uint32_t)(((1ull << 32) + d - 1) / d); }

template <class U>
inline TileGeom make_tile_geom(int K) {
    TileGeom t;
    t.upr = K / U::weights;
    t.lpr = 1;
    t.lsh = 0;
    while (t.lpr < t.upr) {
        t.lpr <<= 1;
        t.lsh += 1;
    }
    t.rpt = kWave / t.lpr;
    t.row_bytes = t.upr * U::bytes;
    t.qdiv = recip32((uint32_t)(K / 16));
    t.sdiv = recip32((uint32_t)(K / 128));
    t.fdiv = recip32((uint32_t)(K / 4));
    return t;
}

template <class U>
struct TileSize {
    static constexpr int bytes = kWave * U::bytes;           // a full tile
    static constexpr int instr = (bytes + 1023) / 1024;      // 16-byte loads per lane
    static constexpr int lds = (bytes + 15) / 16 * 16;       // LDS it occupies
};

// ---------------------------------------------------------------- activation staging

// LDS of one CU, and the most the staged activations of a workgroup take.
constexpr int kLdsBytes = 160 * 1024;
constexpr int kActLdsBudget = 44 * 1024;
// 16-byte activation chunks each thread holds in registers while staging.
constexpr int kActRegChunks = 4;

// Register chunks for one pass over `chunks` 16-byte chunks (1, 2 or 4): a
// pass that fits fewer saves the registers and the clamped duplicate reads
// (and, from fp32, the duplicate quantization) of the unused ones.
inline int act_reg_chunks(int chunks, int threads) {
    return chunks <= threads ? 1 : (chunks <= 2 * threads ? 2 : kActRegChunks);
}

template <class U>
__host__ __device__ inline int act_lds_bytes_per_token(int K) {
    return (K / U::weights) * U::rec_dwords * 4;
}

// Tokens staged at once: bounded by the LDS budget, and preferably by what
// one pass of the staging registers holds (larger rows take extra passes).
template <class U>
inline int tokens_per_chunk(int K, int M, int threads, bool f32_input = false) {
    const int budget = min(kActLdsBudget, kLdsBytes - (threads / kWave) * TileSize<U>::lds);
    int mt = budget / act_lds_bytes_per_token<U>(K);
    mt = min(mt, kActRegChunks * threads * (f32_input ? 4 : 16) / K);
    return max(1, min(mt, M));
}

template <class U>
inline size_t gemv_lds_bytes(int waves, int K, int mt) {
    return (size_t)waves * TileSize<U>::lds + (size_t)mt * act_lds_bytes_per_token<U>(K);
}

// Staging of one chunk of tokens [m0, m0 + mtc) of the Q8 activation into
// padded per-unit LDS records, split in two halves: load() issues the global
// reads of the first slice into registers, store() writes the records (and
// reads and writes whatever did not fit the registers in further passes).
// Between the two the caller issues its weight loads, which then stay in
// flight: the waits for the activation registers only cover loads issued
// before them.
template <int FMT, class U, bool ONE, int RC = kActRegChunks>
struct ActStage {
    static constexpr int REC = U::rec_dwords * 4;
    u32x4 q[RC];
    u32x4 d, s;
    uint32_t qdiv, sdiv;  // TileGeom's reciprocals of K / 16 and K / 128

    // token (within the chunk of tokens) of quant chunk c / of scale chunk c:
    // always 0 in the one-token form
    __device__ __forceinline__ int qtok(int c) const { return ONE ? 0 : (int)__umulhi((uint32_t)c, qdiv); }
    __device__ __forceinline__ int stok(int c) const { return ONE ? 0 : (int)__umulhi((uint32_t)c, sdiv); }

    // Chunk c of the token chunk's quants (16 bytes; c < mtc * K / 16).
    template <class TokenRow>
    __device__ __forceinline__ const u32x4 *quant_src(const int8_t *__restrict__ qx, int K, int m0, int c,
                                                      TokenRow token_row) {
        const int cpt = K / 16;
        const int mm = qtok(c);
        return reinterpret_cast<const u32x4 *>(qx + (size_t)token_row(m0 + mm) * K) + (c - mm * cpt);
    }
    __device__ __forceinline__ uint8_t *quant_dst(uint8_t *lds, int K, int c) {
        constexpr int QC = U::weights / 16;  // 16-byte chunks of quants per unit
        const int cpt = K / 16, upr = K / U::weights;
        const int mm = qtok(c);
        const int w = c - mm * cpt;
        const int u = w / QC;
        return lds + (size_t)(mm * upr + u) * REC + (w - u * QC) * 16;
    }
    // Chunk c of the scales (and block sums) of 4 blocks (c < mtc * K / 128).
    template <class TokenRow>
    __device__ __forceinline__ size_t scale_src(int K, int m0, int c, TokenRow token_row) {
        const int spt = K / 128;
        const int mm = stok(c);
        return (size_t)token_row(m0 + mm) * (K / 32) / 4 + (c - mm * spt);
    }
    __device__ __forceinline__ uint8_t *scale_dst(uint8_t *lds, int K, int c) {
        constexpr int SC = U::blocks / 4;  // 16-byte chunks of scales per unit
        const int spt = K / 128, upr = K / U::weights;
        const int mm = stok(c);
        const int w = c - mm * spt;
        const int u = w / SC;
        return lds + (size_t)(mm * upr + u) * REC + U::weights + (w - u * SC) * 16;
    }

    // load() reads the first pass (the registers) and store() writes it,
    // both unconditionally and outside any loop: a thread past the end takes
    // one of the last 64 chunks instead (each lane a different one, so the
    // duplicate writes, of identical bytes to the same place, do not pile on
    // one LDS address).  The waits for the registers then count only the loads
    // issued after them; a conditional load, or a first pass inside the pass
    // loop, would make them wait for the caller's weight loads as well.
    __device__ __forceinline__ static int clamp_chunk(int c, int total) {
        return c < total ? c : max(total - kWave + lane_id(), 0);
    }
    template <class TokenRow>
    __device__ __forceinline__ void load(const int8_t *__restrict__ qx, const float *__restrict__ dx,
                                         const int32_t *__restrict__ sx, int K, int m0, int mtc, TokenRow token_row) {
        const int NT = blockDim.x;
        const int qtotal = mtc * (K / 16), stotal = mtc * (K / 128);
        const int cpt = K / 16, spt = K / 128;
        // the token rows first (a gathered token list costs one round trip
        // for all of them), then the activation reads
        // (index RC: the scales' token)
        int c[RC + 1], mm[RC + 1];
        size_t row[RC + 1];
#pragma unroll
        for (int k = 0; k < RC; ++k) {
            c[k] = clamp_chunk((int)threadIdx.x + k * NT, qtotal);
            mm[k] = qtok(c[k]);
        }
        c[RC] = clamp_chunk((int)threadIdx.x, stotal);
        mm[RC] = stok(c[RC]);
#pragma unroll
        for (int k = 0; k <= RC; ++k) row[k] = (size_t)token_row(m0 + mm[k]);
#pragma unroll
        for (int k = 0; k < RC; ++k)
            q[k] = reinterpret_cast<const u32x4 *>(qx + row[k] * K)[c[k] - mm[k] * cpt];
        const size_t src = row[RC] * (K / 32) / 4 + (c[RC] - mm[RC] * spt);
        d = reinterpret_cast<const u32x4 *>(dx)[src];
        if constexpr (FMT == QG_FMT_Q4K) s = reinterpret_cast<const u32x4 *>(sx)[src];
    }

    template <class TokenRow>
    __device__ __forceinline__ void store(uint8_t *lds, const int8_t *__restrict__ qx, const float *__restrict__ dx,
                                          const int32_t *__restrict__ sx, int K, int m0, int mtc,
                                          TokenRow token_row) {
        const int NT = blockDim.x;
        const int qtotal = mtc * (K / 16), stotal = mtc * (K / 128);
#pragma unroll
        for (int k = 0; k < RC; ++k)
            *reinterpret_cast<u32x4 *>(quant_dst(lds, K, clamp_chunk((int)threadIdx.x + k * NT, qtotal))) = q[k];
        {
            uint8_t *rec = scale_dst(lds, K, clamp_chunk((int)threadIdx.x, stotal));
            *reinterpret_cast<u32x4 *>(rec) = d;
            if constexpr (FMT == QG_FMT_Q4K) *reinterpret_cast<u32x4 *>(rec + 32) = s;
        }
        // further passes (chunks that did not fit the registers)
        for (int base = RC * NT; base < qtotal; base += RC * NT) {
#pragma unroll
            for (int k = 0; k < RC; ++k) {
                const int c = base + (int)threadIdx.x + k * NT;
                if (c < qtotal) q[k] = *quant_src(qx, K, m0, c, token_row);
            }
#pragma unroll
            for (int k = 0; k < RC; ++k) {
                const int c = base + (int)threadIdx.x + k * NT;
                if (c < qtotal) *reinterpret_cast<u32x4 *>(quant_dst(lds, K, c)) = q[k];
            }
        }
        for (int c = NT + (int)threadIdx.x; c < stotal; c += NT) {
            const size_t src = scale_src(K, m0, c, token_row);
            uint8_t *rec = scale_dst(lds, K, c);
            *reinterpret_cast<u32x4 *>(rec) = reinterpret_cast<const u32x4 *>(dx)[src];
            if constexpr (FMT == QG_FMT_Q4K) *reinterpret_cast<u32x4 *>(rec + 32) = reinterpret_cast<const u32x4 *>(sx)[src];
        }
    }
};

// Where a workgroup takes its activation from.  Either a Q8 activation
// (qx/dx/sx, as quantize_act_q8 writes it), or the fp32 activation x, which
// every workgroup quantizes itself while staging (the same 8-lane block
// quantizer, so the records are bit-identical); workgroup 0 then also
// publishes the Q8 activation to pqx/pdx/psx when they are given.
struct ActSrc {
    const int8_t *qx;
    const float *dx;
    const int32_t *sx;
    const float *x;
    int8_t *pqx;
    float *pdx;
    int32_t *psx;
    const float *x2;  // kSrcGLU: the second input (x holds the gate outputs, x2 the up outputs)
    float *ph;        // kSrcGLU: where the publishing workgroup writes h = silu(x) * x2
};

// What a workgroup stages: a Q8 activation, an fp32 activation it quantizes,
// or the SwiGLU product h = silu(g) * v of two fp32 inputs, quantized.
constexpr int kSrcQ8 = 0;
constexpr int kSrcF32 = 1;
constexpr int kSrcGLU = 2;


// Staging from fp32: load() reads the first kActRegChunks 16-byte chunks
// (4 values each) per thread into registers, store() quantizes each 32-block
// on its 8 consecutive lanes and writes the records; chunks beyond what the
// registers held are read and quantized in further passes inside store().
// GLU = true reads two inputs and stages h = silu(g) * v.  As in ActStage,
// the first pass is read and written unconditionally, threads past the end
// taking one of the last 64 chunks (whole 32-blocks per 8-lane group, since
// the chunk count is a multiple of 64), and ONE fixes the token to 0.
template <int FMT, class U, bool GLU, bool ONE, int RC = kActRegChunks>
struct ActStageF32 {
    static constexpr int REC = U::rec_dwords * 4;
    float4 v[RC];
    float4 v2[GLU ? RC : 1];
    uint32_t fdiv;  // TileGeom's reciprocal of K / 4

    __device__ __forceinline__ int ftok(int c) const { return ONE ? 0 : (int)__umulhi((uint32_t)c, fdiv); }
    __device__ __forceinline__ static int clamp_chunk(int c, int total) {
        return c < total ? c : total - kWave + lane_id();
    }

    template <class TokenRow>
    __device__ __forceinline__ void load_pass(const ActSrc &src, int K, int m0, int mtc, int base,
                                              TokenRow token_row) {
        const int NT = blockDim.x;
        const int cpt = K / 4;
#pragma unroll
        for (int k = 0; k < RC; ++k) {
            const int c = base + (int)threadIdx.x + k * NT;
            if (c < mtc * cpt) {
                const int mm = ftok(c);
                const size_t at = (size_t)token_row(m0 + mm) * K;
                v[k] = reinterpret_cast<const float4 *>(src.x + at)[c - mm * cpt];
                if constexpr (GLU) v2[k] = reinterpret_cast<const float4 *>(src.x2 + at)[c - mm * cpt];
            }
        }
    }

    template <class TokenRow>
    __device__ __forceinline__ void load(const ActSrc &src, int K, int m0, int mtc, TokenRow token_row) {
        const int NT = blockDim.x;
        const int cpt = K / 4, total = mtc * cpt;
        int c[RC], mm[RC];
        size_t at[RC];
#pragma unroll
        for (int k = 0; k < RC; ++k) {
            c[k] = clamp_chunk((int)threadIdx.x + k * NT, total);
            mm[k] = ftok(c[k]);
        }
#pragma unroll
        for (int k = 0; k < RC; ++k) at[k] = (size_t)token_row(m0 + mm[k]) * K;
#pragma unroll
        for (int k = 0; k < RC; ++k) {
            v[k] = reinterpret_cast<const float4 *>(src.x + at[k])[c[k] - mm[k] * cpt];
            if constexpr (GLU) v2[k] = reinterpret_cast<const float4 *>(src.x2 + at[k])[c[k] - mm[k] * cpt];
        }
    }

    // quantize chunk c (values of register set k) with its 8-lane group and
    // write the record bytes (and the published copies) when valid
    template <class TokenRow>
    __device__ __forceinline__ void emit(uint8_t *lds, int K, int m0, int c, int k, bool valid, TokenRow token_row,
                                         const ActSrc &src, bool publish) {
        const int cpt = K / 4, upr = K / U::weights;
        float vals[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        if constexpr (GLU) {
            vals[0] = silu(vals[0]) * v2[k].x;
            vals[1] = silu(vals[1]) * v2[k].y;
            vals[2] = silu(vals[2]) * v2[k].z;
            vals[3] = silu(vals[3]) * v2[k].w;
        }
        if (!valid) vals[0] = vals[1] = vals[2] = vals[3] = 0.0f;
        int8_t q[4];
        float d;
        int32_t s;
        quantize_block_8lanes(vals, q, &d, &s);  // every lane takes part (shuffles)
        if (valid) {
            const int mm = ftok(c);
            const int w = c - mm * cpt;
            const int blk = w >> 3, part = w & 7;
            const int u = blk / U::blocks, bi = blk - u * U::blocks;
            const uint32_t packed = (uint32_t)(uint8_t)q[0] | ((uint32_t)(uint8_t)q[1] << 8) |
                                    ((uint32_t)(uint8_t)q[2] << 16) | ((uint32_t)(uint8_t)q[3] << 24);
            uint8_t *rec = lds + (size_t)(mm * upr + u) * REC;
            *reinterpret_cast<uint32_t *>(rec + 32 * bi + 4 * part) = packed;
            if (part == 0) {
                *reinterpret_cast<float *>(rec + U::weights + 4 * bi) = d;
                if constexpr (FMT == QG_FMT_Q4K) *reinterpret_cast<int32_t *>(rec + U::weights + 32 + 4 * bi) = s;
            }
            if (publish) {
                const size_t row = (size_t)token_row(m0 + mm);
                if (GLU && src.ph)
                    *reinterpret_cast<float4 *>(src.ph + row * K + 4 * w) = make_float4(vals[0], vals[1], vals[2], vals[3]);
                if (src.pqx) *reinterpret_cast<uint32_t *>(src.pqx + row * K + 32 * blk + 4 * part) = packed;
                if (part == 0) {
                    if (src.pdx) src.pdx[row * (K / 32) + blk] = d;
                    if (src.psx) src.psx[row * (K / 32) + blk] = s;
                }
            }
        }
    }

    template <class TokenRow>
    __device__ __forceinline__ void store(uint8_t *lds, int K, int m0, int mtc, TokenRow token_row,
                                          const ActSrc &src, bool publish) {
        const int NT = blockDim.x;
        const int total = mtc * (K / 4);
        // 8 consecutive lanes hold one 32-block
#pragma unroll
        for (int k = 0; k < RC; ++k)
            emit(lds, K, m0, clamp_chunk((int)threadIdx.x + k * NT, total), k, true, token_row, src, publish);
        for (int base = RC * NT; base < total; base += RC * NT) {
            load_pass(src, K, m0, mtc, base, token_row);
#pragma unroll
            for (int k = 0; k < RC; ++k) {
                const int c = base + (int)threadIdx.x + k * NT;
                emit(lds, K, m0, c, k, c < total, token_row, src, publish);
            }
        }
    }
};

// ---------------------------------------------------------------- tile engine

// Sum over the lpr lanes of a row as the fixed pairwise tree of an xor
// butterfly: level k adds the partner lane^2^k; every lane of the row ends
// with the same value.  After level k every lane of an aligned 2^k group
// holds the same value, so a mirror inside the next larger group reaches a
// lane of the partner group: levels 1-2 are quad permutations, 3-4 half-row
// and row mirrors (all DPP), 5 a swizzle with xor 16, 6 one lane permute.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_reduce(float p, int lpr) {
    if (lpr >= 2) p += dpp_f32<0xB1>(p);   // quad_perm [1, 0, 3, 2]: lane ^ 1
    if (lpr >= 4) p += dpp_f32<0x4E>(p);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    if (lpr >= 8) p += dpp_f32<0x141>(p);  // row_half_mirror: the other quad of 8
    if (lpr >= 16) p += dpp_f32<0x140>(p); // row_mirror: the other 8 of 16
    if (lpr >= 32)                         // swizzle, bit mode and 0x1f, xor 0x10
        p += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, p), 0x401F));
    if (lpr >= 64) p += shfl_xor(p, 32);
    return p;
}

template <class U>
struct TileRegs {
    u32x4 v[TileSize<U>::instr];
};

// Issue the 16-byte non-temporal loads of tile `tile` (rows tile*rpt ..
// +rpt clipped to N).  Lanes past the end of the tile re-read its last
// chunk, so every lane issues every load and none leaves the matrix.
template <class U>
__device__ __forceinline__ void load_tile(const uint8_t *__restrict__ W, int N, const TileGeom &tg, int tile,
                                          TileRegs<U> &r) {
    const int lane = lane_id();
    const int row0 = tile * tg.rpt;
    const int nrows = min(tg.rpt, N - row0);
    const int last = nrows * tg.row_bytes / 16 - 1;
    const auto *src = as_global<u32x4>(W + (size_t)row0 * tg.row_bytes);
#pragma unroll
    for (int i = 0; i < TileSize<U>::instr; ++i) {
        const int c = min(i * kWave + lane, last);
        r.v[i] = __builtin_nontemporal_load(src + c);
    }
}

// Write a loaded tile to the wave's LDS buffer and read this lane's unit back.
template <class U>
__device__ __forceinline__ void tile_to_unit(const TileRegs<U> &r, uint8_t *lw, int unit_index, bool valid,
                                             UnitRegs<U> &u) {
    const int lane = lane_id();
    __builtin_amdgcn_wave_barrier();  // this wave's earlier reads of the buffer are issued first
#pragma unroll
    for (int i = 0; i < TileSize<U>::instr; ++i)
        if (i * 1024 + lane * 16 < TileSize<U>::bytes) *reinterpret_cast<u32x4 *>(lw + i * 1024 + lane * 16) = r.v[i];
    __builtin_amdgcn_wave_barrier();  // LDS executes one wave's accesses in order
    if (valid) read_unit<U>(lw + unit_index * U::bytes, u);
}

// The workgroup engine (blockDim.x / 64 waves).  Wave w of the workgroup processes tiles
// tile_base + w*tpw + i (i < tpw, tile < ntiles) of matrix W against M tokens.
// token_row(m) gives the activation row of token m; out(m, row, v) stores one
// result; isum_out(m, row, unit, sums) receives the exact block sums when
// DEBUG_ISUM.  Tokens are staged in chunks of mt; with more than one chunk,
// tpw must be 1 (the tile stays in registers across chunks).  Every wave of
// the workgroup must call this (it synchronizes).  PIPE = false limits tpw
// to 1 and keeps only one tile register set; ONE = true is the M = 1 form
// (no token loop, fewer live registers); SRC picks what is staged (kSrcQ8,
// kSrcF32 or kSrcGLU, see ActSrc); RC is the 16-byte chunks of activation
// each thread stages per pass (act_reg_chunks).
template <int FMT, int NB, bool DEBUG_ISUM, bool PIPE, bool ONE, int SRC, int RC = kActRegChunks,
          class TokenRow, class Out, class IsumOut>
__device__ __forceinline__ void gemv_workgroup(const uint8_t *__restrict__ W, int N, int K, const TileGeom &tg,
                                               int tile_base, int tpw, int ntiles, const ActSrc &src, int M, int mt,
                                               uint8_t *smem, TokenRow token_row, Out out, IsumOut isum_out) {
    using U = Unit<FMT, NB>;
    constexpr int REC = U::rec_dwords * 4;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    uint8_t *lw = smem + wave * TileSize<U>::lds;
    uint8_t *lact = smem + (blockDim.x / kWave) * TileSize<U>::lds;
    const int tile0 = tile_base + wave * tpw;
    const int r = lane >> tg.lsh;
    const int g = lane & (tg.lpr - 1);

    auto compute = [&](const UnitRegs<U> &u, int tile, bool valid, int m0, int mtc) {
        const int row = tile * tg.rpt + r;
        if (ONE) mtc = 1;
        for (int mm = 0; mm < mtc; ++mm) {
            float p = 0.0f;
            if (valid) {
                int32_t isum_tmp[U::blocks];
                p = unit_dot<FMT, NB>(u, lact + (size_t)(mm * tg.upr + g) * REC, DEBUG_ISUM ? isum_tmp : nullptr);
                if (DEBUG_ISUM) isum_out(m0 + mm, row, g, isum_tmp);
            }
            p = row_reduce(p, tg.lpr);
            if (!DEBUG_ISUM && valid && g == 0) out(m0 + mm, row, p);
        }
    };
    auto unit_valid = [&](int tile) { return tile < ntiles && g < tg.upr && tile * tg.rpt + r < N; };

    TileRegs<U> ra, rb;
    UnitRegs<U> u;
    constexpr bool F32 = SRC != kSrcQ8;
    ActStage<FMT, U, ONE, RC> st;
    st.qdiv = tg.qdiv;
    st.sdiv = tg.sdiv;
    ActStageF32<FMT, U, SRC == kSrcGLU, ONE, RC> stf;
    stf.fdiv = tg.fdiv;
    // fp32 input: workgroup (0, 0) publishes the Q8 activation; SwiGLU input:
    // workgroup 0 of each blockIdx.y (one expert: its own pairs) publishes h
    const bool publish = SRC == kSrcF32 ? (blockIdx.x == 0 && blockIdx.y == 0) : (SRC == kSrcGLU && blockIdx.x == 0);
    auto act_load = [&](int m0, int mtc) {
        if constexpr (F32)
            stf.load(src, K, m0, mtc, token_row);
        else
            st.load(src.qx, src.dx, src.sx, K, m0, mtc, token_row);
    };
    auto act_store = [&](int m0, int mtc) {
        if constexpr (F32)
            stf.store(lact, K, m0, mtc, token_row, src, publish);
        else
            st.store(lact, src.qx, src.dx, src.sx, K, m0, mtc, token_row);
    };
    if (ONE || M <= mt) {
        if (ONE) M = 1;
        // one chunk of tokens: activation reads first, then up to two tiles in
        // flight; tpw tiles in total
        // (the first tiles are read unconditionally, clamped to the last tile,
        // so the staging waits count them exactly; see ActStage)
        act_load(0, M);
        load_tile<U>(W, N, tg, min(tile0, ntiles - 1), ra);
        if (PIPE) load_tile<U>(W, N, tg, min(tile0 + 1, ntiles - 1), rb);
        __builtin_amdgcn_sched_barrier(0);  // every load is issued before the first wait
        act_store(0, M);
        lds_barrier();
        for (int i = 0; i < tpw; i += 2) {
            const int ta = tile0 + i, tb = tile0 + i + 1;
            if (ta < ntiles) {
                const bool v = unit_valid(ta);
                tile_to_unit<U>(ra, lw, r * tg.upr + g, v, u);
                if (PIPE && i + 2 < tpw && ta + 2 < ntiles) load_tile<U>(W, N, tg, ta + 2, ra);
                compute(u, ta, v, 0, M);
            }
            if (PIPE && i + 1 < tpw && tb < ntiles) {
                const bool v = unit_valid(tb);
                tile_to_unit<U>(rb, lw, r * tg.upr + g, v, u);
                if (i + 3 < tpw && tb + 2 < ntiles) load_tile<U>(W, N, tg, tb + 2, rb);
                compute(u, tb, v, 0, M);
            }
        }
    } else if (!ONE) {
        // several chunks of tokens: one tile, kept in registers across chunks;
        // the next chunk's activation is read into the staging registers while
        // the current chunk is multiplied
        const bool v = unit_valid(tile0);
        act_load(0, min(mt, M));
        load_tile<U>(W, N, tg, min(tile0, ntiles - 1), ra);
        __builtin_amdgcn_sched_barrier(0);
        act_store(0, min(mt, M));
        lds_barrier();
        if (tile0 < ntiles) tile_to_unit<U>(ra, lw, r * tg.upr + g, v, u);
        for (int m0 = 0; m0 < M; m0 += mt) {
            const int n0 = m0 + mt;
            if (n0 < M) act_load(n0, min(mt, M - n0));
            if (tile0 < ntiles) compute(u, tile0, v, m0, min(mt, M - m0));
            if (n0 < M) {
                lds_barrier();  // every wave is done with this chunk
                act_store(n0, min(mt, M - n0));
                lds_barrier();
            }
        }
    }
}

// Tiles per wave for a launch: about one round of the chip's resident waves,
// at most 4 (one chunk of tokens only).
inline int tiles_per_wave(int ntiles, int resident_waves, bool single_chunk) {
    if (!single_chunk) return 1;
    const int t = (ntiles + resident_waves - 1) / resident_waves;
    return t < 1 ? 1 : (t > 4 ? 4 : t);
}

// The matrix-core form of the Q8_0 / Q4_K mat-vec on a Q8 activation
// (gemv_mm.hip): same arguments and results, bit for bit, as the engine above
// for one matrix (W1 = NULL) or a pair, G groups, M tokens (sx: Q4_K only).
int gemv_mm(int fmt, const uint8_t *W0, int N0, float *y0, const uint8_t *W1, int N1, float *y1, int K,
            const int8_t *qx, const float *dx, const int32_t *sx, int M, int G, hipStream_t stream);

}  // namespace qg
