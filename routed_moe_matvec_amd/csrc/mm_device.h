// The matrix-core tile of the batched block-quantized mat-vec (Q8_0 and Q4_K
// weights x Q8 activation on v_mfma_i32_32x32x32_i8), shared by the dense
// batched calls and prefill (gemv_mm.hip) and the routed experts with many
// pairs (moe.hip).  The numerics are those of the one-token engine of
// gemv_device.h; see gemv_mm.hip.
#pragma once

#include <type_traits>

#include "common.h"
#include "gemv_device.h"

namespace qg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kMmRows = 32;    // weight rows of a workgroup
constexpr int kMmTokens = 32;  // tokens of a workgroup

// Per format: 16-byte parts of a row's 256-weight group (Q8_0: 8 blocks of
// 34 bytes; Q4_K: one 144-byte superblock), the load instructions that move
// a group of 32 rows (the last one 32 chunks), and the per-group scale table
// (Q8_0: fp16 block scales; Q4_K: fp32 d*sc and dmin*m of each sub-block).
template <int FMT>
struct MmFmt;
template <>
struct MmFmt<QG_FMT_Q8_0> {
    static constexpr int parts = 17;
    static constexpr int table_bytes = 8 * kMmRows * 2;
};
template <>
struct MmFmt<QG_FMT_Q4K> {
    static constexpr int parts = 9;
    static constexpr int table_bytes = 8 * kMmRows * 4 * 2;
};
template <int FMT>
constexpr int mm_stage_bytes() { return MmFmt<FMT>::parts * kMmRows * 16; }
template <int FMT>
constexpr int mm_loads() { return (MmFmt<FMT>::parts * kMmRows + kWave - 1) / kWave; }
// Whether a tile of gps groups per slice and tt token tiles stages its
// activation through LDS (below): where the extra LDS costs no waves per CU.
constexpr bool mm_act_lds(int gps, int tt) { return tt > 1 || (gps >= 2 && gps <= 4); }
// The LDS activation tile of a wave: 8 16-byte chunks x 32 tokens, token
// stride 33 chunks.
constexpr int kMmActTile = 8 * 33 * 16;
// LDS of a wave: the stage, the scale table, the pending tree levels 1 and 2
// (slices of four or eight groups) and the activation tile
template <int FMT>
constexpr int mm_wave_lds(int gps, int tt = 1) {
    return mm_stage_bytes<FMT>() + MmFmt<FMT>::table_bytes + (gps >= 8 ? 2 : gps >= 4 ? 1 : 0) * 16 * 64 * 4 +
           (mm_act_lds(gps, tt) ? kMmActTile : 0);
}
constexpr int kMmMaxSlices = 8;       // waves of a workgroup
constexpr int kMmMaxGroups = 8;       // groups of a slice (three stored tree levels)
constexpr int kMmTargetWaves = 2048;  // about two waves per SIMD over the chip

// One workgroup's tile: rows row0 .. row0 + 31 of the N-row matrix W against
// tokens m0 .. m0 + 31 of M; act_row(m) is token m's row in qx / dx / sx,
// out(m, row, v) stores a result.
struct MmTile {
    const uint8_t *W;
    int N, row0, m0, M;
    const int8_t *qx;
    const float *dx;
    const int32_t *sx;
    int K, row_bytes, groups, gps, KS;
};

// An empty statement that reads and writes 16 registers: the values are
// computed before it, and it keeps its place among the statements with side
// effects (memory operations, scheduling barriers).
__device__ __forceinline__ void pin16(float (&v)[16]) {
    asm volatile(""
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                   "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),
                   "+v"(v[15]));
}

template <int FMT, int NB, int GPS, int TT, class ActRow, class Out>
__device__ __forceinline__ void mm_tile(const MmTile &t, ActRow act_row, Out out, uint8_t *smem) {
    using F = MmFmt<FMT>;
    static_assert(TT == 1 || FMT == QG_FMT_Q8_0, "token tiles share a stage for Q8_0 only");
    constexpr int kParts = F::parts, kGroupBytes = kParts * 16, kStage = mm_stage_bytes<FMT>();
    // TT token tiles of 32 share each slice's stage: a wave loads 1/TT of a group
    constexpr int kChunks = kParts * kMmRows, kShare = kChunks / TT, kLoads = (kShare + kWave - 1) / kWave;
    static_assert(kShare * TT == kChunks && kLoads >= 2, "stage share");
    // the wave index is uniform over the wave: keep it (and every slice bound) scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int KS = t.KS;
    const int sl = TT == 1 ? wave : wave % KS;  // K slice
    const int tt = TT == 1 ? 0 : wave / KS;     // token tile within the workgroup
    const uint8_t *W = t.W;
    const int N = t.N, row0 = t.row0, m0 = t.m0 + kMmTokens * tt;
    // LDS: TT = 1, per wave [stage | table | levels | activation tile]; TT >
    // 1, per slice two stages (double-buffered: one barrier per group), then
    // per wave [table | levels | activation tile] (the activation tile only
    // where ACTL)
    constexpr int kWaveLds = mm_wave_lds<FMT>(GPS, TT);
    constexpr bool ACTL = mm_act_lds(GPS, TT);
    uint8_t *stage0 = TT == 1 ? smem + wave * kWaveLds : smem + sl * 2 * kStage;
    uint8_t *stab = TT == 1 ? stage0 + kStage : smem + KS * 2 * kStage + wave * (kWaveLds - kStage);

    const int grp0 = sl * t.gps;
    const int ngroups = min(max(t.groups - grp0, 0), t.gps);

    // Group loads: the 32 rows x kParts parts (16 bytes) of a group in row
    // order, chunk c = kParts r + p; the wave's share is chunks tt kShare ..
    // + kShare, instruction i / lane l taking chunk tt kShare + 64 i + l, so
    // that an instruction reads a few contiguous runs of a row's group (few
    // cache lines per instruction: the address units, not HBM, bounded an
    // earlier pattern of 16 rows x 64 bytes).  Lanes past the share repeat the
    // chunk 64 before (the same bytes to the same place).  Rows past N re-read
    // row N - 1.
    const int r32 = lane & 31, half = lane >> 5;
    const uint8_t *wt = W + (size_t)row0 * t.row_bytes;
    uint32_t goff[kLoads], soff[TT == 1 ? 1 : kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        int idx = tt * kShare + 64 * i + lane;
        if (idx >= (tt + 1) * kShare) idx -= 64;
        const int r = idx / kParts, p = idx - kParts * r;
        goff[i] = (uint32_t)(min(row0 + r, N - 1) - row0) * (uint32_t)t.row_bytes + 16u * p;
        if constexpr (TT > 1) soff[i] = 16u * idx;
    }
    // activation: token lane % 32 (tokens past M re-read token M - 1; their
    // columns are not stored), 16 quants of each block per lane half.
    // ACTL: the 32 tokens x 128 bytes of a half group are read with 16-byte
    // loads in which lane l takes token 8 i + l / 8 of instruction i < 4 and
    // bytes 16 (l % 8) of the half group (8 runs of 128 bytes per
    // instruction, instead of 32 tokens x 32 bytes: the address units bounded
    // the latter), into the wave's LDS activation tile [chunk][token], from
    // which each block's B operand is one conflict-free 16-byte read.
    const size_t arow = (size_t)act_row(min(m0 + r32, t.M - 1));
    const int8_t *xp = t.qx + arow * t.K + 16 * half;
    // ACTL: byte offsets of tokens 8 i + l / 8, in 32 bits: every caller's
    // activation is below 4 GiB (qx rows x K < 2^32; the dense calls route
    // larger batches to the dot-product engine; the routed experts index at
    // most QG_MAX_MOE_PAIRS rows of at most QG_MAX_K bytes)
    uint32_t crow[ACTL ? 4 : 1];
    if constexpr (ACTL) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            crow[i] = (uint32_t)act_row(min(m0 + 8 * i + (lane >> 3), t.M - 1)) * (uint32_t)t.K + 16u * (lane & 7);
    }
    constexpr int kLevels = GPS >= 8 ? 2 : GPS >= 4 ? 1 : 0;
    uint8_t *atile = stab + F::table_bytes + kLevels * 16 * 64 * 4;
    const float *dp = t.dx + arow * (t.K / 32);
    const int32_t *sp = FMT == QG_FMT_Q4K ? t.sx + arow * (t.K / 32) : nullptr;

    auto load_w = [&](int gi, u32x4 (&w)[kLoads]) __attribute__((always_inline)) {
        const uint8_t *base = wt + (size_t)gi * kGroupBytes;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) w[i] = __builtin_nontemporal_load(as_global<u32x4>(base + goff[i]));
    };
    // the 8 block scales of the token (and, Q4_K, the 8 block sums as floats)
    auto load_dx = [&](int gi, float4 (&d)[4]) __attribute__((always_inline)) {
        d[0] = reinterpret_cast<const float4 *>(dp + 8 * gi)[0];
        d[1] = reinterpret_cast<const float4 *>(dp + 8 * gi)[1];
        if constexpr (FMT == QG_FMT_Q4K) {
            const int4 s0 = reinterpret_cast<const int4 *>(sp + 8 * gi)[0];
            const int4 s1 = reinterpret_cast<const int4 *>(sp + 8 * gi)[1];
            d[2] = make_float4((float)s0.x, (float)s0.y, (float)s0.z, (float)s0.w);
            d[3] = make_float4((float)s1.x, (float)s1.y, (float)s1.z, (float)s1.w);
        }
    };
    auto load_act = [&](int gi, int b) __attribute__((always_inline)) { return *reinterpret_cast<const i32x4 *>(xp + (size_t)gi * 256 + 32 * b); };
    // ACTL: half ph of group gi's activation into registers, and into the tile
    auto load_half = [&](int gi, int ph, u32x4 (&c)[4]) __attribute__((always_inline)) {
        const int8_t *base = t.qx + (size_t)gi * 256 + 128 * ph;
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = *reinterpret_cast<const u32x4 *>(base + crow[i]);
    };
    auto write_half = [&](const u32x4 (&c)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4 *>(atile + 16 * ((lane & 7) * 33 + 8 * i + (lane >> 3))) = c[i];
    };

    // Stage layout: row r's group bytes at kParts * 16 r, i.e. chunk
    // kParts r + p at 16 times that, so the loads' chunks are written
    // linearly; a 16-lane pass reading one part of 16 rows hits 16 different
    // 16-byte bank groups (row strides of 68 and 36 dwords).
    auto store_w = [&](uint8_t *stage, const u32x4 (&w)[kLoads]) __attribute__((always_inline)) {
        if constexpr (TT == 1) {
            // chunk 64 i + l; the last instruction's lanes 32..63 hold repeats
#pragma unroll
            for (int i = 0; i < kLoads - 1; ++i) *reinterpret_cast<u32x4 *>(stage + 16 * (64 * i + lane)) = w[i];
            if (lane < 32) *reinterpret_cast<u32x4 *>(stage + 16 * (64 * (kLoads - 1) + lane)) = w[kLoads - 1];
        } else {
#pragma unroll
            for (int i = 0; i < kLoads; ++i) *reinterpret_cast<u32x4 *>(stage + soff[i]) = w[i];
        }
    };
    // A-operand reads: part p0 + half of row lane % 32 sits at abase + 16 p0
    const int abase = kParts * 16 * r32 + 16 * half;
    // Scale table of the stage, arranged so that a lane half reads the 16 rows
    // 8q + 4 half + t of its MFMA result as consecutive entries: Q8_0 the fp16
    // block scales [block][slot]; Q4_K d*sc_j and dmin*m_j as fp32
    // [sub-block][a | bm][slot] (exact products: 11-bit by 6-bit)
    const int slot = ((r32 >> 2) & 1) * 16 + (r32 >> 3) * 4 + (r32 & 3);
    auto build_scales = [&](const uint8_t *stage) __attribute__((always_inline)) {
        if constexpr (FMT == QG_FMT_Q8_0) {
            // (all four reads before the writes: one LDS round trip)
            uint16_t v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = *reinterpret_cast<const uint16_t *>(stage + kParts * 16 * r32 + 34 * (4 * half + j));
#pragma unroll
            for (int j = 0; j < 4; ++j) *reinterpret_cast<uint16_t *>(stab + 2 * ((4 * half + j) * 32 + slot)) = v[j];
        } else {
            const u32x4 hd = *reinterpret_cast<const u32x4 *>(stage + kParts * 16 * r32);
            const float d = half_bits_to_float(hd.x), dmin = half_bits_to_float(hd.x >> 16);
            float *tab = reinterpret_cast<float *>(stab);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int jj = 4 * half + j;
                tab[(2 * jj) * 32 + slot] = d * (float)q4k_field(hd.y, hd.z, hd.w, jj);
                tab[(2 * jj + 1) * 32 + slot] = dmin * (float)q4k_field(hd.y, hd.z, hd.w, 8 + jj);
            }
        }
    };

    // Tree levels of the slice: st0 (registers) holds a pending group node;
    // a pending pair (level 1) and quad (level 2) wait in the wave's LDS level
    // area (16 floats per lane, lane-interleaved); top receives the slice's
    // full subtree.  Group i of the slice enters with a static index (the step
    // loop is unrolled), so every carry is fixed code.
    float st0[16], top[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) st0[e] = top[e] = 0.0f;
    float *lvl = reinterpret_cast<float *>(stab + F::table_bytes);  // [level - 1][16][64]
    auto lvl_store = [&](int k, const float (&v)[16]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) lvl[((k - 1) * 16 + e) * kWave + lane] = v[e];
    };
    auto lvl_add = [&](int k, float (&v)[16]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = lvl[((k - 1) * 16 + e) * kWave + lane] + v[e];
    };
    auto push = [&](float (&v)[16], auto index) __attribute__((always_inline)) {
        constexpr int i = decltype(index)::value;
        if constexpr (GPS == 1) {
#pragma unroll
            for (int e = 0; e < 16; ++e) top[e] = v[e];
        } else if constexpr (!(i & 1)) {
#pragma unroll
            for (int e = 0; e < 16; ++e) st0[e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = st0[e] + v[e];
            if constexpr (GPS == 2) {
#pragma unroll
                for (int e = 0; e < 16; ++e) top[e] = v[e];
            } else if constexpr (!(i & 2)) {
                lvl_store(1, v);
            } else {
                lvl_add(1, v);
                if constexpr (GPS == 4) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) top[e] = v[e];
                } else if constexpr (!(i & 4)) {
                    lvl_store(2, v);
                } else {
                    lvl_add(2, v);
#pragma unroll
                    for (int e = 0; e < 16; ++e) top[e] = v[e];
                }
            }
        }
    };

    // Group j of the slice, clamped to the slice's last group (and to the
    // row's last group for an empty slice): steps past the slice's end re-read
    // a valid group.
    auto gclamp = [&](int j) __attribute__((always_inline)) {
        return min(grp0 + min(j, max(ngroups - 1, 0)), t.groups - 1);
    };
    // Weights are requested two groups ahead (two register sets), activations
    // and their scales one group ahead.  A step's weight request for the group
    // after next is issued after its activation requests for the next group:
    // loads complete in order, so the next step's activation waits do not
    // wait for those weights.
    // dxv: the token's 8 block scales, then (Q4_K) its 8 block sums as floats
    constexpr int DXV = FMT == QG_FMT_Q4K ? 4 : 2;
    u32x4 wreg[2][kLoads];
    float4 dxv[4];
    i32x4 act[ACTL ? 1 : 8];
    u32x4 actc[ACTL ? 2 : 1][4];  // ACTL: the two half groups in flight
    load_dx(gclamp(0), dxv);
    if constexpr (ACTL) {
        load_half(gclamp(0), 0, actc[0]);
        load_half(gclamp(0), 1, actc[1]);
    } else {
#pragma unroll
        for (int b = 0; b < 8; ++b) act[b] = load_act(gclamp(0), b);
    }
    load_w(gclamp(0), wreg[0]);
    if constexpr (GPS > 1) load_w(gclamp(1), wreg[1]);

    // LDS reads of one block of a stage: the 16-byte parts of the A operand
    // and the block's scale-table entries (Q8_0: 32 fp16 scales; Q4_K: 32
    // d*sc and 32 dmin*m)
    struct ARaw {
        u32x4 c0, c1;
        i32x4 bop;  // ACTL: the block's B operand
    };
    struct SRaw {
        u32x4 v[FMT == QG_FMT_Q4K ? 8 : 2];
    };

    // Step s multiplies group grp0 + s.  Every step runs, also past the end of
    // a partial slice, where it re-reads the slice's last group and enters a
    // zero leaf (the one-token engine pads its tree with zeros): with no
    // branch around a step, each wait for a group's weights counts only the
    // loads issued before them (a step behind a branch made it wait for every
    // load in flight).
    auto step = [&](auto index) __attribute__((always_inline)) {
        constexpr int s = decltype(index)::value;
        constexpr bool PF = s + 1 < GPS;   // activation of the next group
        constexpr bool PF2 = s + 2 < GPS;  // weights of the group after it
        const bool real = s < ngroups;
        const int gnext = gclamp(s + 1);
        // steps are not interleaved by the scheduler (registers)
        __builtin_amdgcn_sched_barrier(0);
        uint8_t *stage = TT == 1 ? stage0 : stage0 + (s & 1) * kStage;
        store_w(stage, wreg[s & 1]);
        if constexpr (TT > 1) lds_barrier();  // the slice's whole group is staged
        build_scales(stage);
        float4 dxn[4];
        if constexpr (PF) load_dx(gnext, dxn);
        if constexpr (ACTL) {
            write_half(actc[0]);
            if constexpr (PF) load_half(gnext, 0, actc[0]);
        }
        auto a_read = [&](auto bi) __attribute__((always_inline)) {
            constexpr int b = decltype(bi)::value;
            ARaw r;
            if constexpr (FMT == QG_FMT_Q8_0) {
                constexpr int o = 34 * b + 2;
                constexpr int p0 = o >> 4, sh = o & 15;
                r.c0 = *reinterpret_cast<const u32x4 *>(stage + abase + 16 * p0);
                r.c1 = r.c0;
                if constexpr (sh != 0) r.c1 = *reinterpret_cast<const u32x4 *>(stage + abase + 16 * (p0 + 1));
            } else {
                r.c0 = *reinterpret_cast<const u32x4 *>(stage + abase + 16 * (1 + 2 * (b >> 1)));
                r.c1 = r.c0;
            }
            if constexpr (ACTL) r.bop = *reinterpret_cast<const i32x4 *>(atile + 16 * ((2 * (b & 3) + half) * 33 + r32));
            return r;
        };
        auto s_read = [&](auto bi) __attribute__((always_inline)) {
            constexpr int b = decltype(bi)::value;
            SRaw r;
            if constexpr (FMT == QG_FMT_Q4K) {
                const u32x4 *x = reinterpret_cast<const u32x4 *>(stab + 4 * ((2 * b) * 32 + 16 * half));
                const u32x4 *y = reinterpret_cast<const u32x4 *>(stab + 4 * ((2 * b + 1) * 32 + 16 * half));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    r.v[q] = x[q];
                    r.v[4 + q] = y[q];
                }
            } else {
                r.v[0] = *reinterpret_cast<const u32x4 *>(stab + 64 * b + 32 * half);
                r.v[1] = *reinterpret_cast<const u32x4 *>(stab + 64 * b + 32 * half + 16);
            }
            return r;
        };
        // block b's integer sums: A operand = quants 16 half .. 16 half + 15 of
        // block (Q4_K: sub-block) b of row lane % 32 (Q8_0: realigned bytes;
        // Q4_K: the low / high nibbles of the 32 bytes that sub-blocks 2p and
        // 2p + 1 share); without ACTL the next group's activation for block b
        // is requested after it
        auto block_sums = [&](auto bi, const ARaw &r) __attribute__((always_inline)) {
            constexpr int b = decltype(bi)::value;
            i32x4 A;
            if constexpr (FMT == QG_FMT_Q8_0) {
                constexpr int o = 34 * b + 2;
                constexpr int sh = o & 15, wd = sh >> 2, bs = sh & 3;
                const uint32_t D[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) A[k] = (int)(bs ? align_bytes(D[wd + k + 1], D[wd + k], bs) : D[wd + k]);
            } else {
                const uint32_t D[4] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) A[k] = (int)(((b & 1) ? (D[k] >> 4) : D[k]) & 0x0F0F0F0Fu);
            }
            const i32x16 zero = {};
            i32x16 is;
            if constexpr (ACTL) {
                is = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, r.bop, zero, 0, 0, 0);
            } else {
                is = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, act[b], zero, 0, 0, 0);
                if constexpr (PF) act[b] = load_act(gnext, b);
            }
            return is;
        };
        float acc[16], acc2[16];
        // scale and accumulate block b (the next block's product is already issued)
        auto block_scale = [&](auto bi, const i32x16 &is, const SRaw &sr) __attribute__((always_inline)) {
            constexpr int b = decltype(bi)::value;
            if constexpr (FMT == QG_FMT_Q4K) {
                // the one-token engine's sub-block step: inner = d sc_j isum -
                // dmin m_j sx_j (one fma on the rounded product), then
                // acc = fma(inner, dx_j, acc) from +0
                float av[16], bv[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 x = sr.v[q], y = sr.v[4 + q];
                    av[4 * q] = __uint_as_float(x.x), av[4 * q + 1] = __uint_as_float(x.y);
                    av[4 * q + 2] = __uint_as_float(x.z), av[4 * q + 3] = __uint_as_float(x.w);
                    bv[4 * q] = __uint_as_float(y.x), bv[4 * q + 1] = __uint_as_float(y.y);
                    bv[4 * q + 2] = __uint_as_float(y.z), bv[4 * q + 3] = __uint_as_float(y.w);
                }
                const float dxb = dxv[b >> 2][b & 3], sxb = dxv[2 + (b >> 2)][b & 3];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float inner = fmaf_exact(av[e], (float)is[e], -(bv[e] * sxb));
                    acc[e] = fmaf_exact(inner, dxb, b == 0 ? 0.0f : acc[e]);
                }
            } else {
                const uint32_t S[8] = {sr.v[0].x, sr.v[0].y, sr.v[0].z, sr.v[0].w,
                                       sr.v[1].x, sr.v[1].y, sr.v[1].z, sr.v[1].w};
                const float dxb = b < 4 ? dxv[0][b & 3] : dxv[1][b & 3];
                float *ac = (NB == 4 && b >= 4) ? acc2 : acc;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t pair = S[e >> 1];
                    const half2v h = __builtin_bit_cast(half2v, pair);
                    const float dw = (float)((e & 1) ? h.y : h.x);
                    // fp32 product dw * dx (the +0 addend lets it issue as one
                    // mixed-precision fma; a -0 product would become +0, which
                    // no later sum can tell apart, since no sum starts at -0)
                    const float sc = __builtin_fmaf(dw, dxb, 0.0f);
                    const float prev = (b % NB == 0) ? 0.0f : ac[e];
                    ac[e] = fmaf_exact((float)is[e], sc, prev);
                }
            }
        };
        // LDS reads run ahead of their use: block b + 2's A operand, and
        // (Q8_0) block b + 1's scales, are read while block b is scaled; Q4_K
        // reads a block's 32 table entries with it (a second set would not
        // fit the registers of two waves per SIMD)
        constexpr bool kScalesAhead = FMT == QG_FMT_Q8_0;
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        ARaw an = a_read(I0{});
        SRaw sn;
        if constexpr (kScalesAhead) sn = s_read(I0{});
        i32x16 cur = block_sums(I0{}, an);
        an = a_read(I1{});
        auto body = [&](auto bi) __attribute__((always_inline)) {
            constexpr int b = decltype(bi)::value;
            SRaw sc;
            if constexpr (kScalesAhead) sc = sn;
            i32x16 nxt;
            if constexpr (b < 7) nxt = block_sums(std::integral_constant<int, b + 1>{}, an);
            if constexpr (ACTL && b == 2) {
                // blocks 4-7: the second half group (block 3's operand is read)
                write_half(actc[1]);
                if constexpr (PF) load_half(gnext, 1, actc[1]);
            }
            if constexpr (b + 2 < 8) an = a_read(std::integral_constant<int, b + 2>{});
            if constexpr (kScalesAhead && b + 1 < 8) sn = s_read(std::integral_constant<int, b + 1>{});
            if constexpr (!kScalesAhead) sc = s_read(bi);
            __builtin_amdgcn_sched_barrier(0);
            block_scale(bi, cur, sc);
            // the scaling is plain arithmetic: pinned here, in the slot whose
            // LDS reads it hides, instead of sunk towards its last use (which
            // kept every block's product live)
            pin16((NB == 4 && FMT == QG_FMT_Q8_0 && b >= 4) ? acc2 : acc);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (b < 7) cur = nxt;
        };
        body(std::integral_constant<int, 0>{});
        body(std::integral_constant<int, 1>{});
        body(std::integral_constant<int, 2>{});
        body(std::integral_constant<int, 3>{});
        body(std::integral_constant<int, 4>{});
        body(std::integral_constant<int, 5>{});
        body(std::integral_constant<int, 6>{});
        body(std::integral_constant<int, 7>{});
        if constexpr (NB == 4) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = acc[e] + acc2[e];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = real ? acc[e] : 0.0f;
        push(acc, index);
        if constexpr (PF2) load_w(gclamp(s + 2), wreg[s & 1]);
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < DXV; ++i) dxv[i] = dxn[i];
        }
    };
    static_assert(GPS == 1 || GPS == 2 || GPS == 4 || GPS == 8, "groups per slice");
    step(std::integral_constant<int, 0>{});
    if constexpr (GPS > 1) step(std::integral_constant<int, 1>{});
    if constexpr (GPS > 2) {
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
    }
    if constexpr (GPS > 4) {
        step(std::integral_constant<int, 4>{});
        step(std::integral_constant<int, 5>{});
        step(std::integral_constant<int, 6>{});
        step(std::integral_constant<int, 7>{});
    }

    // The slice's subtree (zero leaves past a partial slice's end).
    float r[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) r[e] = top[e];
    // slices meet in LDS: TT = 1, in each wave's own stage; TT > 1, in its
    // slice's stages (4 KiB per token tile) once every wave is done with them
    static_assert(TT == 1 || TT * 4096 <= 2 * kStage, "combine area");
    auto comb_at = [&](int s_) __attribute__((always_inline)) {
        return reinterpret_cast<float *>(TT == 1 ? smem + s_ * kWaveLds : smem + s_ * 2 * kStage + tt * 4096);
    };
    if constexpr (TT > 1) lds_barrier();
    float *comb = comb_at(sl);
#pragma unroll
    for (int e = 0; e < 16; ++e) comb[e * 64 + lane] = r[e];
    lds_barrier();
    for (int idx = sl * kWave + lane; idx < 16 * 64; idx += KS * kWave) {
        float v[kMmMaxSlices];
#pragma unroll
        for (int s = 0; s < kMmMaxSlices; ++s) v[s] = s < KS ? comb_at(s)[idx] : 0.0f;
#pragma unroll
        for (int w = 1; w < kMmMaxSlices; w <<= 1)
#pragma unroll
            for (int s = 0; s + w < kMmMaxSlices; s += 2 * w)
                if (s + w < KS) v[s] = v[s] + v[s + w];
        const int e = idx >> 6, l = idx & 63;
        const int token = m0 + (l & 31);
        const int row = row0 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
        if (token < t.M && row < N) out(token, row, v[0]);
    }
}

// Slices (waves) per workgroup and groups per slice for `groups` 256-weight
// groups per row and `tiles` workgroup tiles: at most eight groups per slice,
// at most eight slices, and more slices while the grid has fewer than about
// two waves per SIMD.
inline void mm_slices(int groups, long tiles, int *ks_out, int *gps_out) {
    int gpow2 = 1;
    while (gpow2 < groups) gpow2 <<= 1;
    int ks = gpow2 > kMmMaxGroups ? gpow2 / kMmMaxGroups : 1;
    const int ks_max = gpow2 < kMmMaxSlices ? gpow2 : kMmMaxSlices;
    while (ks < ks_max && tiles * ks < kMmTargetWaves) ks <<= 1;
    *ks_out = ks;
    *gps_out = gpow2 / ks;
}

}  // namespace qg
