// Routed-MoE decode over a compact selected-expert table.
//
// "ROCm: restore DeepSeek V4 Flash decode performance and Q4 SSD streaming"
// (antirez/ds4 PR 623), Summary and Correctness: the compact table of the
// selected experts must be staged before the pointer-backed routed-MoE
// launch; its absence, or an expert id outside the expert range, is a hard
// decode error.  Routing is 6 of 256/384 experts with sigmoid-normalized
// weights (ROCm/ATOM "DeepSeek-V4 Usage Guide", opening paragraph and MoE
// tips).  The experts are Q4_K (the "Q4KExperts" model of PR 623), or FP8
// E4M3 with 128 x 128 block scales / FP4 E2M1 with 1 x 32 scales (the routed
// expert formats of the same guide, section "FP8 on MI308 / gfx942"), which
// run gate/up and down on the engine of mx_device.h.
//
// Launches on the caller's stream, none of which returns data to the host:
//   1. table   : validate ids, distinct experts ascending, slots, CSR pair lists
//                (one wave: bitmap of the selected experts, popcount ranks,
//                ballot-based stable fill)
//   2. gate/up : per distinct expert, gate and up rows against each of its
//                pairs' tokens (weights streamed once per expert)
//   3. h       : h = silu(g) * up, Q8-quantized per 32-block (T > 1 only)
//   4. down    : per distinct expert, down rows against each pair's Q8 h
//   5. combine : y[t] = sum_k rw[t,k] * o[t,k] in k order
// Grids 2 and 4 are sized for the largest possible number of distinct experts,
// min(T*topk, E); workgroups beyond the device-side count exit at once.  With
// one token every expert has one pair (or a few, if the token repeats an id):
// then 2 and 4 use the single-token form of the engine, once per pair, and 4
// computes and quantizes h itself while staging it, so 3 is not launched.
#include "common.h"
#include "gemv_device.h"
#include "mm_device.h"
#include "mx_device.h"
#include "quantize_device.h"

namespace qg {

constexpr int kMoeWaves = 4;
// tokens staged at once by the several-token expert kernels: most experts of
// a decode batch have a few pairs, and a staging area of up to three tokens
// still lets three workgroups share a CU's LDS (four would leave two)
constexpr int kMoeChunk = 3;
constexpr int kTableWords = QG_MAX_EXPERTS / 32;  // bitmap words over the expert ids
// Q4_K experts with at least kMoeMm pairs run on the matrix cores (tiles of 32
// pairs) when T >= kMoeMm; the dot-product kernels leave them out
constexpr int kMoeMm = QG_MOE_MM_PAIRS;
// matrix-core work items: a bound on the sum over such experts of their
// 32-pair tiles (at most P / kMoeMm experts, P / 32 + one partial tile each)
static inline int moe_mm_cap(int P) { return P / 32 + P / kMoeMm + 1; }

struct MoeWs {
    int32_t *nuniq, *uniq, *slot, *pair_off, *pairs;
    float *g, *v, *h;
    int8_t *hq;
    float *hd;
    int32_t *hs;
    float *o;
    int32_t *hot;  // [0]: matrix-core work items; then (slot, first pair) per item
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int moe_shape_ok(int T, int topk, int E, int D, int F) {
    if (T < 1 || topk < 1 || E < 1 || E > QG_MAX_EXPERTS) return 0;
    if ((long long)T * topk > QG_MAX_MOE_PAIRS) return 0;
    if (D < kGroupWeights || D > QG_MAX_K || D % kGroupWeights) return 0;
    if (F < kGroupWeights || F > QG_MAX_K || F % kGroupWeights) return 0;
    return 1;
}

// Byte offsets of the workspace regions; returns the total size.
static size_t moe_layout(int T, int topk, int E, int D, int F, size_t off[QG_WS_COUNT]) {
    const size_t P = (size_t)T * topk;
    const size_t Ucap = P < (size_t)E ? P : (size_t)E;
    const size_t sz[QG_WS_COUNT] = {
        4,                      // NUNIQ
        4 * Ucap,               // UNIQ
        4 * P,                  // SLOT
        4 * (Ucap + 1),         // PAIR_OFF
        4 * P,                  // PAIRS
        4 * P * F,              // G
        4 * P * F,              // V
        4 * P * F,              // H
        P * F,                  // HQ
        4 * P * (F / 32),       // HD
        4 * P * (F / 32),       // HS
        4 * P * D,              // O
        4 * (1 + 2 * (size_t)moe_mm_cap((int)P)),  // HOT
    };
    size_t at = 0;
    for (int i = 0; i < QG_WS_COUNT; ++i) {
        off[i] = at;
        at = align256(at + sz[i]);
    }
    return at;
}

// ---------------------------------------------------------------- 1. table

__device__ __forceinline__ bool bad_pointer(const void *p) { return p == nullptr || ((uintptr_t)p & 15) != 0; }

// Exclusive prefix sum over the 64 lanes of the wave; *total gets the sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int *total) {
    const int lane = lane_id();
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    *total = __shfl(incl, kWave - 1, kWave);
    return incl - v;
}

// One wave.  sid: the ids, staged once (every later pass reads LDS, so the
// pair loops wait for no global load); bm: bitmap of the selected usable
// experts; wpre[w]: number of set bits in words below w, so rank(e) =
// wpre[e/32] + popcount of the bits of word e/32 below e.
__global__ __launch_bounds__(kWave) void moe_table_kernel(const int32_t *__restrict__ ids, int P, int E,
                                                         const void *const *gate, const void *const *up,
                                                         const void *const *down, MoeWs ws, int32_t *status,
                                                         int mm_on) {
    __shared__ uint32_t bm[kTableWords];
    __shared__ int wpre[kTableWords];
    __shared__ int cur[QG_MAX_EXPERTS];  // pairs per distinct expert, then the next free position
    __shared__ int sid[QG_MAX_MOE_PAIRS];
    constexpr int kBatch = 8;  // independent global loads in flight per lane
    const int l = threadIdx.x;
    for (int w = l; w < kTableWords; w += kWave) bm[w] = 0u;
    for (int p0 = 0; p0 < P; p0 += kBatch * kWave) {
        int v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) v[i] = ids[min(p0 + i * kWave + l, P - 1)];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (p0 + i * kWave + l < P) sid[p0 + i * kWave + l] = v[i];
    }
    lds_barrier();
    bool bad_id = false;
    for (int p = l; p < P; p += kWave) {
        const int e = sid[p];
        if (e < 0 || e >= E)
            bad_id = true;
        else
            atomicOr(&bm[e >> 5], 1u << (e & 31));
    }
    lds_barrier();
    // experts with a NULL or misaligned matrix are dropped (checked per pair,
    // kBatch pairs per lane at a time, so the pointer loads overlap)
    bool bad_ptr = false;
    for (int p0 = 0; p0 < P; p0 += kBatch * kWave) {
        const void *pg[kBatch], *pu[kBatch], *pd[kBatch];
        int ev[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int p = p0 + i * kWave + l;
            const int e = p < P ? sid[p] : -1;
            ev[i] = e >= 0 && e < E ? e : -1;
            const int ec = ev[i] < 0 ? 0 : ev[i];
            pg[i] = gate[ec];
            pu[i] = up[ec];
            pd[i] = down[ec];
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int e = ev[i];
            if (e >= 0 && (bad_pointer(pg[i]) || bad_pointer(pu[i]) || bad_pointer(pd[i]))) {
                atomicAnd(&bm[e >> 5], ~(1u << (e & 31)));
                bad_ptr = true;
            }
        }
    }
    // the first error in pair order of the checks wins: an id outside the
    // range before an unusable expert
    const bool any_bad_id = __ballot(bad_id) != 0ull, any_bad_ptr = __ballot(bad_ptr) != 0ull;
    if (l == 0) *status = any_bad_id ? QG_DEV_BAD_EXPERT : (any_bad_ptr ? QG_DEV_NULL_EXPERT : QG_DEV_OK);
    lds_barrier();
    // ranks: each lane owns kTableWords / 64 consecutive words
    constexpr int WPL = kTableWords / kWave;
    int c = 0;
#pragma unroll
    for (int i = 0; i < WPL; ++i) c += __popc(bm[WPL * l + i]);
    int U;
    int run = wave_exclusive_scan(c, &U);
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
        const int w = WPL * l + i;
        wpre[w] = run;
        run += __popc(bm[w]);
    }
    if (l == 0) *ws.nuniq = U;
    for (int u = l; u < U; u += kWave) cur[u] = 0;
    lds_barrier();
    // the distinct ids in increasing order: one lane per id
    for (int e = l; e < E; e += kWave) {
        const uint32_t word = bm[e >> 5], bit = 1u << (e & 31);
        if (word & bit) ws.uniq[wpre[e >> 5] + __popc(word & (bit - 1u))] = e;
    }
    // each pair's slot (-1: invalid or dropped) replaces its id in sid
    for (int p = l; p < P; p += kWave) {
        const int e = sid[p];
        int s = -1;
        if (e >= 0 && e < E) {
            const uint32_t word = bm[e >> 5], bit = 1u << (e & 31);
            if (word & bit) s = wpre[e >> 5] + __popc(word & (bit - 1u));
        }
        sid[p] = s;
        ws.slot[p] = s;
        if (s >= 0) atomicAdd(&cur[s], 1);
    }
    lds_barrier();
    // CSR offsets: lane l scans experts [l*per, (l+1)*per)
    const int per = (U + kWave - 1) / kWave;
    const int lo = min(U, l * per), hi = min(U, lo + per);
    // (and the matrix-core work items: each 32-pair tile of an expert with
    // at least kMoeMm pairs, in slot order)
    int sum = 0, msum = 0;
    for (int u = lo; u < hi; ++u) {
        sum += cur[u];
        if (mm_on && cur[u] >= kMoeMm) msum += (cur[u] + 31) / 32;
    }
    int npairs, nmm;
    int at = wave_exclusive_scan(sum, &npairs);
    int mat = wave_exclusive_scan(msum, &nmm);
    for (int u = lo; u < hi; ++u) {
        const int n = cur[u];
        ws.pair_off[u] = at;
        cur[u] = at;
        at += n;
        if (mm_on && n >= kMoeMm)
            for (int m0 = 0; m0 < n; m0 += 32, ++mat) {
                ws.hot[1 + 2 * mat] = u;
                ws.hot[2 + 2 * mat] = m0;
            }
    }
    if (l == 0) {
        ws.pair_off[U] = npairs;
        ws.hot[0] = nmm;
    }
    lds_barrier();
    // stable fill, 64 pairs at a time: a pair's place among the chunk's pairs of
    // the same expert.  The lanes holding the same slot are found bit by bit
    // (one ballot per bit of a slot number, whatever the number of distinct
    // slots in the chunk): a lane keeps the lanes that agree with it on
    // every bit.
    const uint64_t below = (1ull << l) - 1ull;
    const int sbits = 32 - __clz(max(U - 1, 1));  // bits of the largest slot number
    for (int c0 = 0; c0 < P; c0 += kWave) {
        const int p = c0 + l;
        const int s = p < P ? sid[p] : -1;
        uint64_t m = __ballot(s >= 0);
        for (int b = 0; b < sbits; ++b) {
            const bool one = (s >> b) & 1;
            const uint64_t ones = __ballot(one);
            m &= one ? ones : ~ones;
        }
        const int before = __popcll(m & below), same = __popcll(m);
        if (s >= 0) ws.pairs[cur[s] + before] = p;
        lds_barrier();
        if (s >= 0 && before == 0) cur[s] += same;  // one lane per expert present in the chunk
        lds_barrier();
    }
}

// ---------------------------------------------------------------- 2./3. expert GEMVs

struct MoeArgs {
    const int8_t *qx;
    const float *dx;
    const int32_t *sx;
    int T, D, F, topk;
    const void *const *gate;
    const void *const *up;
    const void *const *down;
    MoeWs ws;
    TileGeom tg;  // of the projection this kernel runs
    int mt;       // tokens per LDS chunk
    int mm_on;    // experts with kMoeMm pairs or more are left to the matrix-core kernels
    // for the gate/up launch that builds the table of one token itself
    const int32_t *ids;
    int P, E;
    int32_t *status;
};

// ---------------------------------------------------------------- the table of one token

// One token with at most 64 pairs: the table in the registers of one wave,
// lane l holding pair l.  It has the table kernel's contents (the same
// slots, pair order and status), so the first expert launch can derive each
// workgroup's expert itself and write the table for the later launches.
struct TokenTable {
    int e;                 // id of this lane's pair
    bool in_range;         // 0 <= e < E (lanes past P: false)
    bool usable;           // and the expert's three matrices are usable
    uint64_t same;         // in-range lanes with the same id
    int rank;              // usable: the slot of the expert (distinct usable ids below it)
    int off;               // usable: the expert's first place in the pair list
    uint64_t first;        // wave-uniform: the first lane of each usable expert
    uintptr_t pg, pu, pd;  // the expert's gate, up and down matrices
};

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int j) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, j);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), j);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ TokenTable token_table(const int32_t *ids, int P, int E, const void *const *gate,
                                                  const void *const *up, const void *const *down) {
    TokenTable t;
    const int l = lane_id();
    t.e = as_global<int32_t>(ids)[min(l, P - 1)];
    t.in_range = l < P && t.e >= 0 && t.e < E;
    const int ec = t.in_range ? t.e : 0;
    t.pg = as_global<uintptr_t>(gate)[ec];
    t.pu = as_global<uintptr_t>(up)[ec];
    t.pd = as_global<uintptr_t>(down)[ec];
    // the in-range lanes with the same id and with a smaller one, bit by bit
    // from the top: a lane keeps the lanes that agree with it on the bits so
    // far (eq), and those that agree above bit b and hold 0 where it holds 1
    // are smaller (lt)
    const int ebits = 32 - __clz(max(E - 1, 1));
    uint64_t eq = __ballot(t.in_range), lt = 0;
    for (int b = ebits - 1; b >= 0; --b) {
        const bool one = (t.e >> b) & 1;
        const uint64_t ones = __ballot(one);
        if (one) lt |= eq & ~ones;
        eq &= one ? ones : ~ones;
    }
    t.same = eq;
    const auto unusable = [](uintptr_t q) { return q == 0 || (q & 15) != 0; };
    t.usable = t.in_range && !unusable(t.pg) && !unusable(t.pu) && !unusable(t.pd);
    t.first = __ballot(t.usable && (eq & ((1ull << l) - 1ull)) == 0);
    // slot: the usable experts with a smaller id; first place: their pairs
    // (an expert is usable for all of its pairs or none)
    t.rank = __popcll(lt & t.first);
    t.off = __popcll(lt & __ballot(t.usable));
    return t;
}

// The table and the status word, as the table kernel writes them (one wave).
__device__ __forceinline__ void write_token_table(const TokenTable &t, int P, const MoeWs &ws, int32_t *status) {
    const int l = lane_id();
    const uint64_t below = (1ull << l) - 1ull;
    const bool any_bad_id = __ballot(l < P && !t.in_range) != 0ull;
    const bool any_bad_ptr = __ballot(t.in_range && !t.usable) != 0ull;
    const int npairs = __popcll(__ballot(t.usable));
    const int U = __popcll(t.first);
    if (l < P) ws.slot[l] = t.usable ? t.rank : -1;
    if (t.usable) ws.pairs[t.off + __popcll(t.same & below)] = l;
    if ((t.first >> l) & 1) {
        ws.uniq[t.rank] = t.e;
        ws.pair_off[t.rank] = t.off;
    }
    if (l == 0) {
        *ws.nuniq = U;
        ws.pair_off[U] = npairs;
        ws.hot[0] = 0;
        *status = any_bad_id ? QG_DEV_BAD_EXPERT : (any_bad_ptr ? QG_DEV_NULL_EXPERT : QG_DEV_OK);
    }
}

// The gate/up launch of one token that builds the table itself: every wave
// derives it (token_table), workgroup (0, 0) writes it, and the workgroup
// takes the expert of slot u: its id, its pairs (bit p: pair p) and its gate
// or up matrix.  False past the last slot.
__device__ __forceinline__ bool token_slot(const MoeArgs &a, int u, bool is_up, int *e, uint64_t *pairs,
                                           const uint8_t **W) {
    const TokenTable t = token_table(a.ids, a.P, a.E, a.gate, a.up, a.down);
    if (blockIdx.x == 0 && u == 0 && threadIdx.x < kWave) write_token_table(t, a.P, a.ws, a.status);
    // the first lane of the expert in slot u, if there is one
    const uint64_t hit = __ballot(((t.first >> lane_id()) & 1) && t.rank == u);
    if (hit == 0ull) return false;
    const int j = __ffsll((unsigned long long)hit) - 1;
    *e = __builtin_amdgcn_readlane(t.e, j);
    *pairs = readlane64(t.same, j);
    *W = reinterpret_cast<const uint8_t *>(readlane64(is_up ? t.pu : t.pg, j));
    return true;
}

// Place of the n-th set bit of m (n < popcount(m)).
__device__ __forceinline__ int nth_bit(uint64_t m, int n) {
    for (int i = 0; i < n; ++i) m &= m - 1ull;
    return __ffsll((unsigned long long)m) - 1;
}

// Expert slot u of the table: its id, first pair and pair count; false when
// u is past the number of distinct experts.  The four values are read
// together and all of them decide the result, so none is deferred past it.
__device__ __forceinline__ bool moe_slot(const MoeWs &ws, int u, int *e, int *p0, int *cnt) {
    const int nu = load_uniform(ws.nuniq);
    const int id = load_uniform(ws.uniq + u);
    const int a = load_uniform(ws.pair_off + u), b = load_uniform(ws.pair_off + u + 1);
    *e = id;
    *p0 = a;
    *cnt = b - a;
    return u < nu && id >= 0 && b > a;
}

using QU = Unit<QG_FMT_Q4K, 8>;

// gate and up of expert uniq[blockIdx.y]: workgroups [0, nwg) take gate rows,
// [nwg, 2 nwg) up rows; the tokens are the expert's pairs' tokens.  ONE: the
// single-token engine, run once per pair.  RC: staging register chunks of
// the one-token form (act_reg_chunks of the activation's row).  OWN (one
// token, at most 64 pairs, no table kernel before): every wave derives the
// table from the ids (token_table) and workgroup (0, 0) writes it.
template <bool ONE, int RC, bool OWN>
__global__ __launch_bounds__(kMoeWaves *kWave) void moe_gate_up_kernel(MoeArgs a) {
    static_assert(ONE || !OWN, "the table is built in the kernel for one token only");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int u = blockIdx.y;
    const int ntiles = (a.F + a.tg.rpt - 1) / a.tg.rpt;
    const int nwg = (ntiles + kMoeWaves - 1) / kMoeWaves;
    const bool is_up = (int)blockIdx.x >= nwg;
    const int wg = is_up ? (int)blockIdx.x - nwg : (int)blockIdx.x;
    int e, p0 = 0, cnt;
    uint64_t own = 0;  // OWN: the expert's pairs, one bit each
    const uint8_t *W;
    if constexpr (OWN) {
        if (!token_slot(a, u, is_up, &e, &own, &W)) return;  // the whole workgroup leaves
        cnt = __popcll(own);
    } else {
        // the expert's entry is read with the count (blockIdx.y < Ucap keeps
        // it inside the table), all as scalars in one round trip; the slots
        // past the count leave
        if (!moe_slot(a.ws, u, &e, &p0, &cnt)) return;  // the whole workgroup leaves
        if (a.mm_on && cnt >= kMoeMm) return;  // the matrix-core kernels take this expert
        W = reinterpret_cast<const uint8_t *>(load_uniform(is_up ? a.up + e : a.gate + e));
    }
    float *dst = is_up ? a.ws.v : a.ws.g;
    const int32_t *pairs = a.ws.pairs + p0;
    const int topk = a.topk, F = a.F;
    ActSrc act{};
    act.qx = a.qx;
    act.dx = a.dx;
    act.sx = a.sx;
    if constexpr (ONE) {
        for (int m = 0; m < cnt; ++m) {
            if (m > 0) lds_barrier();  // the previous pair's staged activation is no longer read
            int p;
            if constexpr (OWN) {
                p = __ffsll((unsigned long long)own) - 1;  // the pairs in increasing order
                own &= own - 1ull;
            } else {
                p = load_uniform(pairs + m);
            }
            gemv_workgroup<QG_FMT_Q4K, 8, false, false, true, kSrcQ8, RC>(
                W, F, a.D, a.tg, wg * kMoeWaves, 1, ntiles, act, 1, a.mt, smem, [=](int) { return p / topk; },
                [=](int, int row, float v) { dst[(size_t)p * F + row] = v; }, [](int, int, int, const int32_t *) {});
        }
    } else if (cnt == 1) {
        // a one-pair expert of a batch: the one-token form, its token read once as a scalar
        const int p = load_uniform(pairs);
        gemv_workgroup<QG_FMT_Q4K, 8, false, false, true, kSrcQ8, RC>(
            W, F, a.D, a.tg, wg * kMoeWaves, 1, ntiles, act, 1, a.mt, smem, [=](int) { return p / topk; },
            [=](int, int row, float v) { dst[(size_t)p * F + row] = v; }, [](int, int, int, const int32_t *) {});
    } else {
        gemv_workgroup<QG_FMT_Q4K, 8, false, false, false, kSrcQ8>(
            W, F, a.D, a.tg, wg * kMoeWaves, 1, ntiles, act, cnt, a.mt, smem, [=](int m) { return pairs[m] / topk; },
            [=](int m, int row, float v) { dst[(size_t)pairs[m] * F + row] = v; },
            [](int, int, int, const int32_t *) {});
    }
}

// down of expert uniq[blockIdx.y] against the Q8 form of h = silu(g) * v of
// each of its pairs.  ONE: h is computed and quantized while it is staged
// (workgroup 0 of the expert stores h, hq, hd, hs of its pairs), once per
// pair; otherwise moe_h_quant_kernel has stored hq/hd/hs before.
template <bool ONE, int RC>
__global__ __launch_bounds__(kMoeWaves *kWave) void moe_down_kernel(MoeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int u = blockIdx.y;
    // the expert's entry is read with the count (blockIdx.y < Ucap keeps it
    // inside the table), all as scalars in one round trip; the slots past the
    // count leave
    int e, p0, cnt;
    if (!moe_slot(a.ws, u, &e, &p0, &cnt)) return;  // the whole workgroup leaves
    if (a.mm_on && cnt >= kMoeMm) return;  // the matrix-core kernels take this expert
    const int ntiles = (a.D + a.tg.rpt - 1) / a.tg.rpt;
    const uint8_t *W = reinterpret_cast<const uint8_t *>(load_uniform(a.down + e));
    const int32_t *pairs = a.ws.pairs + p0;
    float *o = a.ws.o;
    const int D = a.D;
    ActSrc act{};
    act.x = a.ws.g;
    act.x2 = a.ws.v;
    act.ph = a.ws.h;
    act.pqx = a.ws.hq;
    act.pdx = a.ws.hd;
    act.psx = a.ws.hs;
    if constexpr (ONE) {
        for (int m = 0; m < cnt; ++m) {
            if (m > 0) lds_barrier();
            const int p = load_uniform(pairs + m);
            gemv_workgroup<QG_FMT_Q4K, 8, false, false, true, kSrcGLU, RC>(
                W, D, a.F, a.tg, (int)blockIdx.x * kMoeWaves, 1, ntiles, act, 1, a.mt, smem, [=](int) { return p; },
                [=](int, int row, float v) { o[(size_t)p * D + row] = v; }, [](int, int, int, const int32_t *) {});
        }
    } else {
        ActSrc hq{};
        hq.qx = a.ws.hq;
        hq.dx = a.ws.hd;
        hq.sx = a.ws.hs;
        if (cnt == 1) {
            const int p = load_uniform(pairs);
            gemv_workgroup<QG_FMT_Q4K, 8, false, false, true, kSrcQ8, RC>(
                W, D, a.F, a.tg, (int)blockIdx.x * kMoeWaves, 1, ntiles, hq, 1, a.mt, smem, [=](int) { return p; },
                [=](int, int row, float v) { o[(size_t)p * D + row] = v; }, [](int, int, int, const int32_t *) {});
            return;
        }
        gemv_workgroup<QG_FMT_Q4K, 8, false, false, false, kSrcQ8>(
            W, D, a.F, a.tg, (int)blockIdx.x * kMoeWaves, 1, ntiles, hq, cnt, a.mt, smem,
            [=](int m) { return pairs[m]; }, [=](int m, int row, float v) { o[(size_t)pairs[m] * D + row] = v; },
            [](int, int, int, const int32_t *) {});
    }
}

// Experts with kMoeMm pairs or more on the matrix cores: work item
// blockIdx.y is one 32-pair tile of one such expert (the table lists them);
// workgroup x takes a 32-row tile of gate (x < ntF) or up.  Same results, bit
// for bit, as the dot-product kernels.
template <int GPS>
__global__ __launch_bounds__(kMmMaxSlices *kWave) void moe_mm_gate_up_kernel(MoeArgs a, int ks) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int item = blockIdx.y;
    if (item >= load_uniform(a.ws.hot)) return;  // the whole workgroup leaves
    const int u = load_uniform(a.ws.hot + 1 + 2 * item);
    const int e = load_uniform(a.ws.uniq + u);
    const int p0 = load_uniform(a.ws.pair_off + u);
    const int ntF = (a.F + kMmRows - 1) / kMmRows;
    const bool is_up = (int)blockIdx.x >= ntF;
    MmTile t;
    t.W = reinterpret_cast<const uint8_t *>(load_uniform(is_up ? a.up + e : a.gate + e));
    t.N = a.F;
    t.row0 = ((int)blockIdx.x - (is_up ? ntF : 0)) * kMmRows;
    t.m0 = load_uniform(a.ws.hot + 2 + 2 * item);
    t.M = load_uniform(a.ws.pair_off + u + 1) - p0;
    t.qx = a.qx;
    t.dx = a.dx;
    t.sx = a.sx;
    t.K = a.D;
    t.row_bytes = a.D / 256 * 144;
    t.groups = a.D / 256;
    t.gps = GPS;
    t.KS = ks;
    const int32_t *pairs = a.ws.pairs + p0;
    float *dst = is_up ? a.ws.v : a.ws.g;
    const int topk = a.topk, F = a.F;
    mm_tile<QG_FMT_Q4K, 8, GPS, 1>(
        t, [=](int m) { return pairs[m] / topk; }, [=](int m, int row, float v) { dst[(size_t)pairs[m] * F + row] = v; },
        smem);
}

// down of the matrix-core experts against each pair's Q8 h
template <int GPS>
__global__ __launch_bounds__(kMmMaxSlices *kWave) void moe_mm_down_kernel(MoeArgs a, int ks) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int item = blockIdx.y;
    if (item >= load_uniform(a.ws.hot)) return;
    const int u = load_uniform(a.ws.hot + 1 + 2 * item);
    const int e = load_uniform(a.ws.uniq + u);
    const int p0 = load_uniform(a.ws.pair_off + u);
    MmTile t;
    t.W = reinterpret_cast<const uint8_t *>(load_uniform(a.down + e));
    t.N = a.D;
    t.row0 = (int)blockIdx.x * kMmRows;
    t.m0 = load_uniform(a.ws.hot + 2 + 2 * item);
    t.M = load_uniform(a.ws.pair_off + u + 1) - p0;
    t.qx = a.ws.hq;
    t.dx = a.ws.hd;
    t.sx = a.ws.hs;
    t.K = a.F;
    t.row_bytes = a.F / 256 * 144;
    t.groups = a.F / 256;
    t.gps = GPS;
    t.KS = ks;
    const int32_t *pairs = a.ws.pairs + p0;
    float *o = a.ws.o;
    const int D = a.D;
    mm_tile<QG_FMT_Q4K, 8, GPS, 1>(
        t, [=](int m) { return pairs[m]; }, [=](int m, int row, float v) { o[(size_t)pairs[m] * D + row] = v; },
        smem);
}

// Block-scaled expert formats (FP8 E4M3 128 x 128, FP4 E2M1 1 x 32): gate and
// up of expert uniq[blockIdx.y] on the mx engine, workgroups [0, nwg) on gate
// rows and [nwg, 2 nwg) on up rows, the tokens being the expert's pairs'.
template <int FMT, int CPL, bool OWN>
__global__ __launch_bounds__(mx_routed_waves(FMT) * kWave) void moe_gate_up_mx_kernel(MoeArgs a, int nwg) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int R = mx_rows_per_wave(kMxLoadsRouted, CPL);
    const int u = blockIdx.y;
    const bool is_up = (int)blockIdx.x >= nwg;
    const int wg = is_up ? (int)blockIdx.x - nwg : (int)blockIdx.x;
    int e, p0 = 0, cnt;
    uint64_t own = 0;  // OWN (one token, the table built here): the expert's pairs, one bit each
    const uint8_t *W;
    if constexpr (OWN) {
        if (!token_slot(a, u, is_up, &e, &own, &W)) return;  // the whole workgroup leaves
        cnt = __popcll(own);
    } else {
        // the expert's entry is read with the count (blockIdx.y < Ucap keeps
        // it inside the table), all as scalars in one round trip; the slots
        // past the count leave
        if (!moe_slot(a.ws, u, &e, &p0, &cnt)) return;  // the whole workgroup leaves
        W = reinterpret_cast<const uint8_t *>(load_uniform(is_up ? a.up + e : a.gate + e));
    }
    float *dst = is_up ? a.ws.v : a.ws.g;
    const int32_t *pairs = a.ws.pairs + p0;
    const int topk = a.topk, F = a.F;
    if constexpr (OWN) {
        // one token: every pair's token is 0
        mx_workgroup<FMT, CPL, kMxLoadsRouted, mx_routed_waves(FMT)>(
            W, F, a.D, wg * mx_routed_waves(FMT) * R, cnt, a.mt, a.qx, a.dx, [](int) { return 0; },
            [=](int m, int row, float v) { dst[(size_t)nth_bit(own, m) * F + row] = v; }, smem);
        return;
    }
    if (cnt == 1) {
        // one pair (the usual case in decode): its token is read once, as a
        // scalar, so no vector load has to return before the weights are requested
        const int p = load_uniform(pairs), tok = p / topk;
        mx_workgroup<FMT, CPL, kMxLoadsRouted, mx_routed_waves(FMT)>(
            W, F, a.D, wg * mx_routed_waves(FMT) * R, 1, a.mt, a.qx, a.dx, [=](int) { return tok; },
            [=](int, int row, float v) { dst[(size_t)p * F + row] = v; }, smem);
        return;
    }
    mx_workgroup<FMT, CPL, kMxLoadsRouted, mx_routed_waves(FMT)>(
        W, F, a.D, wg * mx_routed_waves(FMT) * R, cnt, a.mt, a.qx, a.dx, [=](int m) { return pairs[m] / topk; },
        [=](int m, int row, float v) { dst[(size_t)pairs[m] * F + row] = v; }, smem);
}

// down of expert uniq[blockIdx.y] on the mx engine against each pair's Q8 h.
template <int FMT, int CPL, bool GLU>
__global__ __launch_bounds__(mx_routed_waves(FMT) * kWave) void moe_down_mx_kernel(MoeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int R = mx_rows_per_wave(kMxLoadsRouted, CPL);
    constexpr int NW = mx_routed_waves(FMT);
    const int u = blockIdx.y;
    // the expert's entry is read with the count (blockIdx.y < Ucap keeps it
    // inside the table), all as scalars in one round trip; the slots past the
    // count leave
    int e, p0, cnt;
    if (!moe_slot(a.ws, u, &e, &p0, &cnt)) return;  // the whole workgroup leaves
    const uint8_t *W = reinterpret_cast<const uint8_t *>(load_uniform(a.down + e));
    const int32_t *pairs = a.ws.pairs + p0;
    float *o = a.ws.o;
    const int D = a.D, F = a.F;
    const int row_base = (int)blockIdx.x * NW * R;
    if constexpr (GLU) {
        // one token: h of each pair formed and quantized while it is staged
        // (the first row block's workgroup stores h, hq, hd, hs), pair by pair
        for (int m = 0; m < cnt; ++m) {
            if (m > 0) lds_barrier();  // the previous pair's staged h is no longer read
            const int p = load_uniform(pairs + m);
            MxGlu glu{a.ws.g + (size_t)p * F, a.ws.v + (size_t)p * F, nullptr, nullptr, nullptr, nullptr};
            if (blockIdx.x == 0) {
                glu.ph = a.ws.h + (size_t)p * F;
                glu.pqx = a.ws.hq + (size_t)p * F;
                glu.pdx = a.ws.hd + (size_t)p * (F / 32);
                glu.psx = a.ws.hs + (size_t)p * (F / 32);
            }
            mx_workgroup<FMT, CPL, kMxLoadsRouted, NW, true>(
                W, D, F, row_base, 1, 1, nullptr, nullptr, [](int) { return 0; },
                [=](int, int row, float v) { o[(size_t)p * D + row] = v; }, smem, glu);
        }
        return;
    }
    if (cnt == 1) {
        const int p = load_uniform(pairs);
        mx_workgroup<FMT, CPL, kMxLoadsRouted, NW>(
            W, D, F, row_base, 1, a.mt, a.ws.hq, a.ws.hd, [=](int) { return p; },
            [=](int, int row, float v) { o[(size_t)p * D + row] = v; }, smem);
        return;
    }
    mx_workgroup<FMT, CPL, kMxLoadsRouted, NW>(
        W, D, F, row_base, cnt, a.mt, a.ws.hq, a.ws.hd, [=](int m) { return pairs[m]; },
        [=](int m, int row, float v) { o[(size_t)pairs[m] * D + row] = v; }, smem);
}

// h = silu(g) * v and its Q8 form for every valid pair, before the down
// projection of more than one token: 8 lanes per 32-block, the quantizer of
// the activation staging (so the records match the single-token form).
__global__ __launch_bounds__(256) void moe_h_quant_kernel(MoeWs ws, int P, int F) {
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int nblk = P * (F / 32);
    const int blk = gid >> 3, part = gid & 7;
    const int p = blk / (F / 32);
    const bool live = blk < nblk && ws.slot[p] >= 0;  // uniform over the 8 lanes of a block
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    const size_t base = (size_t)blk * 32 + part * 4;
    if (live) {
        const float4 g = *reinterpret_cast<const float4 *>(ws.g + base);
        const float4 v = *reinterpret_cast<const float4 *>(ws.v + base);
        h[0] = silu(g.x) * v.x;
        h[1] = silu(g.y) * v.y;
        h[2] = silu(g.z) * v.z;
        h[3] = silu(g.w) * v.w;
    }
    int8_t q[4];
    float d;
    int32_t s;
    quantize_block_8lanes(h, q, &d, &s);
    if (live) {
        *reinterpret_cast<float4 *>(ws.h + base) = make_float4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint32_t *>(ws.hq + base) = (uint32_t)(uint8_t)q[0] | ((uint32_t)(uint8_t)q[1] << 8) |
                                                     ((uint32_t)(uint8_t)q[2] << 16) |
                                                     ((uint32_t)(uint8_t)q[3] << 24);
        if (part == 0) {
            ws.hd[blk] = d;
            ws.hs[blk] = s;
        }
    }
}

// ---------------------------------------------------------------- 4. combine

// V consecutive outputs per thread (1, 2 or 4; D % 4 == 0): fewer per
// thread spread a small batch's loads over more CUs.
template <int V>
struct CombineVec;
template <>
struct CombineVec<1> {
    typedef float type;
};
template <>
struct CombineVec<2> {
    typedef float2 type;
};
template <>
struct CombineVec<4> {
    typedef float4 type;
};

template <int V>
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeWs ws, const float *__restrict__ rw, int T, int D,
                                                          int topk, float *__restrict__ y) {
    typedef typename CombineVec<V>::type vec;
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int per_t = D / V;
    if (gid >= T * per_t) return;
    const int t = gid / per_t, n = gid - t * per_t;
    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.0f;
    // eight pairs at a time: every load is issued before the first use (a
    // load behind a branch on the slot would wait twice per pair); pairs past
    // topk re-read the last one and are not used
    constexpr int kU = 8;
    for (int k0 = 0; k0 < topk; k0 += kU) {
        int sl[kU];
        float r[kU];
        vec o[kU];
#pragma unroll
        for (int j = 0; j < kU; ++j) {
            const int p = t * topk + min(k0 + j, topk - 1);
            sl[j] = ws.slot[p];
            r[j] = rw[p];
            o[j] = *reinterpret_cast<const vec *>(ws.o + (size_t)p * D + V * n);
        }
#pragma unroll
        for (int j = 0; j < kU; ++j) {
            // an invalid id or unusable expert (slot -1) contributes nothing
            if (k0 + j < topk && sl[j] >= 0) {
                const float *oj = reinterpret_cast<const float *>(&o[j]);
#pragma unroll
                for (int e = 0; e < V; ++e) acc[e] = fmaf_exact(r[j], oj[e], acc[e]);
            }
        }
    }
    *reinterpret_cast<vec *>(y + (size_t)t * D + V * n) = *reinterpret_cast<const vec *>(acc);
}

// The combine launch: one output per thread while the batch's outputs fill
// fewer than 64 workgroups of 256 threads that way, else four.
static int launch_combine(const MoeWs &w, const float *rw, int T, int D, int topk, float *y, hipStream_t st) {
    const long long n1 = (long long)T * D;
    if (n1 < 64LL * 256) {
        hipLaunchKernelGGL(moe_combine_kernel<1>, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, st, w, rw, T, D,
                           topk, y);
    } else {
        const long long n4 = n1 / 4;
        hipLaunchKernelGGL(moe_combine_kernel<4>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, w, rw, T, D,
                           topk, y);
    }
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

static MoeWs ws_pointers(void *ws, const size_t off[QG_WS_COUNT]) {
    uint8_t *b = reinterpret_cast<uint8_t *>(ws);
    MoeWs w;
    w.nuniq = reinterpret_cast<int32_t *>(b + off[QG_WS_NUNIQ]);
    w.uniq = reinterpret_cast<int32_t *>(b + off[QG_WS_UNIQ]);
    w.slot = reinterpret_cast<int32_t *>(b + off[QG_WS_SLOT]);
    w.pair_off = reinterpret_cast<int32_t *>(b + off[QG_WS_PAIR_OFF]);
    w.pairs = reinterpret_cast<int32_t *>(b + off[QG_WS_PAIRS]);
    w.g = reinterpret_cast<float *>(b + off[QG_WS_G]);
    w.v = reinterpret_cast<float *>(b + off[QG_WS_V]);
    w.h = reinterpret_cast<float *>(b + off[QG_WS_H]);
    w.hq = reinterpret_cast<int8_t *>(b + off[QG_WS_HQ]);
    w.hd = reinterpret_cast<float *>(b + off[QG_WS_HD]);
    w.hs = reinterpret_cast<int32_t *>(b + off[QG_WS_HS]);
    w.o = reinterpret_cast<float *>(b + off[QG_WS_O]);
    w.hot = reinterpret_cast<int32_t *>(b + off[QG_WS_HOT]);
    return w;
}

template <class Kern>
static bool raise_lds_limit(Kern *k, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes) == hipSuccess;
}

// Every block-scaled expert kernel of format FMT (all chunk counts, both
// table and h forms).
template <int FMT, int CPL>
static bool raise_mx_cpl() {
    return raise_lds_limit(moe_gate_up_mx_kernel<FMT, CPL, false>, kMxLdsMax) &&
           raise_lds_limit(moe_gate_up_mx_kernel<FMT, CPL, true>, kMxLdsMax) &&
           raise_lds_limit(moe_down_mx_kernel<FMT, CPL, false>, kMxLdsMax) &&
           raise_lds_limit(moe_down_mx_kernel<FMT, CPL, true>, kMxLdsMax);
}
template <int FMT>
static bool raise_mx_all() {
    return raise_mx_cpl<FMT, 1>() && raise_mx_cpl<FMT, 2>() && raise_mx_cpl<FMT, 4>() && raise_mx_cpl<FMT, 8>() &&
           raise_mx_cpl<FMT, 16>();
}

// gate/up (K = D, F rows each) and down (K = F, D rows) on the mx engine.
template <int FMT, int CPL, bool OWN>
static int launch_moe_gate_up_mx_own(MoeArgs a, int Ucap, hipStream_t st) {
    const int rows_per_wg = mx_routed_waves(FMT) * mx_rows_per_wave(kMxLoadsRouted, CPL);
    const int nwg = (a.F + rows_per_wg - 1) / rows_per_wg;
    a.mt = mx_tokens_per_chunk(a.D, QG_MAX_MOE_PAIRS);
    hipLaunchKernelGGL((moe_gate_up_mx_kernel<FMT, CPL, OWN>), dim3(2 * nwg, Ucap),
                       dim3(mx_routed_waves(FMT) * kWave),
                       (size_t)a.mt * mx_token_rec(a.D) +
                           mx_scale_lds<FMT>(a.D, CPL, kMxLoadsRouted, mx_routed_waves(FMT)),
                       st, a, nwg);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

// own: one token, the table built in this launch (no table kernel before)
template <int FMT, int CPL>
static int launch_moe_gate_up_mx(const MoeArgs &a, int Ucap, bool own, hipStream_t st) {
    return own ? launch_moe_gate_up_mx_own<FMT, CPL, true>(a, Ucap, st)
               : launch_moe_gate_up_mx_own<FMT, CPL, false>(a, Ucap, st);
}

template <int FMT, int CPL, bool GLU>
static int launch_moe_down_mx_glu(MoeArgs a, int Ucap, hipStream_t st) {
    const int rows_per_wg = mx_routed_waves(FMT) * mx_rows_per_wave(kMxLoadsRouted, CPL);
    const int nwg = (a.D + rows_per_wg - 1) / rows_per_wg;
    a.mt = mx_tokens_per_chunk(a.F, QG_MAX_MOE_PAIRS);
    hipLaunchKernelGGL((moe_down_mx_kernel<FMT, CPL, GLU>), dim3(nwg, Ucap),
                       dim3(mx_routed_waves(FMT) * kWave),
                       (size_t)a.mt * mx_token_rec(a.F) +
                           mx_scale_lds<FMT>(a.F, CPL, kMxLoadsRouted, mx_routed_waves(FMT)),
                       st, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

// glu: one token, h formed while the down projection stages it (no h launch)
template <int FMT, int CPL>
static int launch_moe_down_mx(const MoeArgs &a, int Ucap, bool glu, hipStream_t st) {
    return glu ? launch_moe_down_mx_glu<FMT, CPL, true>(a, Ucap, st) : launch_moe_down_mx_glu<FMT, CPL, false>(a, Ucap, st);
}

template <int FMT>
// own: the gate/up launch builds the table; glu: the down launch forms h
// itself (both for one token only)
static int launch_moe_mx(const MoeArgs &a, int Ucap, bool down, bool own, bool glu, hipStream_t st) {
    switch (mx_chunks_per_lane<FMT>(down ? a.F : a.D)) {
        case 1:
            return down ? launch_moe_down_mx<FMT, 1>(a, Ucap, glu, st)
                        : launch_moe_gate_up_mx<FMT, 1>(a, Ucap, own, st);
        case 2:
            return down ? launch_moe_down_mx<FMT, 2>(a, Ucap, glu, st)
                        : launch_moe_gate_up_mx<FMT, 2>(a, Ucap, own, st);
        case 4:
            return down ? launch_moe_down_mx<FMT, 4>(a, Ucap, glu, st)
                        : launch_moe_gate_up_mx<FMT, 4>(a, Ucap, own, st);
        case 8:
            return down ? launch_moe_down_mx<FMT, 8>(a, Ucap, glu, st)
                        : launch_moe_gate_up_mx<FMT, 8>(a, Ucap, own, st);
        case 16:
            return down ? launch_moe_down_mx<FMT, 16>(a, Ucap, glu, st)
                        : launch_moe_gate_up_mx<FMT, 16>(a, Ucap, own, st);
        default: return QG_ERR_SHAPE;
    }
}

}  // namespace qg

namespace qg {

// The matrix-core expert kernels over `cap` possible work items; K = the
// projection's input width, tiles = 32-row tiles per item.
template <bool DOWN, int GPS>
static int launch_moe_mm_gps(const MoeArgs &a, int tiles, int cap, int ks, hipStream_t st) {
    auto kern = DOWN ? moe_mm_down_kernel<GPS> : moe_mm_gate_up_kernel<GPS>;
    hipLaunchKernelGGL(kern, dim3(tiles, cap), dim3(ks * kWave), (size_t)ks * mm_wave_lds<QG_FMT_Q4K>(GPS), st, a, ks);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

template <bool DOWN>
static int launch_moe_mm(const MoeArgs &a, int P, hipStream_t st) {
    const int K = DOWN ? a.F : a.D, N = DOWN ? a.D : a.F;
    const int tiles = (DOWN ? 1 : 2) * ((N + kMmRows - 1) / kMmRows);
    const int cap = moe_mm_cap(P);
    // the most slices: few of the cap work items are real (the popular
    // experts of a batch), so each wave should take few groups
    int ks, gps;
    mm_slices(K / 256, 1, &ks, &gps);
    switch (gps) {
        case 1: return launch_moe_mm_gps<DOWN, 1>(a, tiles, cap, ks, st);
        case 2: return launch_moe_mm_gps<DOWN, 2>(a, tiles, cap, ks, st);
        case 4: return launch_moe_mm_gps<DOWN, 4>(a, tiles, cap, ks, st);
        case 8: return launch_moe_mm_gps<DOWN, 8>(a, tiles, cap, ks, st);
        default: return QG_ERR_SHAPE;
    }
}

template <int RC>
bool raise_moe_lds() {
    return raise_lds_limit(moe_gate_up_kernel<false, RC, false>, kLdsBytes) &&
           raise_lds_limit(moe_gate_up_kernel<true, RC, false>, kLdsBytes) &&
           raise_lds_limit(moe_gate_up_kernel<true, RC, true>, kLdsBytes) &&
           raise_lds_limit(moe_down_kernel<false, RC>, kLdsBytes) && raise_lds_limit(moe_down_kernel<true, RC>, kLdsBytes);
}

template <int GPS>
bool raise_moe_mm() {
    return raise_lds_limit(moe_mm_gate_up_kernel<GPS>, kMmMaxSlices * mm_wave_lds<QG_FMT_Q4K>(GPS)) &&
           raise_lds_limit(moe_mm_down_kernel<GPS>, kMmMaxSlices * mm_wave_lds<QG_FMT_Q4K>(GPS));
}

// Raise the dynamic-LDS limit of every expert kernel of one format on the
// current device (run once per device and format by once_per_device, before
// a call enqueues anything).
static int moe_kernels_init(const void *, int fmt) {
    bool ok;
    if (fmt == QG_FMT_Q4K)
        ok = raise_moe_lds<1>() && raise_moe_lds<2>() && raise_moe_lds<kActRegChunks>() && raise_moe_mm<1>() &&
             raise_moe_mm<2>() && raise_moe_mm<4>() && raise_moe_mm<8>();
    else if (fmt == QG_FMT_FP8_E4M3_B128)
        ok = raise_mx_all<QG_FMT_FP8_E4M3_B128>();
    else
        ok = raise_mx_all<QG_FMT_FP4_E2M1_MX>();
    return ok ? QG_OK : QG_ERR_LAUNCH;
}
static const char g_moe_init_key[4] = {0, 0, 0, 0};  // one key per format (its address)

template <bool DOWN, bool ONE, int RC, bool OWN>
void launch_moe_dot_rc(dim3 grid, size_t lds, hipStream_t st, const MoeArgs &a) {
    if constexpr (DOWN)
        hipLaunchKernelGGL((moe_down_kernel<ONE, RC>), grid, dim3(kMoeWaves * kWave), lds, st, a);
    else
        hipLaunchKernelGGL((moe_gate_up_kernel<ONE, RC, OWN>), grid, dim3(kMoeWaves * kWave), lds, st, a);
}

// The dot-product expert kernel of gate/up or down, in its one-token or
// several-token form, with rc staging register chunks (1, 2 or 4); own: the
// one-token gate/up launch that builds the table itself.
template <bool DOWN, bool OWN>
void launch_moe_dot_own(bool one, int rc, dim3 grid, size_t lds, hipStream_t st, const MoeArgs &a) {
    if (one) {
        if (rc == 1) return launch_moe_dot_rc<DOWN, true, 1, OWN>(grid, lds, st, a);
        if (rc == 2) return launch_moe_dot_rc<DOWN, true, 2, OWN>(grid, lds, st, a);
        return launch_moe_dot_rc<DOWN, true, kActRegChunks, OWN>(grid, lds, st, a);
    }
    if constexpr (!OWN) {
        if (rc == 1) return launch_moe_dot_rc<DOWN, false, 1, false>(grid, lds, st, a);
        if (rc == 2) return launch_moe_dot_rc<DOWN, false, 2, false>(grid, lds, st, a);
        return launch_moe_dot_rc<DOWN, false, kActRegChunks, false>(grid, lds, st, a);
    }
}

template <bool DOWN>
void launch_moe_dot(bool one, bool own, int rc, dim3 grid, size_t lds, hipStream_t st, const MoeArgs &a) {
    if (own && !DOWN && one) return launch_moe_dot_own<false, true>(true, rc, grid, lds, st, a);
    return launch_moe_dot_own<DOWN, false>(one, rc, grid, lds, st, a);
}

}  // namespace qg

extern "C" size_t moe_routed_workspace_bytes(int T, int topk, int E, int D, int F) {
    if (!qg::moe_shape_ok(T, topk, E, D, F)) return 0;
    size_t off[QG_WS_COUNT];
    return qg::moe_layout(T, topk, E, D, F, off);
}

extern "C" int moe_routed_workspace_layout(int T, int topk, int E, int D, int F, size_t *offsets) {
    if (!offsets) return QG_ERR_NULL;
    if (!qg::moe_shape_ok(T, topk, E, D, F)) return QG_ERR_SHAPE;
    qg::moe_layout(T, topk, E, D, F, offsets);
    return QG_OK;
}

extern "C" int moe_routed_qgemv_fmt(int fmt, const int8_t *qx, const float *dx, const int32_t *sx, int T, int D,
                                    int F, int E, int topk, const int32_t *ids, const float *rw,
                                    const void *const *gate, const void *const *up, const void *const *down,
                                    float *y, void *ws, size_t ws_bytes, int32_t *d_status, void *stream) {
    using namespace qg;
    if (fmt != QG_FMT_Q4K && fmt != QG_FMT_FP8_E4M3_B128 && fmt != QG_FMT_FP4_E2M1_MX) return QG_ERR_FORMAT;
    if (!qx || !dx || !sx || !ids || !rw || !gate || !up || !down || !y || !ws || !d_status) return QG_ERR_NULL;
    if (!moe_shape_ok(T, topk, E, D, F)) return QG_ERR_SHAPE;
    size_t off[QG_WS_COUNT];
    const size_t need = moe_layout(T, topk, E, D, F, off);
    if (ws_bytes < need) return QG_ERR_WORKSPACE;
    const uintptr_t a16 = (uintptr_t)qx | (uintptr_t)dx | (uintptr_t)sx | (uintptr_t)y | (uintptr_t)ws;
    const uintptr_t a8 = (uintptr_t)gate | (uintptr_t)up | (uintptr_t)down;
    if ((a16 & 15) || (a8 & 7) || ((uintptr_t)ids & 3) || ((uintptr_t)rw & 3) || ((uintptr_t)d_status & 3))
        return QG_ERR_ALIGN;
    clear_stale_error();
    // every kernel this call may use gets its LDS limit before the first launch
    if (once_per_device(&g_moe_init_key[fmt], moe_kernels_init, fmt) != QG_OK) return QG_ERR_LAUNCH;
    hipStream_t st = (hipStream_t)stream;
    const int P = T * topk;
    const int Ucap = P < E ? P : E;
    MoeWs w = ws_pointers(ws, off);

    // Q4_K experts with many pairs go to the matrix cores (possible from kMoeMm tokens on)
    const int mm_on = fmt == QG_FMT_Q4K && T >= kMoeMm;
    // one token with at most 64 pairs: the gate/up launch builds the table
    // itself; otherwise the table kernel runs first.  (Batches with few
    // pairs measured slower so: each of their many workgroup rounds pays the
    // ids-then-pointers chain, T = 8: 123.8 -> 130.0 us.)
    const bool own_table = T == 1 && P <= kWave;
    if (!own_table) {
        hipLaunchKernelGGL(moe_table_kernel, dim3(1), dim3(kWave), 0, st, ids, P, E, gate, up, down, w, d_status,
                           mm_on);
        if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;
    }

    MoeArgs a{};
    a.qx = qx;
    a.dx = dx;
    a.sx = sx;
    a.T = T;
    a.D = D;
    a.F = F;
    a.topk = topk;
    a.gate = gate;
    a.up = up;
    a.down = down;
    a.ws = w;
    a.mm_on = mm_on;
    a.ids = ids;
    a.P = P;
    a.E = E;
    a.status = d_status;
    if (fmt != QG_FMT_Q4K) {
        // block-scaled experts: gate/up, h quantized once per pair (for one
        // token with FP4 experts while the down projection stages it, else its
        // own launch), down, combine.  (FP8's 8-wave down workgroups would
        // lose half their occupancy to the staging's registers: measured
        // slower, 40.4 -> 41.6 us; FP4 33.3 -> 32.7.)
        const bool glu = T == 1 && fmt == QG_FMT_FP4_E2M1_MX;
        int rc = fmt == QG_FMT_FP8_E4M3_B128
                     ? launch_moe_mx<QG_FMT_FP8_E4M3_B128>(a, Ucap, false, own_table, false, st)
                     : launch_moe_mx<QG_FMT_FP4_E2M1_MX>(a, Ucap, false, own_table, false, st);
        if (rc) return rc;
        if (!glu) {
            const long long hthreads = (long long)P * (F / 32) * 8;
            hipLaunchKernelGGL(moe_h_quant_kernel, dim3((unsigned)((hthreads + 255) / 256)), dim3(256), 0, st, w, P,
                               F);
            if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;
        }
        rc = fmt == QG_FMT_FP8_E4M3_B128 ? launch_moe_mx<QG_FMT_FP8_E4M3_B128>(a, Ucap, true, false, glu, st)
                                         : launch_moe_mx<QG_FMT_FP4_E2M1_MX>(a, Ucap, true, false, glu, st);
        if (rc) return rc;
        return launch_combine(w, rw, T, D, topk, y, st);
    }
    const bool one = T == 1;  // every expert then has a single pair (a few if the token repeats an id)
    constexpr int threads = kMoeWaves * kWave;

    // gate/up: K = D, Q8 activation of the tokens
    a.tg = make_tile_geom<QU>(D);
    a.mt = one ? 1 : min(kMoeChunk, tokens_per_chunk<QU>(D, QG_MAX_MOE_PAIRS, threads));
    size_t lds = gemv_lds_bytes<QU>(kMoeWaves, D, a.mt);
    int nwg = ((F + a.tg.rpt - 1) / a.tg.rpt + kMoeWaves - 1) / kMoeWaves;
    launch_moe_dot<false>(one, own_table, act_reg_chunks(D / 16, threads), dim3(2 * nwg, Ucap), lds, st, a);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;
    if (mm_on) {
        const int rc = launch_moe_mm<false>(a, P, st);
        if (rc) return rc;
    }

    // down: K = F.  One token: h = silu(g) * v staged from fp32 and quantized
    // there; several: h quantized once per pair first (each expert's
    // workgroups would otherwise all redo it for every pair)
    if (!one) {
        const long long hthreads = (long long)P * (F / 32) * 8;
        hipLaunchKernelGGL(moe_h_quant_kernel, dim3((unsigned)((hthreads + 255) / 256)), dim3(256), 0, st, w, P, F);
        if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;
    }
    a.tg = make_tile_geom<QU>(F);
    a.mt = one ? 1 : min(kMoeChunk, tokens_per_chunk<QU>(F, QG_MAX_MOE_PAIRS, threads));
    lds = gemv_lds_bytes<QU>(kMoeWaves, F, a.mt);
    nwg = ((D + a.tg.rpt - 1) / a.tg.rpt + kMoeWaves - 1) / kMoeWaves;
    // (one token: h staged from fp32, 4 values per chunk; else the Q8 h of a
    // one-pair expert, 16 per chunk)
    launch_moe_dot<true>(one, false, act_reg_chunks(one ? F / 4 : F / 16, threads), dim3(nwg, Ucap), lds, st, a);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;
    if (mm_on) {
        const int rc = launch_moe_mm<true>(a, P, st);
        if (rc) return rc;
    }

    return launch_combine(w, rw, T, D, topk, y, st);
}

extern "C" int moe_routed_qgemv(const int8_t *qx, const float *dx, const int32_t *sx, int T, int D, int F, int E,
                                int topk, const int32_t *ids, const float *rw, const void *const *gate,
                                const void *const *up, const void *const *down, float *y, void *ws,
                                size_t ws_bytes, int32_t *d_status, void *stream) {
    return moe_routed_qgemv_fmt(QG_FMT_Q4K, qx, dx, sx, T, D, F, E, topk, ids, rw, gate, up, down, y, ws, ws_bytes,
                                d_status, stream);
}
