// Routed-MoE decode over a compact selected-expert table.
//
// "ROCm: restore DeepSeek V4 Flash decode performance and Q4 SSD streaming"
// (antirez/ds4 PR 623), Summary and Correctness: the compact table of the
// selected experts must be staged before the pointer-backed routed-MoE
// launch; its absence, or an expert id outside the expert range, is a hard
// decode error.  Routing is 6 of 256/384 experts with sigmoid-normalized
// weights (ROCm/ATOM "DeepSeek-V4 Usage Guide", opening paragraph and MoE
// tips).  The experts are Q4_K (the "Q4KExperts" model of PR 623).
//
// Five launches on the caller's stream, none of which returns data to the host:
//   1. table   : validate ids, distinct experts ascending, slots, CSR pair lists
//   2. gate/up : per distinct expert, gate and up rows against each of its
//                pairs' tokens (weights streamed once per expert)
//   3. h       : h = silu(g) * up, Q8-quantized per 32-block
//   4. down    : per distinct expert, down rows against each pair's h
//   5. combine : y[t] = sum_k rw[t,k] * o[t,k] in k order
// Grids 2 and 4 are sized for the largest possible number of distinct experts,
// min(T*topk, E); workgroups beyond the device-side count exit at once.
#include "common.h"
#include "gemv_device.h"
#include "quantize_device.h"

namespace qg {

constexpr int kMoeWaves = 4;
constexpr int kTableThreads = 1024;

struct MoeWs {
    int32_t *nuniq, *uniq, *slot, *pair_off, *pairs;
    float *g, *v, *h;
    int8_t *hq;
    float *hd;
    int32_t *hs;
    float *o;
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
    };
    size_t at = 0;
    for (int i = 0; i < QG_WS_COUNT; ++i) {
        off[i] = at;
        at = align256(at + sz[i]);
    }
    return at;
}

// ---------------------------------------------------------------- 1. table

// Exclusive scan of v[0..n) in place (n <= 4 * kTableThreads), whole block.
// Returns the total.  tmp: kTableThreads ints of LDS.
__device__ int block_exclusive_scan(int *v, int n, int *tmp) {
    const int t = threadIdx.x;
    int local[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = 4 * t + i;
        local[i] = idx < n ? v[idx] : 0;
        sum += local[i];
    }
    tmp[t] = sum;
    __syncthreads();
    for (int off = 1; off < kTableThreads; off <<= 1) {
        const int add = t >= off ? tmp[t - off] : 0;
        __syncthreads();
        tmp[t] += add;
        __syncthreads();
    }
    int run = tmp[t] - sum;  // exclusive prefix of this thread's 4 entries
    const int total = tmp[kTableThreads - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = 4 * t + i;
        if (idx < n) v[idx] = run;
        run += local[i];
    }
    __syncthreads();
    return total;
}

__device__ __forceinline__ bool bad_pointer(const void *p) { return p == nullptr || ((uintptr_t)p & 15) != 0; }

__global__ __launch_bounds__(kTableThreads) void moe_table_kernel(const int32_t *__restrict__ ids, int P, int E,
                                                                 const void *const *gate, const void *const *up,
                                                                 const void *const *down, MoeWs ws,
                                                                 int32_t *status) {
    __shared__ int flag[QG_MAX_EXPERTS];  // selected and usable
    __shared__ int rank[QG_MAX_EXPERTS];  // index in uniq
    __shared__ int cnt[QG_MAX_EXPERTS];   // pairs per distinct expert, then running fill position
    __shared__ int tmp[kTableThreads];
    __shared__ int chunk_slot[kTableThreads];
    const int t = threadIdx.x;
    if (t == 0) atomicExch(status, QG_DEV_OK);
    for (int e = t; e < E; e += kTableThreads) flag[e] = 0;
    __threadfence();
    __syncthreads();
    for (int p = t; p < P; p += kTableThreads) {
        const int e = ids[p];
        if (e < 0 || e >= E)
            atomicCAS(status, QG_DEV_OK, QG_DEV_BAD_EXPERT);
        else
            flag[e] = 1;
    }
    __syncthreads();
    for (int e = t; e < E; e += kTableThreads) {
        if (flag[e] && (bad_pointer(gate[e]) || bad_pointer(up[e]) || bad_pointer(down[e]))) {
            flag[e] = 0;
            atomicCAS(status, QG_DEV_OK, QG_DEV_NULL_EXPERT);
        }
        rank[e] = flag[e];
    }
    __syncthreads();
    const int U = block_exclusive_scan(rank, E, tmp);
    for (int e = t; e < E; e += kTableThreads)
        if (flag[e]) ws.uniq[rank[e]] = e;
    if (t == 0) *ws.nuniq = U;
    for (int u = t; u < U; u += kTableThreads) cnt[u] = 0;
    __syncthreads();
    for (int p = t; p < P; p += kTableThreads) {
        const int e = ids[p];
        const int s = (e >= 0 && e < E && flag[e]) ? rank[e] : -1;
        ws.slot[p] = s;
        if (s >= 0) atomicAdd(&cnt[s], 1);
    }
    __syncthreads();
    const int npairs = block_exclusive_scan(cnt, U, tmp);  // cnt[u] = first position of expert u
    for (int u = t; u < U; u += kTableThreads) ws.pair_off[u] = cnt[u];
    if (t == 0) ws.pair_off[U] = npairs;
    // stable fill: pairs of one expert keep ascending pair order
    for (int c0 = 0; c0 < P; c0 += kTableThreads) {
        const int p = c0 + t;
        int s = -1;
        if (p < P) {
            const int e = ids[p];
            s = (e >= 0 && e < E && flag[e]) ? rank[e] : -1;
        }
        chunk_slot[t] = s;
        __syncthreads();
        int before = 0, same = 0;
        if (s >= 0) {
            for (int j = 0; j < kTableThreads && c0 + j < P; ++j) {
                const int sj = chunk_slot[j];
                same += sj == s;
                before += (sj == s) & (j < t);
            }
            ws.pairs[cnt[s] + before] = p;
        }
        __syncthreads();
        if (s >= 0 && before == 0) cnt[s] += same;  // one thread per expert present in the chunk
        __syncthreads();
    }
}

// ---------------------------------------------------------------- 2./4. expert GEMVs

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
};

using QU = Unit<QG_FMT_Q4K, 8>;

// gate and up of expert uniq[blockIdx.y]: workgroups [0, nwg) take gate rows,
// [nwg, 2 nwg) up rows; the tokens are the expert's pairs' tokens.
__global__ __launch_bounds__(kMoeWaves *kWave) void moe_gate_up_kernel(MoeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int u = blockIdx.y;
    if (u >= *a.ws.nuniq) return;  // the whole workgroup leaves
    const int e = a.ws.uniq[u];
    const int p0 = a.ws.pair_off[u];
    const int cnt = a.ws.pair_off[u + 1] - p0;
    const int ntiles = (a.F + a.tg.rpt - 1) / a.tg.rpt;
    const int nwg = (ntiles + kMoeWaves - 1) / kMoeWaves;
    const bool is_up = (int)blockIdx.x >= nwg;
    const int wg = is_up ? (int)blockIdx.x - nwg : (int)blockIdx.x;
    const uint8_t *W = reinterpret_cast<const uint8_t *>(is_up ? a.up[e] : a.gate[e]);
    float *dst = is_up ? a.ws.v : a.ws.g;
    const int32_t *pairs = a.ws.pairs + p0;
    const int topk = a.topk, F = a.F;
    ActSrc act{};
    act.qx = a.qx;
    act.dx = a.dx;
    act.sx = a.sx;
    gemv_workgroup<QG_FMT_Q4K, 8, false, false, false, false>(
        W, F, a.D, a.tg, wg * kMoeWaves, 1, ntiles, act, cnt, a.mt, smem,
        [=](int m) { return pairs[m] / topk; },
        [=](int m, int row, float v) { dst[(size_t)pairs[m] * F + row] = v; },
        [](int, int, int, const int32_t *) {});
}

// down of expert uniq[blockIdx.y] against the quantized h of each of its pairs
__global__ __launch_bounds__(kMoeWaves *kWave) void moe_down_kernel(MoeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int u = blockIdx.y;
    if (u >= *a.ws.nuniq) return;
    const int e = a.ws.uniq[u];
    const int p0 = a.ws.pair_off[u];
    const int cnt = a.ws.pair_off[u + 1] - p0;
    const int ntiles = (a.D + a.tg.rpt - 1) / a.tg.rpt;
    const uint8_t *W = reinterpret_cast<const uint8_t *>(a.down[e]);
    const int32_t *pairs = a.ws.pairs + p0;
    float *o = a.ws.o;
    const int D = a.D;
    ActSrc act{};
    act.qx = a.ws.hq;
    act.dx = a.ws.hd;
    act.sx = a.ws.hs;
    gemv_workgroup<QG_FMT_Q4K, 8, false, false, false, false>(
        W, D, a.F, a.tg, (int)blockIdx.x * kMoeWaves, 1, ntiles, act, cnt, a.mt, smem,
        [=](int m) { return pairs[m]; }, [=](int m, int row, float v) { o[(size_t)pairs[m] * D + row] = v; },
        [](int, int, int, const int32_t *) {});
}

// ---------------------------------------------------------------- 3. h = silu(g) * v, Q8

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// 8 lanes per 32-block of h, as in the activation quantizer.
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

// ---------------------------------------------------------------- 5. combine

__global__ __launch_bounds__(256) void moe_combine_kernel(MoeWs ws, const float *__restrict__ rw, int T, int D,
                                                          int topk, float *__restrict__ y) {
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int per_t = D / 4;
    if (gid >= T * per_t) return;
    const int t = gid / per_t, n4 = gid - t * per_t;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < topk; ++k) {
        const int p = t * topk + k;
        if (ws.slot[p] < 0) continue;  // invalid id or unusable expert: contributes nothing
        const float r = rw[p];
        const float4 o = *reinterpret_cast<const float4 *>(ws.o + (size_t)p * D + 4 * n4);
        acc.x = fmaf_exact(r, o.x, acc.x);
        acc.y = fmaf_exact(r, o.y, acc.y);
        acc.z = fmaf_exact(r, o.z, acc.z);
        acc.w = fmaf_exact(r, o.w, acc.w);
    }
    *reinterpret_cast<float4 *>(y + (size_t)t * D + 4 * n4) = acc;
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
    return w;
}

template <class Kern>
static bool raise_lds_limit(Kern *k, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes) == hipSuccess;
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

extern "C" int moe_routed_qgemv(const int8_t *qx, const float *dx, const int32_t *sx, int T, int D, int F, int E,
                                int topk, const int32_t *ids, const float *rw, const void *const *gate,
                                const void *const *up, const void *const *down, float *y, void *ws,
                                size_t ws_bytes, int32_t *d_status, void *stream) {
    using namespace qg;
    if (!qx || !dx || !sx || !ids || !rw || !gate || !up || !down || !y || !ws || !d_status) return QG_ERR_NULL;
    if (!moe_shape_ok(T, topk, E, D, F)) return QG_ERR_SHAPE;
    size_t off[QG_WS_COUNT];
    const size_t need = moe_layout(T, topk, E, D, F, off);
    if (ws_bytes < need) return QG_ERR_WORKSPACE;
    const uintptr_t a16 = (uintptr_t)qx | (uintptr_t)dx | (uintptr_t)sx | (uintptr_t)y | (uintptr_t)ws;
    const uintptr_t a8 = (uintptr_t)gate | (uintptr_t)up | (uintptr_t)down;
    if ((a16 & 15) || (a8 & 7) || ((uintptr_t)ids & 3) || ((uintptr_t)rw & 3) || ((uintptr_t)d_status & 3))
        return QG_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    const int P = T * topk;
    const int Ucap = P < E ? P : E;
    MoeWs w = ws_pointers(ws, off);

    hipLaunchKernelGGL(moe_table_kernel, dim3(1), dim3(kTableThreads), 0, st, ids, P, E, gate, up, down, w,
                       d_status);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;

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

    // gate/up: K = D
    constexpr int threads = kMoeWaves * kWave;
    a.tg = make_tile_geom<QU>(D);
    a.mt = tokens_per_chunk<QU>(D, QG_MAX_MOE_PAIRS, threads);
    size_t lds = gemv_lds_bytes<QU>(kMoeWaves, D, a.mt);
    static bool lds_gu = false, lds_dn = false;  // idempotent: raise the dynamic-LDS limit once
    const size_t lds_max = kLdsBytes;
    if (!lds_gu) lds_gu = raise_lds_limit(moe_gate_up_kernel, lds_max);
    int nwg = ((F + a.tg.rpt - 1) / a.tg.rpt + kMoeWaves - 1) / kMoeWaves;
    hipLaunchKernelGGL(moe_gate_up_kernel, dim3(2 * nwg, Ucap), dim3(threads), lds, st, a);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;

    const long long hthreads = (long long)P * (F / 32) * 8;
    hipLaunchKernelGGL(moe_h_quant_kernel, dim3((unsigned)((hthreads + 255) / 256)), dim3(256), 0, st, w, P, F);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;

    // down: K = F
    a.tg = make_tile_geom<QU>(F);
    a.mt = tokens_per_chunk<QU>(F, QG_MAX_MOE_PAIRS, threads);
    lds = gemv_lds_bytes<QU>(kMoeWaves, F, a.mt);
    if (!lds_dn) lds_dn = raise_lds_limit(moe_down_kernel, lds_max);
    nwg = ((D + a.tg.rpt - 1) / a.tg.rpt + kMoeWaves - 1) / kMoeWaves;
    hipLaunchKernelGGL(moe_down_kernel, dim3(nwg, Ucap), dim3(threads), lds, st, a);
    if (hipGetLastError() != hipSuccess) return QG_ERR_LAUNCH;

    const long long cthreads = (long long)T * (D / 4);
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((cthreads + 255) / 256)), dim3(256), 0, st, w, rw, T, D,
                       topk, y);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}
