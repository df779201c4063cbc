// Dense decode mat-vec entry points: regular (qgemv_q8_0, qgemv_q4k), paired
// (qgemv_paired) and the per-block integer-sum export.
//
// The regular and paired Q8_0 projections on a prequantized activation are
// the call sites whose restoration the page measures ("ROCm: restore DeepSeek
// V4 Flash decode performance and Q4 SSD streaming", antirez/ds4 PR 623,
// Summary and the per-stage timing table in the review comments); the Q4_K
// dense projections are those of "Support AProjQ4 GGUFs" (antirez/ds4 PR 621).
#include "common.h"
#include "gemv_device.h"

namespace qg {

constexpr int kGemvMaxWaves = 8;
// smallest Q8_0 token batch served by the matrix-core form (measured at
// 16384 x 4096: the dot-product engine takes 17.8 / 20.8-21.3 / 22.1-22.6 us
// at 4 / 7 / 8 tokens, the matrix-core form 21.8-22.0 / 21.2-21.3 /
// 21.3-21.5)
constexpr int kMmMinTokens = 8;
// the same for Q4_K (8192 x 4096 at 8 tokens: 10.6 us on the engine, 11.2 on
// the matrix cores)
constexpr int kMmMinTokensQ4K = 9;

struct GemvArgs {
    const uint8_t *W0;
    float *y0;
    int N0, nt0, nwg0;  // rows, tiles, workgroups of matrix 0
    const uint8_t *W1;
    float *y1;
    int N1, nt1;
    int K;
    TileGeom tg;
    ActSrc act;  // Q8 activation, or fp32 activation quantized in the kernel
    int M;
    int mt;         // tokens staged in LDS per chunk
    int tpw;        // tiles per wave
    int waves;      // waves per workgroup
    int32_t *isum;  // per-block sums of matrix 0 (test export), else unused
    int G;          // groups (blockIdx.y): matrix g of W0 against input slice g, 1 otherwise
};

template <int FMT, int NB, bool DEBUG_ISUM, bool PIPE, bool ONE, bool F32, int RC = kActRegChunks>
__global__ __launch_bounds__(kGemvMaxWaves *kWave) void qgemv_kernel(GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // workgroups [0, nwg0) cover matrix 0, the rest matrix 1 (paired call)
    const bool second = (int)blockIdx.x >= a.nwg0;
    const int wg = second ? (int)blockIdx.x - a.nwg0 : (int)blockIdx.x;
    const uint8_t *W = second ? a.W1 : a.W0;
    float *y = second ? a.y1 : a.y0;
    const int N = second ? a.N1 : a.N0;
    const int nt = second ? a.nt1 : a.nt0;
    const int nb = a.K / 32;
    int32_t *isum = a.isum;
    // grouped call: group g = blockIdx.y takes matrix g and slice g of every
    // token's activation (row m*G + g of the [M*G, K] view), writing y[m, g, :]
    const int G = a.G, g = blockIdx.y;
    W += (size_t)g * N * a.tg.row_bytes;
    gemv_workgroup<FMT, NB, DEBUG_ISUM, PIPE, ONE, F32 ? kSrcF32 : kSrcQ8, RC>(
        W, N, a.K, a.tg, wg * a.waves * a.tpw, a.tpw, nt, a.act, a.M, a.mt, smem,
        [=](int m) { return m * G + g; }, [=](int m, int row, float v) { y[((size_t)m * G + g) * N + row] = v; },
        [=](int m, int row, int unit, const int32_t *s) {
            int32_t *o = isum + ((size_t)m * N + row) * nb + unit * NB;
#pragma unroll
            for (int b = 0; b < NB; ++b) o[b] = s[b];
        });
}

static inline bool misaligned(const void *p) { return ((uintptr_t)p & 15) != 0; }

template <int FMT, int NB, bool DEBUG_ISUM, bool PIPE, bool ONE, bool F32, int RC = kActRegChunks>
static int launch_kernel(const GemvArgs &a, int grid, size_t lds, hipStream_t stream) {
    if (ensure_lds_limit(reinterpret_cast<const void *>(&qgemv_kernel<FMT, NB, DEBUG_ISUM, PIPE, ONE, F32, RC>),
                         kLdsBytes) != QG_OK)
        return QG_ERR_LAUNCH;
    hipLaunchKernelGGL((qgemv_kernel<FMT, NB, DEBUG_ISUM, PIPE, ONE, F32, RC>), dim3(grid, a.G),
                       dim3(a.waves * kWave), lds, stream, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

template <int FMT, int NB, bool DEBUG_ISUM, bool F32>
static int launch_gemv(GemvArgs &a, hipStream_t stream) {
    using U = Unit<FMT, NB>;
    a.tg = make_tile_geom<U>(a.K);
    a.nt0 = (a.N0 + a.tg.rpt - 1) / a.tg.rpt;
    a.nt1 = a.W1 ? (a.N1 + a.tg.rpt - 1) / a.tg.rpt : 0;
    const int cus = device_cu_count();
    const int tiles = (a.nt0 + a.nt1) * a.G;
    // waves per workgroup: 8 when there are tiles for 8-wave workgroups on
    // every CU, else fewer so that the grid still spreads over the CUs
    a.waves = kGemvMaxWaves;
    while (a.waves > 1 && tiles < a.waves * cus) a.waves >>= 1;
    // one-token Q4_K: 4-wave workgroups (8192 x 4096: 5.92 -> 5.57 us)
    if (FMT == QG_FMT_Q4K && a.M == 1 && a.waves > 4) a.waves = 4;
    const int threads = a.waves * kWave;
    a.mt = tokens_per_chunk<U>(a.K, a.M, threads, F32);
    const size_t lds = gemv_lds_bytes<U>(a.waves, a.K, a.mt);
    // about one round of resident waves (LDS bounds the workgroups per CU)
    const int wg_per_cu = max(1, min(32 / a.waves, (int)(kLdsBytes / lds)));
    // Two tiles per wave only pay when registers allow the extra set: for
    // M = 1 more workgroups in staggered rounds measured faster, and the
    // 8-block Q8_0 unit would spill.  The second register set also leaves
    // room for only one 8-wave workgroup per CU, so where the LDS admits two,
    // one tile per wave is taken (16384 x 4096, 2 tokens: 17.7 -> 14.7 us).
    a.tpw = tiles_per_wave(tiles, cus * wg_per_cu * a.waves,
                           a.M > 1 && a.M <= a.mt && !(FMT == QG_FMT_Q8_0 && NB == 8) &&
                               !(a.waves == kGemvMaxWaves && wg_per_cu >= 2));
    const int per_wg = a.waves * a.tpw;
    a.nwg0 = (a.nt0 + per_wg - 1) / per_wg;
    const int grid = a.nwg0 + (a.nt1 + per_wg - 1) / per_wg;
    if (a.M == 1) {  // (one token: tiles_per_wave gives 1)
        // staging registers for one pass over the token's row where it fits
        // (the int-sum export keeps the default)
        if constexpr (!DEBUG_ISUM) {
            const int rc = act_reg_chunks(F32 ? a.K / 4 : a.K / 16, threads);
            if (rc == 1) return launch_kernel<FMT, NB, false, false, true, F32, 1>(a, grid, lds, stream);
            if (rc == 2) return launch_kernel<FMT, NB, false, false, true, F32, 2>(a, grid, lds, stream);
        }
        return launch_kernel<FMT, NB, DEBUG_ISUM, false, true, F32>(a, grid, lds, stream);
    }
    return a.tpw > 1 ? launch_kernel<FMT, NB, DEBUG_ISUM, true, false, F32>(a, grid, lds, stream)
                     : launch_kernel<FMT, NB, DEBUG_ISUM, false, false, F32>(a, grid, lds, stream);
}

template <bool DEBUG_ISUM, bool F32>
static int launch_fmt(int fmt, GemvArgs &a, hipStream_t stream) {
    if (fmt == QG_FMT_Q4K) return launch_gemv<QG_FMT_Q4K, 8, DEBUG_ISUM, F32>(a, stream);
    if (a.K <= 8192) return launch_gemv<QG_FMT_Q8_0, 4, DEBUG_ISUM, F32>(a, stream);
    return launch_gemv<QG_FMT_Q8_0, 8, DEBUG_ISUM, F32>(a, stream);
}

static int check_common(int N, int K, int M) {
    if (N < 1 || M < 1 || M > QG_MAX_M) return QG_ERR_SHAPE;
    if (K < kGroupWeights || K > QG_MAX_K || K % kGroupWeights != 0) return QG_ERR_SHAPE;
    return QG_OK;
}

// Shared argument checks and launch.  Exactly one activation source is
// given: (qx, dx[, sx]) or the fp32 x (then pqx/pdx/psx optionally receive
// the Q8 activation).
static int gemv_dispatch(int fmt, const void *W1, int N1, const void *W2, int N2, int K, const ActSrc &act, int M,
                         float *y1, float *y2, int32_t *isum, hipStream_t stream, int G = 1) {
    if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    const bool f32 = act.x != nullptr;
    if (!W1 || (!y1 && !isum)) return QG_ERR_NULL;
    if (!f32 && (!act.qx || !act.dx || (fmt == QG_FMT_Q4K && !act.sx))) return QG_ERR_NULL;
    if (W2 && !y2) return QG_ERR_NULL;
    int rc = check_common(N1, K, M);
    if (rc) return rc;
    if (W2 && N2 < 1) return QG_ERR_SHAPE;
    if (G < 1 || G > 65535 || (G > 1 && (W2 || isum))) return QG_ERR_SHAPE;
    if (misaligned(W1) || misaligned(act.qx) || misaligned(act.dx) || misaligned(act.sx) || misaligned(act.x) ||
        misaligned(act.pqx) || misaligned(act.pdx) || misaligned(act.psx) || (y1 && misaligned(y1)) ||
        misaligned(W2) || misaligned(y2) || misaligned(isum))
        return QG_ERR_ALIGN;
    GemvArgs a{};
    a.K = K;
    a.W0 = (const uint8_t *)W1;
    a.y0 = y1;
    a.N0 = N1;
    if (W2) {
        a.W1 = (const uint8_t *)W2;
        a.y1 = y2;
        a.N1 = N2;
    }
    a.act = act;
    a.M = M;
    a.isum = isum;
    a.G = G;
    clear_stale_error();
    // larger batches go to the matrix cores (same results bit for bit), whose
    // activation offsets are 32-bit: a grouped batch with M G K >= 2^32 bytes
    // of activation stays on the dot-product engine
    if (!f32 && !isum && M >= (fmt == QG_FMT_Q8_0 ? kMmMinTokens : kMmMinTokensQ4K) &&
        (uint64_t)M * (uint64_t)G * (uint64_t)K < (1ull << 32))
        return gemv_mm(fmt, a.W0, N1, y1, a.W1, N2, y2, K, act.qx, act.dx, act.sx, M, G, stream);
    if (isum) return launch_fmt<true, false>(fmt, a, stream);
    return f32 ? launch_fmt<false, true>(fmt, a, stream) : launch_fmt<false, false>(fmt, a, stream);
}

static ActSrc q8_src(const int8_t *qx, const float *dx, const int32_t *sx) {
    ActSrc s{};
    s.qx = qx;
    s.dx = dx;
    s.sx = sx;
    return s;
}

static ActSrc f32_src(const float *x, int8_t *qx, float *dx, int32_t *sx) {
    ActSrc s{};
    s.x = x;
    s.pqx = qx;
    s.pdx = dx;
    s.psx = sx;
    return s;
}

}  // namespace qg

extern "C" int qgemv_q8_0(const void *W, int N, int K, const int8_t *qx, const float *dx, int M, float *y,
                          void *stream) {
    if (!qx || !dx) return QG_ERR_NULL;
    return qg::gemv_dispatch(QG_FMT_Q8_0, W, N, nullptr, 0, K, qg::q8_src(qx, dx, nullptr), M, y, nullptr, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_q4k(const void *W, int N, int K, const int8_t *qx, const float *dx, const int32_t *sx, int M,
                         float *y, void *stream) {
    if (!qx || !dx || !sx) return QG_ERR_NULL;
    return qg::gemv_dispatch(QG_FMT_Q4K, W, N, nullptr, 0, K, qg::q8_src(qx, dx, sx), M, y, nullptr, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_paired(int fmt, const void *W1, int N1, const void *W2, int N2, int K, const int8_t *qx,
                            const float *dx, const int32_t *sx, int M, float *y1, float *y2, void *stream) {
    if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!W2 || !y2 || !y1 || !qx || !dx) return QG_ERR_NULL;
    return qg::gemv_dispatch(fmt, W1, N1, W2, N2, K, qg::q8_src(qx, dx, sx), M, y1, y2, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_grouped(int fmt, const void *W, int G, int N, int K, const int8_t *qx, const float *dx,
                             const int32_t *sx, int M, float *y, void *stream) {
    if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!qx || !dx || (fmt == QG_FMT_Q4K && !sx)) return QG_ERR_NULL;
    return qg::gemv_dispatch(fmt, W, N, nullptr, 0, K, qg::q8_src(qx, dx, sx), M, y, nullptr, nullptr,
                             (hipStream_t)stream, G);
}

extern "C" int qgemv_q8_0_f32(const void *W, int N, int K, const float *x, int M, float *y, int8_t *qx, float *dx,
                              int32_t *sx, void *stream) {
    if (!x) return QG_ERR_NULL;
    return qg::gemv_dispatch(QG_FMT_Q8_0, W, N, nullptr, 0, K, qg::f32_src(x, qx, dx, sx), M, y, nullptr, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_q4k_f32(const void *W, int N, int K, const float *x, int M, float *y, int8_t *qx, float *dx,
                             int32_t *sx, void *stream) {
    if (!x) return QG_ERR_NULL;
    return qg::gemv_dispatch(QG_FMT_Q4K, W, N, nullptr, 0, K, qg::f32_src(x, qx, dx, sx), M, y, nullptr, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_paired_f32(int fmt, const void *W1, int N1, const void *W2, int N2, int K, const float *x, int M,
                                float *y1, float *y2, int8_t *qx, float *dx, int32_t *sx, void *stream) {
    if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!W2 || !y2 || !y1 || !x) return QG_ERR_NULL;
    return qg::gemv_dispatch(fmt, W1, N1, W2, N2, K, qg::f32_src(x, qx, dx, sx), M, y1, y2, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_debug_block_isums(int fmt, const void *W, int N, int K, const int8_t *qx, int M, int32_t *isum,
                                       void *stream) {
    if (!isum) return QG_ERR_NULL;
    // The decoders also read dx (and sx for Q4_K).  The export has no scales,
    // so it hands the decoder the quant buffer itself in their place (those
    // reads stay inside qx: M*K/8 bytes <= M*K); the fp32 result is discarded
    // and only the exact integer sums are written.
    if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!qx) return QG_ERR_NULL;
    return qg::gemv_dispatch(fmt, W, N, nullptr, 0, K,
                             qg::q8_src(qx, reinterpret_cast<const float *>(qx), reinterpret_cast<const int32_t *>(qx)),
                             M, nullptr, nullptr, isum, (hipStream_t)stream);
}
