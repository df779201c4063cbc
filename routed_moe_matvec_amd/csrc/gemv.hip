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

constexpr int kGemvWaves = 4;

struct GemvArgs {
    const uint8_t *W0;
    float *y0;
    int N0, nt0;
    const uint8_t *W1;
    float *y1;
    int N1, nt1;
    int K;
    TileGeom tg;
    const int8_t *qx;
    const float *dx;
    const int32_t *sx;
    int M;
    int mt;         // tokens staged in LDS per chunk
    int32_t *isum;  // per-block sums of matrix 0 (test export), else unused
};

template <int FMT, bool DEBUG_ISUM>
__global__ __launch_bounds__(kGemvWaves *kWave) void qgemv_kernel(GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int wave = threadIdx.x / kWave;
    int tile = blockIdx.x * kGemvWaves + wave;
    const bool second = tile >= a.nt0;
    if (second) tile -= a.nt0;
    // a wave without a tile still takes part in the workgroup's barriers
    const bool has_tile = !second || tile < a.nt1;
    const uint8_t *W = second ? a.W1 : a.W0;
    float *y = second ? a.y1 : a.y0;
    const int N = second ? a.N1 : a.N0;
    const int nb = a.K / 32;
    int32_t *isum = a.isum;
    gemv_tiles_workgroup<FMT, kGemvWaves, DEBUG_ISUM>(
        W, N, a.K, a.tg, tile, has_tile, a.qx, a.dx, a.sx, a.M, a.mt, smem, [](int m) { return m; },
        [=](int m, int row, float v) { y[(size_t)m * N + row] = v; },
        [=](int m, int row, int g, const int32_t *s8) {
            int32_t *o = isum + ((size_t)m * N + row) * nb + g * 8;
#pragma unroll
            for (int b = 0; b < 8; ++b) o[b] = s8[b];
        });
}

static inline bool misaligned(const void *p) { return ((uintptr_t)p & 15) != 0; }

template <int FMT, bool DEBUG_ISUM>
static int launch_gemv(GemvArgs &a, hipStream_t stream) {
    constexpr int GB = GroupBytes<FMT>::value;
    a.mt = tokens_per_chunk<FMT>(a.K, a.M);
    const size_t lds = gemv_lds_bytes<FMT>(kGemvWaves, a.K, a.mt);
    static bool attr_set = false;  // idempotent: raising the dynamic-LDS limit once per kernel
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(&qgemv_kernel<FMT, DEBUG_ISUM>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                kGemvWaves * kWave * GB + kActLdsBudget + 16 * 1024) != hipSuccess)
            return QG_ERR_LAUNCH;
        attr_set = true;
    }
    const int tiles = a.nt0 + a.nt1;
    const int grid = (tiles + kGemvWaves - 1) / kGemvWaves;
    hipLaunchKernelGGL((qgemv_kernel<FMT, DEBUG_ISUM>), dim3(grid), dim3(kGemvWaves * kWave), lds, stream, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

static int check_common(int N, int K, int M) {
    if (N < 1 || M < 1 || M > QG_MAX_M) return QG_ERR_SHAPE;
    if (K < kGroupWeights || K > QG_MAX_K || K % kGroupWeights != 0) return QG_ERR_SHAPE;
    return QG_OK;
}

static int gemv_dispatch(int fmt, const void *W1, int N1, const void *W2, int N2, int K, const int8_t *qx,
                         const float *dx, const int32_t *sx, int M, float *y1, float *y2, int32_t *isum,
                         hipStream_t stream) {
    if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!W1 || !qx || !dx || (!y1 && !isum)) return QG_ERR_NULL;
    if (fmt == QG_FMT_Q4K && !sx) return QG_ERR_NULL;
    if (W2 && !y2) return QG_ERR_NULL;
    int rc = check_common(N1, K, M);
    if (rc) return rc;
    if (W2 && N2 < 1) return QG_ERR_SHAPE;
    if (misaligned(W1) || misaligned(qx) || misaligned(dx) || (y1 && misaligned(y1)) || misaligned(W2) ||
        misaligned(y2) || misaligned(sx) || misaligned(isum))
        return QG_ERR_ALIGN;
    GemvArgs a{};
    a.tg = make_tile_geom(K);
    a.K = K;
    a.W0 = (const uint8_t *)W1;
    a.y0 = y1;
    a.N0 = N1;
    a.nt0 = (N1 + a.tg.rpt - 1) / a.tg.rpt;
    if (W2) {
        a.W1 = (const uint8_t *)W2;
        a.y1 = y2;
        a.N1 = N2;
        a.nt1 = (N2 + a.tg.rpt - 1) / a.tg.rpt;
    }
    a.qx = qx;
    a.dx = dx;
    a.sx = sx;
    a.M = M;
    a.isum = isum;
    if (isum) {
        return fmt == QG_FMT_Q8_0 ? launch_gemv<QG_FMT_Q8_0, true>(a, stream)
                                  : launch_gemv<QG_FMT_Q4K, true>(a, stream);
    }
    return fmt == QG_FMT_Q8_0 ? launch_gemv<QG_FMT_Q8_0, false>(a, stream) : launch_gemv<QG_FMT_Q4K, false>(a, stream);
}

}  // namespace qg

extern "C" int qgemv_q8_0(const void *W, int N, int K, const int8_t *qx, const float *dx, int M, float *y,
                          void *stream) {
    return qg::gemv_dispatch(QG_FMT_Q8_0, W, N, nullptr, 0, K, qx, dx, nullptr, M, y, nullptr, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_q4k(const void *W, int N, int K, const int8_t *qx, const float *dx, const int32_t *sx, int M,
                         float *y, void *stream) {
    return qg::gemv_dispatch(QG_FMT_Q4K, W, N, nullptr, 0, K, qx, dx, sx, M, y, nullptr, nullptr,
                             (hipStream_t)stream);
}

extern "C" int qgemv_paired(int fmt, const void *W1, int N1, const void *W2, int N2, int K, const int8_t *qx,
                            const float *dx, const int32_t *sx, int M, float *y1, float *y2, void *stream) {
    if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4K) return QG_ERR_FORMAT;
    if (!W2 || !y2 || !y1) return QG_ERR_NULL;
    return qg::gemv_dispatch(fmt, W1, N1, W2, N2, K, qx, dx, sx, M, y1, y2, nullptr, (hipStream_t)stream);
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
    return qg::gemv_dispatch(fmt, W, N, nullptr, 0, K, qx, reinterpret_cast<const float *>(qx),
                             reinterpret_cast<const int32_t *>(qx), M, nullptr, nullptr, isum, (hipStream_t)stream);
}
