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
// LDS for staged activations per workgroup (the weight tiles take
// kGemvWaves * 64 * group bytes on top; Q8_0: 68 KiB, Q4_K: 36 KiB).
constexpr int kActLdsBudget = 44 * 1024;

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

// Stage tokens [m0, m0 + mt) of the Q8 activation into padded LDS records
// (whole workgroup; global -> VGPR -> LDS, 16 bytes per access).
template <int FMT>
__device__ __forceinline__ void stage_activations(const int8_t *__restrict__ qx, const float *__restrict__ dx,
                                                  const int32_t *__restrict__ sx, int K, int m0, int mt,
                                                  uint8_t *lds) {
    constexpr int REC = ActRecord<FMT>::bytes;
    const int gpr = K / kGroupWeights;
    const int nq = mt * K / 16;  // 16-byte chunks of quants
    const uint4 *q = reinterpret_cast<const uint4 *>(qx + (size_t)m0 * K);
    for (int c = threadIdx.x; c < nq; c += kGemvWaves * kWave) {
        const int tg = c >> 4;  // token * gpr + group
        *reinterpret_cast<uint4 *>(lds + (size_t)tg * REC + (c & 15) * 16) = q[c];
    }
    const int ns = mt * gpr * 2;  // 16-byte chunks of scales (two per group)
    const uint4 *d = reinterpret_cast<const uint4 *>(dx + (size_t)m0 * (K / 32));
    const uint4 *su = reinterpret_cast<const uint4 *>(sx + (size_t)m0 * (K / 32));
    for (int c = threadIdx.x; c < ns; c += kGemvWaves * kWave) {
        uint8_t *rec = lds + (size_t)(c >> 1) * REC + 256 + (c & 1) * 16;
        *reinterpret_cast<uint4 *>(rec) = d[c];
        if (FMT == QG_FMT_Q4K) *reinterpret_cast<uint4 *>(rec + 32) = su[c];
    }
}

template <int FMT, bool DEBUG_ISUM>
__global__ __launch_bounds__(kGemvWaves *kWave) void qgemv_kernel(GemvArgs a) {
    constexpr int GB = GroupBytes<FMT>::value;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    int tile = blockIdx.x * kGemvWaves + wave;
    const bool second = tile >= a.nt0;
    if (second) tile -= a.nt0;
    // a wave without a tile still takes part in the workgroup's barriers
    const bool has_tile = !second || tile < a.nt1;
    const uint8_t *W = second ? a.W1 : a.W0;
    float *y = second ? a.y1 : a.y0;
    const int N = second ? a.N1 : a.N0;
    const TileGeom tg = a.tg;
    const int K = a.K;
    const int nb = K / 32;

    uint8_t *lw = smem + wave * kWave * GB;
    uint8_t *lact = smem + kGemvWaves * kWave * GB;
    constexpr int REC = ActRecord<FMT>::bytes;

    // 1. this wave's weight tile: HBM -> LDS, left in flight
    int nrows = 0;
    if (has_tile) nrows = issue_tile_to_lds<FMT>(W, N, tg, tile, lw);
    const int r = lane >> tg.lsh;
    const int g = lane & (tg.lpr - 1);
    const bool valid = has_tile && g < tg.gpr && r < nrows;
    const int row = tile * tg.rpt + r;
    GroupRegs<FMT> regs;

    for (int m0 = 0; m0 < a.M; m0 += a.mt) {
        const int mt = min(a.mt, a.M - m0);
        if (m0 > 0) __syncthreads();  // every wave is done with the previous chunk
        // 2. the chunk's activation quants, scales (and block sums), shared by the workgroup
        stage_activations<FMT>(a.qx, a.dx, a.sx, K, m0, mt, lact);
        wait_vmem_all();  // this wave's weight tile has landed in LDS
        __syncthreads();
        if (m0 == 0 && valid) read_group<FMT>(lw + (r * tg.gpr + g) * GB, regs);

        for (int mm = 0; mm < mt; ++mm) {
            const int m = m0 + mm;
            float p = 0.0f;
            if (valid) {
                int32_t isum_tmp[8];
                const uint8_t *rec = lact + (size_t)(mm * tg.gpr + g) * REC;
                p = group_dot<FMT>(regs, reinterpret_cast<const int8_t *>(rec),
                                   reinterpret_cast<const float *>(rec + 256),
                                   reinterpret_cast<const int32_t *>(rec + 288), DEBUG_ISUM ? isum_tmp : nullptr);
                if (DEBUG_ISUM) {
                    int32_t *o = a.isum + ((size_t)m * N + row) * nb + g * 8;
#pragma unroll
                    for (int b = 0; b < 8; ++b) o[b] = isum_tmp[b];
                }
            }
            p = row_reduce(p, tg.lpr);
            if (!DEBUG_ISUM && valid && g == 0) y[(size_t)m * N + row] = p;
        }
    }
}

static inline bool misaligned(const void *p) { return ((uintptr_t)p & 15) != 0; }

template <int FMT, bool DEBUG_ISUM>
static int launch_gemv(GemvArgs &a, hipStream_t stream) {
    constexpr int GB = GroupBytes<FMT>::value;
    const int per_token = act_lds_bytes_per_token<FMT>(a.K);
    a.mt = max(1, min(a.M, kActLdsBudget / per_token));
    const size_t lds = (size_t)kGemvWaves * kWave * GB + (size_t)a.mt * per_token;
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
