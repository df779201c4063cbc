// Dense mat-vec for the block-scaled expert formats (FP8 E4M3 128 x 128, FP4
// E2M1 1 x 32, UE8M0 scales) on a Q8 activation, and the matrix sizes of
// every format.  The routed use of the same engine is in moe.hip.
#include "common.h"
#include "mx_device.h"

namespace qg {

struct MxArgs {
    const uint8_t *W;
    int N, K, M, mt;
    const int8_t *qx;
    const float *dx;
    float *y;
};

template <int FMT, int CPL>
__global__ __launch_bounds__(kMxWaves *kWave) void qgemv_mx_kernel(MxArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int L = mx_loads(FMT);
    constexpr int R = mx_rows_per_wave(L, CPL);
    float *y = a.y;
    const int N = a.N;
    mx_workgroup<FMT, CPL, L>(
        a.W, a.N, a.K, (int)blockIdx.x * kMxWaves * R, a.M, a.mt, a.qx, a.dx, [](int m) { return m; },
        [=](int m, int row, float v) { y[(size_t)m * N + row] = v; }, smem);
}

template <int FMT, int CPL>
static int launch_mx_cpl(MxArgs &a, hipStream_t stream) {
    constexpr int rows_per_wg = kMxWaves * mx_rows_per_wave(mx_loads(FMT), CPL);
    if (ensure_lds_limit(reinterpret_cast<const void *>(&qgemv_mx_kernel<FMT, CPL>), kMxLdsMax) != QG_OK)
        return QG_ERR_LAUNCH;
    const int grid = (a.N + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((qgemv_mx_kernel<FMT, CPL>), dim3(grid), dim3(kMxWaves * kWave),
                       (size_t)a.mt * mx_token_rec(a.K) + mx_scale_lds<FMT>(a.K, CPL, mx_loads(FMT)), stream, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

template <int FMT>
static int launch_mx(MxArgs &a, hipStream_t stream) {
    a.mt = mx_tokens_per_chunk(a.K, a.M);
    switch (mx_chunks_per_lane<FMT>(a.K)) {
        case 1: return launch_mx_cpl<FMT, 1>(a, stream);
        case 2: return launch_mx_cpl<FMT, 2>(a, stream);
        case 4: return launch_mx_cpl<FMT, 4>(a, stream);
        case 8: return launch_mx_cpl<FMT, 8>(a, stream);
        case 16: return launch_mx_cpl<FMT, 16>(a, stream);
        default: return QG_ERR_SHAPE;
    }
}

}  // namespace qg

extern "C" size_t qg_matrix_bytes(int fmt, int N, int K) {
    if (N < 1 || K < qg::kGroupWeights || K > QG_MAX_K || K % qg::kGroupWeights) return 0;
    switch (fmt) {
        case QG_FMT_Q8_0: return (size_t)N * (K / 32) * 34;
        case QG_FMT_Q4K: return (size_t)N * (K / 256) * 144;
        case QG_FMT_FP8_E4M3_B128:
            return qg::mx_align16(qg::mx_align256((size_t)N * K) + (size_t)((N + 127) / 128) * (K / 128));
        case QG_FMT_FP4_E2M1_MX: return qg::mx_align16(qg::mx_align256((size_t)N * K / 2) + (size_t)N * (K / 32));
        default: return 0;
    }
}

extern "C" int qgemv_mx(int fmt, const void *W, int N, int K, const int8_t *qx, const float *dx, int M, float *y,
                        void *stream) {
    if (fmt != QG_FMT_FP8_E4M3_B128 && fmt != QG_FMT_FP4_E2M1_MX) return QG_ERR_FORMAT;
    if (!W || !qx || !dx || !y) return QG_ERR_NULL;
    if (N < 1 || M < 1 || M > QG_MAX_M) return QG_ERR_SHAPE;
    if (K < qg::kGroupWeights || K > QG_MAX_K || K % qg::kGroupWeights) return QG_ERR_SHAPE;
    if (((uintptr_t)W | (uintptr_t)qx | (uintptr_t)dx | (uintptr_t)y) & 15) return QG_ERR_ALIGN;
    qg::MxArgs a{};
    a.W = reinterpret_cast<const uint8_t *>(W);
    a.N = N;
    a.K = K;
    a.M = M;
    a.qx = qx;
    a.dx = dx;
    a.y = y;
    qg::clear_stale_error();
    if (fmt == QG_FMT_FP8_E4M3_B128) return qg::launch_mx<QG_FMT_FP8_E4M3_B128>(a, (hipStream_t)stream);
    return qg::launch_mx<QG_FMT_FP4_E2M1_MX>(a, (hipStream_t)stream);
}
