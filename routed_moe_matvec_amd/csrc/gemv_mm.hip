// Batched decode mat-vec on the matrix cores: Q8_0 or Q4_K weights x Q8
// activation for a batch of tokens ("ROCm: restore DeepSeek V4 Flash decode
// performance and Q4 SSD streaming", antirez/ds4 PR 623: the Q8_0 projections
// on a prequantized activation; the page's kernels take one token per call,
// this form serves the batched calls of the same projections, and prefill
// batches of Q8_0 through qgemm_q8_0).
//
// Numerics are those of the one-token engine, so a batched call reproduces
// the one-token call bit for bit on every token:
//   * a v_mfma_i32_32x32x32_i8 per 32-block gives the exact integer block sum
//     isum[n, m, b] for 32 rows x 32 tokens (Q4_K: the A operand holds the
//     sub-block's nibbles);
//   * Q8_0: s = fp32(dw[n, b] * dx[m, b]) and acc = fma(isum, s, acc) in block
//     order inside each unit of NB blocks (the one-token engine's per-lane
//     unit), starting from +0; Q4_K: inner = fma(d sc_j, isum, -(dmin m_j) sx_j)
//     and acc = fma(inner, dx_j, acc) over the superblock's sub-blocks;
//   * the units of a row are summed by the same pairwise tree over the next
//     power of two of units (the one-token engine's xor butterfly, padded
//     with zeros).
//
// Token tiles: a workgroup takes TT tiles of 32 tokens (TT > 1 for Q8_0
// batches of several tiles, whose waves then share each slice's weight
// stage); larger batches run one workgroup per (row tile, token block).
// With several token blocks per row tile, the workgroups are remapped so that
// each XCD runs a contiguous range of row tiles (workgroups are dealt to the
// XCDs in turn), so a row tile's weights are fetched into one XCD's L2.
//
// Work split: a workgroup owns 32 rows of one matrix; its KS slices (waves per
// token tile) take consecutive, power-of-two-aligned runs of the row's
// 256-weight groups, so each slice is a subtree of the unit tree.  A slice
// streams its 32 rows' groups through registers into an LDS stage (the
// groups two ahead stay in flight while the current one is multiplied),
// builds a small table of the stage's scales, and keeps one partial sum per
// tree level.  Where the LDS allows it, the activation goes through a small
// LDS tile too (see mm_device.h).  The slices' subtree sums meet in LDS and
// are added in tree order.
//
// MFMA roles: A = weights (row i = lane % 32, 16 of the block's 32 quants per
// lane half), B = activation (token j = lane % 32).  The 32x32 i32 result puts
// token lane % 32 and rows 8q + 4 (lane / 32) + t (q, t < 4) in a lane's 16
// registers, so one activation scale and 16 weight scales scale a lane's sums.
#include "mm_device.h"

namespace qg {

struct MmArgs {
    const uint8_t *W0, *W1;
    float *y0, *y1;
    int N0, N1;
    int nt0;  // 32-row tiles of matrix 0; matrix 1's follow
    int ntok; // token blocks of TT x 32 tokens: workgroup x takes row tile x / ntok, block x % ntok
    const int8_t *qx;
    const float *dx;
    const int32_t *sx;  // Q4_K: block sums of the activation
    int K, M, G;
    int row_bytes;
    int groups;  // 256-weight groups per row
    int gps;     // groups per slice (power of two)
    int KS;      // slices = waves per workgroup
};

template <int FMT, int NB, int GPS, int TT>
__global__ __launch_bounds__(kMmMaxSlices *kWave) void qgemv_mm_kernel(MmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // token tiles of one row tile are neighbours in the launch order, so the
    // row tile's weights are still in the caches when the next token tile
    // reads them.  With several token tiles per row tile, work item wi of
    // workgroup x goes to the XCD that runs x (workgroups are dealt to the 8
    // XCDs in turn): XCD j takes items j * n / 8 onwards, so a row tile's
    // token tiles share one XCD's L2 instead of each XCD fetching the row
    // tile (512 x 8192 x 4096: 123 -> 111 us; one token tile: unchanged or
    // slower, so kept in launch order)
    const int nblk = (int)gridDim.x;
    int wi = (int)blockIdx.x;
    if (a.ntok > 1 && (nblk & 7) == 0) wi = (wi & 7) * (nblk >> 3) + (wi >> 3);
    const int rtile = wi / a.ntok;
    const bool second = rtile >= a.nt0;
    const int g = blockIdx.y;  // grouped call: matrix g against activation slice g
    const int G = a.G;
    MmTile t;
    t.N = second ? a.N1 : a.N0;
    t.W = (second ? a.W1 : a.W0) + (size_t)g * t.N * a.row_bytes;
    t.row0 = (second ? rtile - a.nt0 : rtile) * kMmRows;
    t.m0 = (wi - rtile * a.ntok) * kMmTokens * TT;
    t.M = a.M;
    t.qx = a.qx;
    t.dx = a.dx;
    t.sx = a.sx;
    t.K = a.K;
    t.row_bytes = a.row_bytes;
    t.groups = a.groups;
    t.gps = a.gps;
    t.KS = a.KS;
    float *y = second ? a.y1 : a.y0;
    const int N = t.N;
    mm_tile<FMT, NB, GPS, TT>(
        t, [=](int m) { return m * G + g; }, [=](int m, int row, float v) { y[((size_t)m * G + g) * N + row] = v; },
        smem);
}

// Dynamic LDS of a workgroup of KS slices x TT token tiles.
template <int FMT>
constexpr size_t mm_lds_bytes(int gps, int ks, int tt) {
    return tt == 1 ? (size_t)ks * mm_wave_lds<FMT>(gps)
                   : (size_t)ks * 2 * mm_stage_bytes<FMT>() +
                         (size_t)ks * tt * (mm_wave_lds<FMT>(gps, tt) - mm_stage_bytes<FMT>());
}

template <int FMT, int NB, int GPS, int TT>
static int launch_mm_gps(const MmArgs &a, int nt1, hipStream_t stream) {
    if (ensure_lds_limit(reinterpret_cast<const void *>(&qgemv_mm_kernel<FMT, NB, GPS, TT>), kLdsBytes) != QG_OK)
        return QG_ERR_LAUNCH;
    hipLaunchKernelGGL((qgemv_mm_kernel<FMT, NB, GPS, TT>), dim3((a.nt0 + nt1) * a.ntok, a.G),
                       dim3(a.KS * TT * kWave), mm_lds_bytes<FMT>(GPS, a.KS, TT), stream, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

template <int FMT, int NB, int TT>
static int launch_mm_tt(const MmArgs &a, int nt1, hipStream_t stream) {
    switch (a.gps) {
        case 1: return launch_mm_gps<FMT, NB, 1, TT>(a, nt1, stream);
        case 2: return launch_mm_gps<FMT, NB, 2, TT>(a, nt1, stream);
        case 4: return launch_mm_gps<FMT, NB, 4, TT>(a, nt1, stream);
        case 8: return launch_mm_gps<FMT, NB, 8, TT>(a, nt1, stream);
        default: return QG_ERR_SHAPE;
    }
}

// K slices as mm_slices chooses them; with several 32-token tiles (prefill)
// TT tiles of Q8_0 share each slice's weight stage (at most 8 waves), so a
// row tile's weights are read once per TT x 32 tokens.
template <int FMT, int NB>
static int launch_mm(MmArgs &a, hipStream_t stream) {
    a.row_bytes = a.K / 256 * MmFmt<FMT>::parts * 16;
    a.groups = a.K / 256;
    const int nt1 = a.W1 ? (a.N1 + kMmRows - 1) / kMmRows : 0;
    a.nt0 = (a.N0 + kMmRows - 1) / kMmRows;
    const int ntok32 = (a.M + kMmTokens - 1) / kMmTokens;
    mm_slices(a.groups, (long)(a.nt0 + nt1) * a.G * ntok32, &a.KS, &a.gps);
    int tt = 1;
    if (FMT == QG_FMT_Q8_0)
        while (tt < 4 && 2 * tt <= ntok32 && a.KS * 2 * tt <= kMmMaxSlices &&
               mm_lds_bytes<FMT>(a.gps, a.KS, 2 * tt) <= (size_t)kLdsBytes)
            tt <<= 1;
    a.ntok = (ntok32 + tt - 1) / tt;
    if constexpr (FMT == QG_FMT_Q8_0) {
        if (tt == 4) return launch_mm_tt<FMT, NB, 4>(a, nt1, stream);
        if (tt == 2) return launch_mm_tt<FMT, NB, 2>(a, nt1, stream);
    }
    return launch_mm_tt<FMT, NB, 1>(a, nt1, stream);
}

int gemv_mm(int fmt, const uint8_t *W0, int N0, float *y0, const uint8_t *W1, int N1, float *y1, int K,
            const int8_t *qx, const float *dx, const int32_t *sx, int M, int G, hipStream_t stream) {
    clear_stale_error();
    MmArgs a{};
    a.W0 = W0;
    a.N0 = N0;
    a.y0 = y0;
    a.W1 = W1;
    a.N1 = N1;
    a.y1 = y1;
    a.K = K;
    a.qx = qx;
    a.dx = dx;
    a.sx = sx;
    a.M = M;
    a.G = G;
    // the unit of the one-token engine: Q4_K one superblock; Q8_0 4 blocks up
    // to K = 8192, else 8
    if (fmt == QG_FMT_Q4K) return launch_mm<QG_FMT_Q4K, 8>(a, stream);
    if (K <= 8192) return launch_mm<QG_FMT_Q8_0, 4>(a, stream);
    return launch_mm<QG_FMT_Q8_0, 8>(a, stream);
}

}  // namespace qg

extern "C" int qgemm_q8_0(const void *W, int N, int K, const int8_t *qx, const float *dx, int M, float *y,
                          void *stream) {
    if (!W || !qx || !dx || !y) return QG_ERR_NULL;
    if (N < 1 || M < 1 || M > QG_MAX_PREFILL_M) return QG_ERR_SHAPE;
    if (K < qg::kGroupWeights || K > QG_MAX_K || K % qg::kGroupWeights != 0) return QG_ERR_SHAPE;
    if (((uintptr_t)W | (uintptr_t)qx | (uintptr_t)dx | (uintptr_t)y) & 15) return QG_ERR_ALIGN;
    return qg::gemv_mm(QG_FMT_Q8_0, reinterpret_cast<const uint8_t *>(W), N, y, nullptr, 0, nullptr, K, qx, dx,
                       nullptr, M, 1, (hipStream_t)stream);
}
