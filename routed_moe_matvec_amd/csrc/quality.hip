// Q8_0 weights x fp32 activation with no activation quantization: the
// exact-activation product that prequantized decode replaced and that stays
// available as its A/B comparator ("ROCm: restore DeepSeek V4 Flash decode
// performance and Q4 SSD streaming", antirez/ds4 PR 623, Summary: the fp32
// shared-x path, kept for the quality mode).
//
//   y[m, n] = sum_b dw[n, b] * sum_{i<32} qw[n, b, i] * x[m, 32b + i]
//
// The weights go through the same tile engine as the Q8 path (a wave streams
// a tile of whole rows with 16-byte non-temporal loads, writes it to a private
// LDS buffer and each lane takes one unit of 4 or 8 blocks back).  The
// activation is staged per workgroup as fp32 records, one per unit, padded to
// an odd multiple of 4 dwords so lanes reading different units hit disjoint
// banks.  Per block, 32 fp32 fmas in element order give the block sum, then
// acc = fma(dw, block sum, acc) in block order, then the fixed xor butterfly
// over the row's lanes.
#include "common.h"
#include "gemv_device.h"

namespace qg {

constexpr int kFxMaxWaves = 8;
constexpr int kFxActBudget = 64 * 1024;  // LDS for staged tokens, when the tiles leave room

template <int NB>
struct FxRec {
    static constexpr int dwords = 32 * NB + 4;  // 132 or 260: odd multiples of 4
};

struct FxArgs {
    const uint8_t *W;
    const float *x;
    float *y;
    int N, K, M;
    TileGeom tg;
    int ntiles, waves, mt;
};

template <int NB>
__device__ __forceinline__ float unit_dot_fx(const uint32_t (&w)[17 * NB / 2], const float *rec) {
    const float4 *xv = reinterpret_cast<const float4 *>(rec);
    float acc = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int byte0 = 34 * b;
        const int dw0 = byte0 / 4;
        const uint32_t sbits = (b & 1) ? (w[dw0] >> 16) : (w[dw0] & 0xffffu);
        const float dwt = half_bits_to_float(sbits);
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t wq = (b & 1) ? w[(byte0 + 2) / 4 + k] : align_bytes(w[dw0 + k + 1], w[dw0 + k], 2);
            const float4 v = xv[8 * b + k];
            s = fmaf_exact((float)(int8_t)(wq & 0xffu), v.x, s);
            s = fmaf_exact((float)(int8_t)((wq >> 8) & 0xffu), v.y, s);
            s = fmaf_exact((float)(int8_t)((wq >> 16) & 0xffu), v.z, s);
            s = fmaf_exact((float)(int8_t)(wq >> 24), v.w, s);
        }
        acc = fmaf_exact(dwt, s, acc);
        // keep the next block's 32 activation reads below this block's fmas, so
        // only one block of activations is live in registers (an empty asm that
        // takes acc and clobbers memory: it orders, and emits no instruction)
        asm volatile("" : "+v"(acc)::"memory");
    }
    return acc;
}

template <int NB>
__global__ __launch_bounds__(kFxMaxWaves *kWave) void qgemv_fx_kernel(FxArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using U = Unit<QG_FMT_Q8_0, NB>;
    constexpr int REC = FxRec<NB>::dwords;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    uint8_t *lw = smem + wave * TileSize<U>::lds;
    float *lact = reinterpret_cast<float *>(smem + a.waves * TileSize<U>::lds);
    const TileGeom tg = a.tg;
    const int tile = blockIdx.x * a.waves + wave;
    const int r = lane >> tg.lsh, g = lane & (tg.lpr - 1);
    const int row = tile * tg.rpt + r;
    const bool live = tile < a.ntiles;  // uniform over the wave
    const bool valid = live && g < tg.upr && row < a.N;
    const int cpt = a.K / 4;  // float4 chunks per token
    auto stage = [&](int m0, int mtc) {
        for (int c = threadIdx.x; c < mtc * cpt; c += blockDim.x) {
            const int mm = c / cpt, wc = c - mm * cpt;
            const int un = (4 * wc) / U::weights, off = 4 * wc - un * U::weights;
            const float4 v = reinterpret_cast<const float4 *>(a.x + (size_t)(m0 + mm) * a.K)[wc];
            *reinterpret_cast<float4 *>(lact + (size_t)(mm * tg.upr + un) * REC + off) = v;
        }
    };
    UnitRegs<U> u;
    auto dots = [&](int m0, int mtc) {
        for (int mm = 0; mm < mtc; ++mm) {
            // the weights' int8 -> fp32 conversions stay inside the token loop
            // (hoisted, they would hold 32*NB registers)
#pragma unroll
            for (int i = 0; i < U::dwords; ++i) asm volatile("" : "+v"(u.w[i]));
            float p = valid ? unit_dot_fx<NB>(u.w, lact + (size_t)(mm * tg.upr + g) * REC) : 0.0f;
            p = row_reduce(p, tg.lpr);
            if (valid && g == 0) a.y[(size_t)(m0 + mm) * a.N + row] = p;
        }
    };
    // first chunk of tokens: the weight tile is loaded once, before the staging
    {
        TileRegs<U> ra;
        if (live) load_tile<U>(a.W, a.N, tg, tile, ra);
        const int mtc = min(a.mt, a.M);
        stage(0, mtc);
        lds_barrier();
        if (live) {
            tile_to_unit<U>(ra, lw, r * tg.upr + g, valid, u);
            dots(0, mtc);
        }
    }
    for (int m0 = a.mt; m0 < a.M; m0 += a.mt) {
        const int mtc = min(a.mt, a.M - m0);
        lds_barrier();  // every wave is done with the previous tokens
        stage(m0, mtc);
        lds_barrier();
        if (live) dots(m0, mtc);
    }
}

template <int NB>
static int launch_fx(FxArgs &a, hipStream_t stream) {
    using U = Unit<QG_FMT_Q8_0, NB>;
    a.tg = make_tile_geom<U>(a.K);
    a.ntiles = (a.N + a.tg.rpt - 1) / a.tg.rpt;
    const size_t per_token = (size_t)a.tg.upr * FxRec<NB>::dwords * 4;
    const int cus = device_cu_count();
    a.waves = kFxMaxWaves;
    while (a.waves > 1 && (a.ntiles < a.waves * cus || a.waves * (size_t)TileSize<U>::lds + per_token > kLdsBytes))
        a.waves >>= 1;
    const size_t tiles_lds = (size_t)a.waves * TileSize<U>::lds;
    const size_t room = kLdsBytes - tiles_lds;
    const size_t budget = room < (size_t)kFxActBudget ? room : (size_t)kFxActBudget;
    a.mt = (int)(budget / per_token);
    if (a.mt < 1) a.mt = 1;
    if (a.mt > a.M) a.mt = a.M;
    const size_t lds = tiles_lds + (size_t)a.mt * per_token;
    if (ensure_lds_limit(reinterpret_cast<const void *>(&qgemv_fx_kernel<NB>), kLdsBytes) != QG_OK)
        return QG_ERR_LAUNCH;
    const int grid = (a.ntiles + a.waves - 1) / a.waves;
    hipLaunchKernelGGL(qgemv_fx_kernel<NB>, dim3(grid), dim3(a.waves * kWave), lds, stream, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // namespace qg

extern "C" int qgemv_q8_0_quality(const void *W, int N, int K, const float *x, int M, float *y, void *stream) {
    if (!W || !x || !y) return QG_ERR_NULL;
    if (N < 1 || M < 1 || M > QG_MAX_M) return QG_ERR_SHAPE;
    if (K < qg::kGroupWeights || K > QG_MAX_K || K % qg::kGroupWeights != 0) return QG_ERR_SHAPE;
    if (((uintptr_t)W | (uintptr_t)x | (uintptr_t)y) & 15) return QG_ERR_ALIGN;
    qg::FxArgs a{};
    a.W = reinterpret_cast<const uint8_t *>(W);
    a.x = x;
    a.y = y;
    a.N = N;
    a.K = K;
    a.M = M;
    qg::clear_stale_error();
    if (K <= 8192) return qg::launch_fx<4>(a, (hipStream_t)stream);
    return qg::launch_fx<8>(a, (hipStream_t)stream);
}
