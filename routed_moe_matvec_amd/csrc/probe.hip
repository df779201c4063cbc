// Streaming-read diagnostic: the HBM read rate that the decode mat-vecs are
// measured against.  It reads a buffer once with the access pattern of the
// mat-vec engine (each wave one burst of consecutive 16-byte non-temporal
// loads, 1 KiB per instruction) and does no other work, so its time for a
// given byte count is the floor a one-pass weight stream can reach on this
// part, launch and drain included.
#include "common.h"

namespace qg {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int L>  // KiB read by one wave (L loads in flight per lane)
__global__ __launch_bounds__(1024) void stream_read_kernel(const u32x4_t *__restrict__ p, size_t n16,
                                                            uint32_t *__restrict__ wg_xor) {
    __shared__ uint32_t part[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t base = ((size_t)blockIdx.x * (blockDim.x >> 6) + wave) * 64 * L;
    u32x4_t v[L];
    // every lane issues every load (indexes past the end re-read the last
    // chunk), so the burst is one run of loads; those values then count as 0
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const size_t idx = base + (size_t)i * 64 + lane;
        v[i] = __builtin_nontemporal_load(p + (idx < n16 ? idx : n16 - 1));
    }
#pragma unroll
    for (int i = 0; i < L; ++i)
        if (base + (size_t)i * 64 + lane >= n16) v[i] = u32x4_t{0, 0, 0, 0};
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r ^= part[w];
        wg_xor[blockIdx.x] = r;
    }
}

template <int L>
static int launch_stream_read(const void *buf, size_t n16, int waves, uint32_t *wg_xor, hipStream_t st) {
    const size_t per_wg = (size_t)waves * 64 * L;
    const size_t grid = (n16 + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(stream_read_kernel<L>, dim3((unsigned)grid), dim3(waves * 64), 0, st,
                       reinterpret_cast<const u32x4_t *>(buf), n16, wg_xor);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // namespace qg

extern "C" size_t qg_stream_read_groups(size_t bytes, int chunk_kib, int waves) {
    if (bytes == 0 || bytes % 16 || waves < 1 || waves > 16) return 0;
    if (chunk_kib != 1 && chunk_kib != 2 && chunk_kib != 4 && chunk_kib != 8 && chunk_kib != 16) return 0;
    const size_t per_wg = (size_t)waves * 1024 * chunk_kib;
    const size_t grid = (bytes + per_wg - 1) / per_wg;
    return grid <= 0x7fffffffu ? grid : 0;
}

extern "C" int qg_stream_read(const void *buf, size_t bytes, int chunk_kib, int waves, uint32_t *wg_xor,
                              size_t wg_xor_len, void *stream) {
    if (!buf || !wg_xor) return QG_ERR_NULL;
    const size_t groups = qg_stream_read_groups(bytes, chunk_kib, waves);
    if (groups == 0 || wg_xor_len < groups) return QG_ERR_SHAPE;
    if (((uintptr_t)buf & 15) || ((uintptr_t)wg_xor & 3)) return QG_ERR_ALIGN;
    const size_t n16 = bytes / 16;
    hipStream_t st = (hipStream_t)stream;
    switch (chunk_kib) {
        case 1: return qg::launch_stream_read<1>(buf, n16, waves, wg_xor, st);
        case 2: return qg::launch_stream_read<2>(buf, n16, waves, wg_xor, st);
        case 4: return qg::launch_stream_read<4>(buf, n16, waves, wg_xor, st);
        case 8: return qg::launch_stream_read<8>(buf, n16, waves, wg_xor, st);
        default: return qg::launch_stream_read<16>(buf, n16, waves, wg_xor, st);
    }
}
