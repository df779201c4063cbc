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
                                                            uint32_t *__restrict__ burst_xor, size_t bursts) {
    const int lane = threadIdx.x & 63;
    const size_t burst = (size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const size_t base = burst * 64 * L;
    // every lane issues every load (indexes past the end re-read the last
    // chunk), so the burst is one run of loads; those values then count as 0
    u32x4_t v[L];
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
    // XOR over the wave in registers (no LDS, no barrier: each wave retires on its own)
    acc ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)acc, 0xB1, 0xF, 0xF, false);   // lane ^ 1
    acc ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)acc, 0x4E, 0xF, 0xF, false);   // lane ^ 2
    acc ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)acc, 0x141, 0xF, 0xF, false);  // other quad of 8
    acc ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)acc, 0x140, 0xF, 0xF, false);  // other 8 of 16
    acc ^= (uint32_t)__builtin_amdgcn_readlane((int)acc, 16) ^ (uint32_t)__builtin_amdgcn_readlane((int)acc, 32) ^
           (uint32_t)__builtin_amdgcn_readlane((int)acc, 48);
    if (burst_xor != nullptr && lane == 0 && burst < bursts) burst_xor[burst] = acc;
}

template <int L>
static int launch_stream_read(const void *buf, size_t n16, int waves, uint32_t *burst_xor, size_t bursts,
                              hipStream_t st) {
    const size_t grid = (bursts + waves - 1) / waves;
    hipLaunchKernelGGL(stream_read_kernel<L>, dim3((unsigned)grid), dim3(waves * 64), 0, st,
                       reinterpret_cast<const u32x4_t *>(buf), n16, burst_xor, bursts);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // namespace qg

extern "C" size_t qg_stream_read_bursts(size_t bytes, int chunk_kib) {
    if (bytes == 0 || bytes % 16) return 0;
    if (chunk_kib != 1 && chunk_kib != 2 && chunk_kib != 4 && chunk_kib != 8 && chunk_kib != 16) return 0;
    const size_t per = (size_t)1024 * chunk_kib;
    const size_t n = (bytes + per - 1) / per;
    return n <= ((size_t)1 << 36) ? n : 0;
}

extern "C" int qg_stream_read(const void *buf, size_t bytes, int chunk_kib, int waves, uint32_t *burst_xor,
                              size_t burst_xor_len, void *stream) {
    if (!buf) return QG_ERR_NULL;
    const size_t bursts = qg_stream_read_bursts(bytes, chunk_kib);
    if (bursts == 0 || waves < 1 || waves > 16 || (burst_xor && burst_xor_len < bursts)) return QG_ERR_SHAPE;
    if ((bursts + waves - 1) / waves > 0x7fffffffu) return QG_ERR_SHAPE;
    if (((uintptr_t)buf & 15) || ((uintptr_t)burst_xor & 3)) return QG_ERR_ALIGN;
    const size_t n16 = bytes / 16;
    hipStream_t st = (hipStream_t)stream;
    qg::clear_stale_error();
    switch (chunk_kib) {
        case 1: return qg::launch_stream_read<1>(buf, n16, waves, burst_xor, bursts, st);
        case 2: return qg::launch_stream_read<2>(buf, n16, waves, burst_xor, bursts, st);
        case 4: return qg::launch_stream_read<4>(buf, n16, waves, burst_xor, bursts, st);
        case 8: return qg::launch_stream_read<8>(buf, n16, waves, burst_xor, bursts, st);
        default: return qg::launch_stream_read<16>(buf, n16, waves, burst_xor, bursts, st);
    }
}
