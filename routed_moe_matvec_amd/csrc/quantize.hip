// Q8 activation quantization: the decode activation is quantized once and fed
// to every Q8 projection ("ROCm: restore DeepSeek V4 Flash decode performance
// and Q4 SSD streaming", antirez/ds4 PR 623, Summary).  Each 32-block keeps
// its fp32 scale and the sum of its quants, which the Q4_K min term needs
// (the Q8 quantizer with a block sum in "DeepSeek V4 Flash on Strix Halo",
// section on the quantized mat-vec profile).
#include "common.h"
#include "quantize_device.h"

namespace qg {

// 8 lanes per 32-element block, 4 consecutive fp32 values per lane (one
// 16-byte load), so a wave covers 8 blocks = 1 KiB of x in one coalesced load.
__global__ __launch_bounds__(256) void quantize_act_q8_kernel(const float *__restrict__ x, int nblocks,
                                                              int8_t *__restrict__ qx, float *__restrict__ dx,
                                                              int32_t *__restrict__ sx) {
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int blk = gid >> 3;
    const int part = gid & 7;
    const bool valid = blk < nblocks;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *reinterpret_cast<const float4 *>(x + (size_t)blk * 32 + part * 4);
    float vals[4] = {v.x, v.y, v.z, v.w};
    int8_t q[4];
    float d;
    int32_t s;
    quantize_block_8lanes(vals, q, &d, &s);
    if (valid) {
        uint32_t packed = (uint32_t)(uint8_t)q[0] | ((uint32_t)(uint8_t)q[1] << 8) |
                          ((uint32_t)(uint8_t)q[2] << 16) | ((uint32_t)(uint8_t)q[3] << 24);
        *reinterpret_cast<uint32_t *>(qx + (size_t)blk * 32 + part * 4) = packed;
        if (part == 0) {
            dx[blk] = d;
            sx[blk] = s;
        }
    }
}

}  // namespace qg

extern "C" int quantize_act_q8(const float *x, int M, int K, int8_t *qx, float *dx, int32_t *sx, void *stream) {
    if (!x || !qx || !dx || !sx) return QG_ERR_NULL;
    if (M < 1 || K < 32 || K % 32 != 0) return QG_ERR_SHAPE;
    if (((uintptr_t)x | (uintptr_t)qx | (uintptr_t)dx | (uintptr_t)sx) & 15) return QG_ERR_ALIGN;
    const long long nblocks = (long long)M * (K / 32);
    if (nblocks * 8 > 0x7fffffffLL) return QG_ERR_SHAPE;
    const int threads = 256;
    const int grid = (int)((nblocks * 8 + threads - 1) / threads);
    qg::clear_stale_error();
    hipLaunchKernelGGL(qg::quantize_act_q8_kernel, dim3(grid), dim3(threads), 0, (hipStream_t)stream, x,
                       (int)nblocks, qx, dx, sx);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}
