// Device-side Q8 quantization of one 32-element block spread over 8 lanes.
#pragma once

#include "common.h"

namespace qg {

// Eight consecutive lanes (an aligned group of 8 within the wave) each hold 4
// consecutive values of one 32-block.  On return every lane of the group holds
// the block scale d and the block sum s; q are the lane's 4 quants.
//   amax = max |x|, d = amax / 127 (IEEE fp32 division, round to nearest),
//   q = rint(x / d) (round half to even) clamped to [-127, 127], 0 when d == 0.
// All lanes of the wave must execute this (it shuffles).
__device__ __forceinline__ void quantize_block_8lanes(const float v[4], int8_t q[4], float *d_out, int32_t *s_out) {
    float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    a = fmaxf(a, shfl_xor(a, 1));
    a = fmaxf(a, shfl_xor(a, 2));
    a = fmaxf(a, shfl_xor(a, 4));
    const float d = a / 127.0f;
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int qi = 0;
        if (d != 0.0f) {
            float r = rintf(v[i] / d);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            qi = (int)r;
        }
        q[i] = (int8_t)qi;
        s += qi;
    }
    s += shfl_xor(s, 1);
    s += shfl_xor(s, 2);
    s += shfl_xor(s, 4);
    *d_out = d;
    *s_out = s;
}

}  // namespace qg
