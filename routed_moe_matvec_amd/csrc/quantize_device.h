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
// The 8-lane max and sum use DPP: quad permutations (lane ^ 1, lane ^ 2), then
// the half-row mirror, which reaches the other quad once every lane of a quad
// holds the quad's value (max and integer add are exact, so any order gives
// the same result).
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float max8(float a) {
    a = fmaxf(a, __builtin_bit_cast(float, dpp_i32<0xB1>(__builtin_bit_cast(int, a))));
    a = fmaxf(a, __builtin_bit_cast(float, dpp_i32<0x4E>(__builtin_bit_cast(int, a))));
    return fmaxf(a, __builtin_bit_cast(float, dpp_i32<0x141>(__builtin_bit_cast(int, a))));
}
__device__ __forceinline__ int sum8(int s) {
    s += dpp_i32<0xB1>(s);
    s += dpp_i32<0x4E>(s);
    return s + dpp_i32<0x141>(s);
}

__device__ __forceinline__ void quantize_block_8lanes(const float v[4], int8_t q[4], float *d_out, int32_t *s_out) {
    float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    a = max8(a);
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
    s = sum8(s);
    *d_out = d;
    *s_out = s;
}

// SiLU, z * sigmoid(z), as z / (1 + e^-z) in fp32 (expf and a correctly
// rounded division): the one definition every kernel that forms
// h = silu(g) * v uses, so their h values agree bit for bit.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace qg
