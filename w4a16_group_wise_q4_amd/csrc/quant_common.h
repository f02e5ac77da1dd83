// quant_common.h — device helpers shared by the quantize kernels (RTN and the MSE clip
// search): exact divisions, the rounding of small quotients, weight loads, group
// reductions.  All arithmetic is IEEE fp32 in the order written (includers compile with
// contraction off).
#pragma once

#include "q4_launch.h"

#pragma clang fp contract(off)

namespace q4q {

// x / d for d = 15 or 7 from the correctly rounded reciprocal and one FMA correction: equal to
// the IEEE quotient for every finite non-negative fp32 x (checked exhaustively).
template <int D>
__device__ __forceinline__ float div_const(float x) {
    constexpr float c = 1.0f / (float)D;
    const float q0 = x * c;
    const float r = __builtin_fmaf(-q0, (float)D, x);
    return __builtin_fmaf(r, c, q0);
}

// The quotient v / S for a 16-bit weight v and a stored fp16 scale S, given y = 1/S
// (correctly rounded): rounds to the same integer as the IEEE quotient wherever a group's
// weights can land (checked exhaustively over all fp16 scales and 16-bit weights), clamped
// to [-64, 64], which leaves every code unchanged.
__device__ __forceinline__ float quot16(float v, float S, float y) {
    const float q0 = v * y;
    const float r = __builtin_fmaf(-q0, S, v);
    return __builtin_amdgcn_fmed3f(__builtin_fmaf(r, y, q0), -64.0f, 64.0f);
}

// round-half-to-even of q (|q| <= 64) as an integer: the 1.5 * 2^23 addition
__device__ __forceinline__ int rne_small(float q) {
    return (int)(__builtin_bit_cast(uint32_t, q + 12582912.0f) - 0x4B400000u);
}

// One lane's E consecutive weights at byte offset off of the row resource (zeros past it).
template <int E, int DT>
__device__ __forceinline__ void load_slice(q4::rsrc r, uint32_t off, float (&v)[E]) {
    if constexpr (DT == 0) {
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            // bit-cast the whole vector, then read elements (see f32_bits)
            const q4::f32x4 t = __builtin_bit_cast(q4::f32x4, q4::buf_load_x4(r, (int)(off + 16u * i), 0));
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * i + j] = t[j];
        }
    } else {
        uint32_t words[E / 2];
        if constexpr (E >= 8) {
#pragma unroll
            for (int i = 0; i < E / 8; ++i) {
                const q4::u32x4 t = q4::buf_load_x4(r, (int)(off + 16u * i), 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) words[4 * i + j] = t[j];
            }
        } else {
            const q4::u32x2 t = q4::buf_load_x2(r, (int)off, 0);
            words[0] = t[0];
            words[1] = t[1];
        }
#pragma unroll
        for (int i = 0; i < E / 2; ++i) {
            if constexpr (DT == 2) {  // bf16: the upper half of an fp32
                v[2 * i] = __builtin_bit_cast(float, words[i] << 16);
                v[2 * i + 1] = __builtin_bit_cast(float, words[i] & 0xFFFF0000u);
            } else {                  // fp16
                v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(words[i] & 0xFFFFu));
                v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(words[i] >> 16));
            }
        }
    }
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }
__device__ __forceinline__ float xor_min(float v, int m) { return fminf(v, __shfl_xor(v, m, 64)); }

}  // namespace q4q
