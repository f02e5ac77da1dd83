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

// One group's quantizer and codes.  The G/E lanes of a group (aligned, consecutive lanes)
// hold E consecutive weights each in v; on return every lane of the group has the stored
// fp16 scale s16, the zero point zi (8 when symmetric: the code offset) and its E codes
// packed 8 per word in natural order.  The arithmetic of the RTN quantizer: zero-extended
// [min, max] (asymmetric) or max |w| (symmetric) over the group, IEEE fp32 in the order
// written, the scale rounded to fp32 and then to fp16.  The statistics are exact, so how
// the group is split over lanes does not change any result.
template <int G, bool SYM, int DT, int E = G / 8>
__device__ __forceinline__ void quant_group(const float (&v)[E], uint16_t& s16_out, int& zi_out,
                                            uint32_t (&packed)[(E + 7) / 8]) {
    constexpr int LPG = G / E;  // lanes per group: 2, 4, 8 or 16
    static_assert(LPG >= 2 && LPG <= 16 && (LPG & (LPG - 1)) == 0, "lanes per group");
    // group statistics: zero-extended [min, max] (asymmetric) or max |w| (symmetric)
    float s, x_min = 0.0f, x_max = 0.0f;
    if constexpr (SYM) {
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
        for (int m = 1; m < LPG; m <<= 1) amax = xor_max(amax, m);
        s = div_const<7>(amax);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            x_min = fminf(x_min, v[e]);
            x_max = fmaxf(x_max, v[e]);
        }
#pragma unroll
        for (int m = 1; m < LPG; m <<= 1) {
            x_min = xor_min(x_min, m);
            x_max = xor_max(x_max, m);
        }
        s = div_const<15>(x_max - x_min);
    }
    // stored fp16 scale: s is rounded to fp32 first, then to fp16 (round-to-nearest-
    // even both times).  The empty asm pins s as an fp32 value: otherwise the compiler
    // folds the last FMA of the division and the conversion into one fp16-rounding
    // instruction, which differs from the double rounding on fp16 ties.
    asm volatile("" : "+v"(s));
    uint16_t s16 = __builtin_bit_cast(uint16_t, (_Float16)s);
    if ((s16 & 0x7FFFu) == 0) s16 = 0x3C00u;
    if (s16 == 0x7C00u) s16 = 0x7BFFu;
    const float S = (float)__builtin_bit_cast(_Float16, s16);

#pragma unroll
    for (int j = 0; j < (E + 7) / 8; ++j) packed[j] = 0;
    int zi = 8;
    if constexpr (DT == 0) {
        // fp32 weights: IEEE quotients
        float zf = 0.0f;
        if constexpr (!SYM) zf = fminf(fmaxf(rintf(-x_min / S), 0.0f), 15.0f);
        constexpr float q_min = SYM ? -8.0f : 0.0f;
        constexpr float q_max = SYM ? 7.0f : 15.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float qf = fminf(fmaxf(rintf(v[e] / S) + zf, q_min), q_max);
            packed[e / 8] |= (uint32_t)((int)qf + (SYM ? 8 : 0)) << (4 * (e % 8));
        }
        if constexpr (!SYM) zi = (int)zf;
    } else {
        // 16-bit weights: correctly rounded reciprocal once, corrected quotients;
        // -x_min is itself one of the group's weights (or 0)
        const float y = 1.0f / S;
        if constexpr (!SYM) zi = min(max(rne_small(quot16(-x_min, S, y)), 0), 15);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int u = min(max(rne_small(quot16(v[e], S, y)) + zi, 0), 15);
            packed[e / 8] |= (uint32_t)u << (4 * (e % 8));
        }
    }
    s16_out = s16;
    zi_out = zi;
}

}  // namespace q4q
