// q4_device.h — device-side helpers shared by the gfx950 kernels of libq4.
//
// Operand types for the CDNA4 16x16x32 MFMA, the exponent-bias nibble decoders, raw
// buffer loads and the decode GEMV's kernel argument types.  Everything here is specific
// to gfx950 (wave64, v_mfma_f32_16x16x32_{bf16,f16}).  The host-side launchers are
// declared in q4_launch.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- MFMA wrappers
// D(16x16, fp32) += A(16x32) * B(32x16).  Lane l supplies row l%16 of A and column l%16
// of B for k-slot block l/16 (8 values each, same slot order in A and B), and receives
// D[4*(l/16) + i][l%16] in element i of the result.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- nibble decoders
// A packed word holds the codes of 8 consecutive columns, column i in bits 4i..4i+3.
// Decoded pairs come out as (column i, column i+4) in one 32-bit register, i = 0..3, so
// operand element 2i is column i and element 2i+1 is column i+4.  The activation operand
// is permuted the same way (pair_perm below).

// A constant held in a VGPR the optimizer cannot see through.  gfx9 VOP3 encodings take no
// literal operand, so (a & K1) | K2 with literal K1, K2 becomes two VOP2 ops; with both
// constants in registers it is a single v_and_or_b32.
__device__ __forceinline__ uint32_t vreg_const(uint32_t k) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(k));
    return r;
}

// bf16 exponent bias: 0x4300 is 128.0 with a zero 7-bit mantissa, so OR-ing a nibble into
// the low mantissa bits gives exactly 128 + u.  mask = 0x000F000F, bias = 0x43004300 (in
// registers, see vreg_const): 3 shifts + 4 v_and_or_b32 per word.
__device__ __forceinline__ u32x4 decode_bf16_biased(uint32_t w, uint32_t mask, uint32_t bias) {
    u32x4 r;
    r[0] = (w & mask) | bias;
    r[1] = ((w >> 4) & mask) | bias;
    r[2] = ((w >> 8) & mask) | bias;
    r[3] = ((w >> 12) & mask) | bias;
    return r;
}

// fp16 exponent bias: 0x6400 is 1024.0 with a zero 10-bit mantissa -> 1024 + u; then a
// packed fp16 subtraction of (1024 + z) leaves the exact small integer u - z.
__device__ __forceinline__ u32x4 decode_f16_exact(uint32_t w, f16x2 bias) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t t = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
        f16x2 v = __builtin_bit_cast(f16x2, t) - bias;
        r[i] = __builtin_bit_cast(uint32_t, v);
    }
    return r;
}

// Activation operand in the decoder's slot order: from 8 consecutive 16-bit values
// x0..x7 (four words, natural order) build pairs (x_i, x_{i+4}).
__device__ __forceinline__ u32x4 pair_perm(u32x4 x) {
    u32x4 r;
    // v_perm_b32 selector: bytes of {src0 (4..7), src1 (0..3)}; pick low/high halves.
    r[0] = __builtin_amdgcn_perm(x[2], x[0], 0x05040100u);  // (x0, x4)
    r[1] = __builtin_amdgcn_perm(x[2], x[0], 0x07060302u);  // (x1, x5)
    r[2] = __builtin_amdgcn_perm(x[3], x[1], 0x05040100u);  // (x2, x6)
    r[3] = __builtin_amdgcn_perm(x[3], x[1], 0x07060302u);  // (x3, x7)
    return r;
}

// Bits of an fp32 value.  Callers pass plain floats: with this compiler, bit-casting an
// element v[i] of an ext_vector_type (directly or after inlining, when v is updated element
// by element) has produced element 0 for every i.
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float f16_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- raw buffer loads
// A buffer resource (V#) in SGPRs: 64-bit base, byte size; the gfx9-family fourth word.
// Raw loads take a per-lane byte offset and a wave-uniform byte offset; any access whose
// offset reaches past num_bytes returns zero instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc make_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                             kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load_x4(rsrc r, int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 buf_load_x2(rsrc r, int voff, int soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_load_x1(rsrc r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_load_u16(rsrc r, int voff, int soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

}  // namespace q4

// ---------------------------------------------------------------- decode GEMV arguments
namespace q4 {
constexpr int kMaxGroup = 8;
// One problem of a grouped decode launch (y = x . x_hat^T); tile0 is filled by the launcher.
struct GemvProblem {
    const void* x;
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* zeros;
    void* y;  // fp32, fp16 or bf16 elements (GemvBatch::ydt)
    int n;
    int tile0;
};
// The problems of one decode launch (a single one, or several sharing m, k, g and dtype):
// workgroups [p[i].tile0, p[i+1].tile0) serve problem i.  ydt: the element type of every
// y (0 fp32, 1 fp16, 2 bf16; the q4_dtype codes).
struct GemvBatch {
    GemvProblem p[kMaxGroup];
    int count;
    int ydt;
};

// ---------------------------------------------------------------- output epilogue
// y elements: fp32 as accumulated, or rounded to nearest even to fp16 / bf16 (the output
// epilogue of a layer that hands 16-bit activations on).
__device__ __forceinline__ uint32_t y_bytes(int ydt) { return ydt == 0 ? 4u : 2u; }
__device__ __forceinline__ uint16_t to_y16(float v, int ydt) {
    if (ydt == 1) return __builtin_bit_cast(uint16_t, (_Float16)v);
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}
// One y element at byte offset off of resource ry (an offset past the resource stores nothing).
__device__ __forceinline__ void store_y(rsrc ry, uint32_t off, float v, int ydt) {
    if (ydt == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ry, (int)off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16(to_y16(v, ydt), ry, (int)off, 0, 0);
}
// One y element at index i of a plain pointer.
__device__ __forceinline__ void store_y(void* y, int64_t i, float v, int ydt) {
    if (ydt == 0)
        reinterpret_cast<float*>(y)[i] = v;
    else
        reinterpret_cast<uint16_t*>(y)[i] = to_y16(v, ydt);
}
}  // namespace q4
