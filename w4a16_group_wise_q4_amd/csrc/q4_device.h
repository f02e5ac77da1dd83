// q4_device.h — device-side helpers shared by the gfx950 kernels of libq4.
//
// Operand types for the CDNA4 16x16x32 MFMA, the exact nibble decoders, raw buffer loads
// and the decode GEMV's kernel argument types.  Everything here is specific
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
// A packed word holds the codes of 8 consecutive columns, column i in bits 4i..4i+3.  Both
// decoders return the exact small integers u - z (|u - z| <= 15 is exact in bf16 and fp16),
// so every MFMA product is exact and only the fp32 sums round: the error of a dot product
// is relative to sum |x| |u - z|, whatever the zero point.
//
// fp16: decoded pairs come out as (column i, column i+4) in one 32-bit register, i = 0..3,
// so operand element 2i is column i and element 2i+1 is column i+4; the activation operand
// is permuted the same way (pair_perm below).  bf16: natural column order (operand element
// j is column j), so the activations are used as loaded.

// A constant held in a VGPR the optimizer cannot see through.  gfx9 VOP3 encodings take no
// literal operand, so (a & K1) | K2 with literal K1, K2 becomes two VOP2 ops; with both
// constants in registers it is a single v_and_or_b32.
__device__ __forceinline__ uint32_t vreg_const(uint32_t k) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(k));
    return r;
}

// Per-group constant of decode_bf16_exact: 128 - z in every byte.
__device__ __forceinline__ uint32_t bf16_zero_bias(int z) { return 0x80808080u - (uint32_t)z * 0x01010101u; }

// bf16: the nibbles of the even columns (bytes of w & 0x0F0F0F0F) and of the odd columns
// (bytes of (w >> 4) & 0x0F0F0F0F) plus 128 - z give 128 + u - z in [113, 143] per byte,
// with no carry between bytes; XOR 0x80 turns each byte into the two's complement of
// u - z.  Each signed byte converts exactly to fp32 (v_cvt_f32_i32 with a sign-extended
// byte select), whose upper half is the exact bf16 value; one v_perm_b32 packs two of
// them.  zb = bf16_zero_bias(z).  7 integer ops, 8 conversions and 4 permutes per word.
__device__ __forceinline__ u32x4 decode_bf16_exact(uint32_t w, uint32_t zb) {
    const uint32_t ev = ((w & 0x0F0F0F0Fu) + zb) ^ 0x80808080u;         // columns 0, 2, 4, 6
    const uint32_t od = (((w >> 4) & 0x0F0F0F0Fu) + zb) ^ 0x80808080u;  // columns 1, 3, 5, 7
    u32x4 r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float e = (float)(int8_t)((ev >> (8 * b)) & 0xFF);
        const float o = (float)(int8_t)((od >> (8 * b)) & 0xFF);
        // upper halves: bytes 2, 3 of e (column 2b) then bytes 2, 3 of o (column 2b + 1)
        r[b] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, o), __builtin_bit_cast(uint32_t, e),
                                     0x07060302u);
    }
    return r;
}

// fp16 exponent bias: 0x6400 is 1024.0 with a zero 10-bit mantissa -> 1024 + u; then a
// packed fp16 subtraction of (1024 + z) leaves the exact small integer u - z.  mask =
// 0x000F000F and magic = 0x64006400 are passed in registers (vreg_const), so each pair is
// one v_and_or_b32 (after a shift) and one v_pk_add_f16: 11 instructions per word.
__device__ __forceinline__ u32x4 decode_f16_exact(uint32_t w, f16x2 bias, uint32_t mask, uint32_t magic) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t t = ((w >> (4 * i)) & mask) | magic;
        f16x2 v = __builtin_bit_cast(f16x2, t) - bias;
        r[i] = __builtin_bit_cast(uint32_t, v);
    }
    return r;
}

// ---------------------------------------------------------------- bf16 activations as fp16
// A bf16 value with exponent field e in [1, 254] (1.m * 2^(e-127), 8 significant bits)
// times 2^t is an exact normal fp16 value when e + t - 127 lies in [-14, 15].  So a set of
// bf16 values whose nonzero exponent fields span emin..emax converts exactly to fp16 after
// scaling by 2^xs, xs = 142 - emax, and a quarter of those values (2^(xs-4)) still does when
// emax - emin <= 25; zeros stay zero.  The decode tile kernel uses this to run bf16
// activations through the cheaper exact fp16 decode below (decode_f16_split), and scales
// its sums back by 2^-xs (exact barring fp32 overflow).

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Running per-half maximum of the magnitudes |b| and minimum of |b| - 1 (mod 2^16, so a
// zero magnitude gives 0xFFFF and never lowers it) of a register of two bf16 values.
// Magnitudes of floats order like their bit patterns.
__device__ __forceinline__ void bf16_mag_range(uint32_t b, u16x2& hi, u16x2& lo) {
    const u16x2 mag = __builtin_bit_cast(u16x2, b & 0x7FFF7FFFu);
    hi = __builtin_elementwise_max(hi, mag);
    lo = __builtin_elementwise_min(lo, mag - (u16x2){1, 1});
}

// Maximum of each 16-bit half over the 64 lanes of a wave (every lane gets the result):
// DPP within rows of 16, then the 16- and 32-lane swaps.
__device__ __forceinline__ uint32_t wave_max_u16x2(uint32_t v) {
    auto op = [](uint32_t a, uint32_t b) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                      __builtin_bit_cast(u16x2, b)));
    };
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(s16[0], s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(s32[0], s32[1]);
}

// Eight bf16 values (natural order, four registers) as the fp16 operand of
// decode_f16_split: pairs (x_i, x_{i+4}) times 2^xs for i = 0, 2 and times 2^(xs-4) for
// i = 1, 3.  Exact under the range condition above.
__device__ __forceinline__ u32x4 bf16_to_f16_split(u32x4 v, int xs) {
    auto cv = [](uint32_t a, uint32_t b, int t) {  // a, b: fp32 bit patterns of two bf16 values
        const float fa = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, a), t);
        const float fb = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, b), t);
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(fa, fb));
    };
    u32x4 r;
    r[0] = cv(v[0] << 16, v[2] << 16, xs);                      // (x0, x4)
    r[1] = cv(v[0] & 0xFFFF0000u, v[2] & 0xFFFF0000u, xs - 4);  // (x1, x5) / 16
    r[2] = cv(v[1] << 16, v[3] << 16, xs);                      // (x2, x6)
    r[3] = cv(v[1] & 0xFFFF0000u, v[3] & 0xFFFF0000u, xs - 4);  // (x3, x7) / 16
    return r;
}

// fp16 pair (1024 + v, 1024 + v) for an integer 0 <= v < 1024 (exact), built with integer
// operations: 1024.0 is 0x6400 and the mantissa's ulp there is 1.
__device__ __forceinline__ f16x2 f16_bias_pair(uint32_t v) {
    const uint32_t b = 0x6400u + v;
    return __builtin_bit_cast(f16x2, b | (b << 16));
}

// The exact fp16 decode in 9 instructions per word: the nibbles of columns 0/4 and 2/6 sit
// in the low mantissa bits (1024 + u), those of columns 1/5 and 3/7 four bits higher
// (1024 + 16u, exact too), so one shift serves all four pairs.  Subtracting 1024 + z and
// 1024 + 16z (bias_lo, bias_hi) leaves u - z and 16(u - z); the activations of the odd
// columns are staged divided by 16 to match (bf16_to_f16_split).  m_lo = 0x000F000F,
// m_hi = 0x00F000F0 and magic = 0x64006400 in registers (vreg_const).
__device__ __forceinline__ u32x4 decode_f16_split(uint32_t w, f16x2 bias_lo, f16x2 bias_hi,
                                                  uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
    const uint32_t w8 = w >> 8;
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, (w & m_lo) | magic) - bias_lo);
    r[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, (w & m_hi) | magic) - bias_hi);
    r[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, (w8 & m_lo) | magic) - bias_lo);
    r[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, (w8 & m_hi) | magic) - bias_hi);
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

// ---------------------------------------------------------------- launch record
// Every kernel launch the library enqueues is recorded (name, count) for the calling
// thread's current entry-point call; q4_last_kernels() and q4_last_launch_count() report
// the record of the last successful call.
void q4k_record(const char* name);
// After a single launch: the launch status, with the launch recorded under name if it
// succeeded.
inline hipError_t q4k_launched(const char* name) {
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) q4k_record(name);
    return e;
}

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
