// gemv.hip — decode W4A16 linear layer, m <= 16, for gfx950.
//
//   y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (u[n][k] - z[n][g])
//
// Path A of "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)"
// (§Kernel이 없으면 압축 이점이 사라진다): packed INT4 weights are loaded, dequantized
// in registers and multiplied with higher-precision (fp32) accumulation.  Decode is
// bandwidth-bound (§Batch와 Context에 따라 속도가 달라진다), so the kernel is built
// around streaming the packed weights once at HBM speed.
//
// Mapping.  A wave owns a tile of 16 output rows.  Lane l handles row n0 + l%16 and
// k-slot block c = l/16 of a 16x16x32 MFMA: the 16 rows are the MFMA's N columns, the
// (zero-padded) activation rows are its M rows, so m = 1..16 costs the same.  A
// workgroup of S waves covers the whole K range of one row tile (wave w takes a
// contiguous slice of 128-column units); partial tiles are summed through LDS, so the
// result is written once, without atomics, in a fixed order.
//
// Loads.  Per group and lane, G/32 consecutive packed words (one dwordx4 for g = 128):
// lane block c holds words [GW*h + LW*c, +LW) of a group of GW = g/8 words, so the 32
// k-slots of each MFMA lie in one group and the per-group scale can be applied to the
// MFMA result.
//
// Dequantization.  bf16 activations: a nibble OR-ed into the mantissa of 128.0 gives
// the exact bf16 value 128 + u (one AND-OR per two weights).  The offset is removed per
// group with a second MFMA whose weight operand is the constant 128 + z (also exact in
// bf16):
//   sum x(u - z) = D - C,   D = sum x(128 + u),  C = sum x(128 + z).
// Where every code of a group equals its zero point (an all-zero group), D and C are the
// same computation on the same operands, so the group contributes exactly zero.
// fp16 activations: 1024 + u in fp16 minus (1024 + z) with one packed fp16 subtraction
// gives the exact u - z.  Either way products are exact and sums are fp32.
#include "q4_device.h"

namespace {

constexpr int kMaxWaves = 8;

template <int G, bool SYM, bool XF16>
__global__ __launch_bounds__(512) void gemv_kernel(const uint16_t* __restrict__ x, int M,
                                                   const uint32_t* __restrict__ qweight,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint32_t* __restrict__ zeros, int N,
                                                   int K, float* __restrict__ y) {
    constexpr int GW = G / 8;   // packed words per group
    constexpr int LW = G / 32;  // words per lane per group (one MFMA per word)
    constexpr int NH = 4 / LW;  // groups per 128-column unit
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int S = blockDim.x >> 6;
    const int col = lane & 15;
    const int c = lane >> 4;
    const int n_real = blockIdx.x * 16 + col;
    const int n = n_real < N ? n_real : N - 1;  // rows past N load row N-1, store nothing
    const int KW = K / 8;
    const int n_groups = K / G;
    const int zwords = (n_groups + 7) >> 3;
    const int units = (K + 127) / 128;
    const int u0 = (int)((int64_t)wave * units / S);
    const int u1 = (int)((int64_t)(wave + 1) * units / S);
    const uint32_t* qrow = qweight + (int64_t)n * KW;
    const uint16_t* xrow = x + (int64_t)col * K;
    const bool xvalid = col < M;

    q4::f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    for (int u = u0; u < u1; ++u) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int wbase = u * 16 + GW * h;  // first packed word of this group
            if (wbase >= KW) break;
            const int gidx = wbase / GW;
            uint32_t wd[LW];
            if constexpr (LW == 4) {
                q4::u32x4 t = *reinterpret_cast<const q4::u32x4*>(qrow + wbase + 4 * c);
                wd[0] = t[0]; wd[1] = t[1]; wd[2] = t[2]; wd[3] = t[3];
            } else if constexpr (LW == 2) {
                q4::u32x2 t = *reinterpret_cast<const q4::u32x2*>(qrow + wbase + 2 * c);
                wd[0] = t[0]; wd[1] = t[1];
            } else {
                wd[0] = qrow[wbase + c];
            }
            q4::u32x4 xa[LW];
#pragma unroll
            for (int a = 0; a < LW; ++a) {
                if (xvalid)
                    xa[a] = q4::pair_perm(
                        *reinterpret_cast<const q4::u32x4*>(xrow + 8 * (wbase + LW * c + a)));
                else
                    xa[a] = q4::u32x4{0u, 0u, 0u, 0u};
            }
            const float s = q4::f16_bits_to_float(scales[(int64_t)n * n_groups + gidx]);
            int z = 8;
            if constexpr (!SYM)
                z = (int)((zeros[(int64_t)n * zwords + (gidx >> 3)] >> (4 * (gidx & 7))) & 0xFu);
            q4::f32x4 d = {0.f, 0.f, 0.f, 0.f};
            if constexpr (XF16) {
                const _Float16 b = (_Float16)(1024 + z);
                const q4::f16x2 bias = {b, b};
#pragma unroll
                for (int a = 0; a < LW; ++a) d = q4::mfma_f16(xa[a], q4::decode_f16_exact(wd[a], bias), d);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += s * d[i];
            } else {
                const uint32_t zb = (0x4300u | (uint32_t)z) * 0x00010001u;  // bf16 (128+z) x2
                const q4::u32x4 zop = {zb, zb, zb, zb};
                q4::f32x4 dc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int a = 0; a < LW; ++a) {
                    d = q4::mfma_bf16(xa[a], q4::decode_bf16_biased(wd[a]), d);
                    dc = q4::mfma_bf16(xa[a], zop, dc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += s * (d[i] - dc[i]);
            }
        }
    }

    __shared__ q4::f32x4 red[kMaxWaves][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && n_real < N) {
        q4::f32x4 t = red[0][lane];
        for (int w = 1; w < S; ++w) {
            const q4::f32x4 r = red[w][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] += r[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * c + i;
            if (m < M) y[(int64_t)m * N + n_real] = t[i];
        }
    }
}

template <int G, bool SYM>
hipError_t launch(const void* x, int xd, int m, const uint32_t* qw, const uint16_t* sc,
                  const uint32_t* zr, int n, int k, float* y, hipStream_t st, const char** kname) {
    const int units = (k + 127) / 128;
    const int waves = units < kMaxWaves ? units : kMaxWaves;
    const dim3 grid((unsigned)((n + 15) / 16)), block(64 * waves);
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
    if (xd == 1) {
        *kname = "q4_gemv_mfma_f16";
        hipLaunchKernelGGL((gemv_kernel<G, SYM, true>), grid, block, 0, st, xp, m, qw, sc, zr, n, k, y);
    } else {
        *kname = "q4_gemv_mfma_bf16";
        hipLaunchKernelGGL((gemv_kernel<G, SYM, false>), grid, block, 0, st, xp, m, qw, sc, zr, n, k, y);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t q4k_gemv(const void* x, int x_dtype, int m, const uint32_t* qweight,
                    const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k, int g,
                    int sym, float* y, hipStream_t stream, const char** kname) {
    const int ni = (int)n, ki = (int)k;
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 65: return launch<32, true>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 128: return launch<64, false>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 129: return launch<64, true>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, stream, kname);
    case 256: return launch<128, false>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, stream, kname);
    default: return launch<128, true>(x, x_dtype, m, qweight, scales, zeros, ni, ki, y, stream, kname);
    }
}
