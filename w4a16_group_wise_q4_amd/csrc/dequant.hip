// dequant.hip — full dequantization of the packed format (path B of
// "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)",
// §Kernel이 없으면 압축 이점이 사라진다): x_hat = S (u - z), the dequantizer of
// §Affine Quantization, with z = 8 for symmetric codes.
//
// One thread per packed word (8 weights).  S (11 significant bits) times u - z (at most
// 5 bits) is exact in fp32; fp16 / bf16 outputs are one round-to-nearest-even of it.
#include "q4_launch.h"

namespace {

template <int G, bool SYM, int OUT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ qweight,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ zeros,
                                                      int64_t k, int64_t words,
                                                      void* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= words) return;
    const int64_t kw = k / 8;
    const int64_t row = idx / kw;
    const int64_t col0 = (idx - row * kw) * 8;
    const int64_t n_groups = k / G;
    const int64_t gidx = col0 / G;
    const float S = q4::f16_bits_to_float(scales[row * n_groups + gidx]);
    int z = 8;
    if constexpr (!SYM) z = (int)((zeros[row * ((n_groups + 7) >> 3) + (gidx >> 3)] >> (4 * (gidx & 7))) & 0xFu);
    const uint32_t w = qweight[idx];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = S * (float)((int)((w >> (4 * i)) & 0xFu) - z);
    const int64_t o = row * k + col0;
    if constexpr (OUT == 0) {
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o);
        p[0] = make_float4(v[0], v[1], v[2], v[3]);
        p[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        q4::u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t lo, hi;
            if constexpr (OUT == 1) {
                lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
            } else {
                lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i + 1]);
            }
            r[i] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        *reinterpret_cast<q4::u32x4*>(reinterpret_cast<uint16_t*>(out) + o) = r;
    }
}

template <int G, bool SYM>
hipError_t launch(const uint32_t* qw, const uint16_t* sc, const uint32_t* zr, int64_t n,
                  int64_t k, void* out, int od, hipStream_t st, const char** kname) {
    const int64_t words = n * (k / 8);
    const dim3 grid((unsigned)((words + 255) / 256)), block(256);
    static const char* names[3] = {"q4_dequant_f32", "q4_dequant_f16", "q4_dequant_bf16"};
    *kname = names[od];
    if (od == 0)
        hipLaunchKernelGGL((dequant_kernel<G, SYM, 0>), grid, block, 0, st, qw, sc, zr, k, words, out);
    else if (od == 1)
        hipLaunchKernelGGL((dequant_kernel<G, SYM, 1>), grid, block, 0, st, qw, sc, zr, k, words, out);
    else
        hipLaunchKernelGGL((dequant_kernel<G, SYM, 2>), grid, block, 0, st, qw, sc, zr, k, words, out);
    return q4k_launched(*kname);
}

}  // namespace

hipError_t q4k_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                       int64_t n, int64_t k, int g, int sym, void* out, int out_dtype,
                       hipStream_t stream, const char** kname) {
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(qweight, scales, zeros, n, k, out, out_dtype, stream, kname);
    case 65: return launch<32, true>(qweight, scales, zeros, n, k, out, out_dtype, stream, kname);
    case 128: return launch<64, false>(qweight, scales, zeros, n, k, out, out_dtype, stream, kname);
    case 129: return launch<64, true>(qweight, scales, zeros, n, k, out, out_dtype, stream, kname);
    case 256: return launch<128, false>(qweight, scales, zeros, n, k, out, out_dtype, stream, kname);
    default: return launch<128, true>(qweight, scales, zeros, n, k, out, out_dtype, stream, kname);
    }
}
