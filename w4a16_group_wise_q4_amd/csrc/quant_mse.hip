// quant_mse.hip — MSE-optimal clip search + pack of W [n][k] into the canonical packed
// format, for gfx950.
//
// Method: the clipping threshold of "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache
// (7/10)" §Clipping Trade-off chosen to minimize the local reconstruction error, the
// MSE-optimal criterion argmin ||x - x_dq||^2 of "Quantization Algorithms 단권화"
// §MSE-optimal, applied per group (§Per-group).  Each group tries the clip ratios
// alpha_i = (20 - i) / 20, i = 0..10: the RTN quantizer of quant_pack.hip with the group's
// range scaled by alpha (asymmetric [alpha*min(x_min,0), alpha*max(x_max,0)], symmetric
// alpha*max|x|; weights outside saturate at the end codes).  A candidate's error is
// sum (x - S(q - z))^2 in IEEE fp64, each lane summing its g/8 consecutive weights in order
// and the 8 lanes of a group then adding pairwise, ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)).
// The first smallest error wins (alpha = 1, plain RTN, unless clipping strictly helps).
// The summation order is fixed so that the choice, an integer decided by floating point,
// is the same on every implementation that follows it.
//
// Work mapping as in quant_pack.hip: one wave = one row x 8 consecutive groups (one
// zero-point word), lane l holds E = g/8 consecutive weights of group l/8; persistent
// waves walk the (row, zero word) tasks.  The search is ALU-bound: per weight and
// candidate about a dozen fp32 and fp64 VALU operations.
#include "quant_common.h"

#pragma clang fp contract(off)

namespace {

using namespace q4q;

constexpr int kCandidates = 11;

// A candidate's stored scale, zero point and reciprocal for clip ratio alpha.
struct Cand {
    uint16_t s16;
    float S, y;
    int z;
};

template <bool SYM>
__device__ __forceinline__ Cand candidate(float alpha, float amax, float x_min, float x_max) {
    float s, lo = 0.0f;
    if constexpr (SYM) {
        s = div_const<7>(alpha * amax);
    } else {
        lo = alpha * x_min;
        const float hi = alpha * x_max;
        s = div_const<15>(hi - lo);
    }
    // fp32 first, then fp16 (both round-to-nearest-even): the empty asm keeps the compiler
    // from fusing the division's last FMA with the conversion into one rounding
    asm volatile("" : "+v"(s));
    uint16_t s16 = __builtin_bit_cast(uint16_t, (_Float16)s);
    if ((s16 & 0x7FFFu) == 0) s16 = 0x3C00u;
    if (s16 == 0x7C00u) s16 = 0x7BFFu;
    Cand c;
    c.s16 = s16;
    c.S = (float)__builtin_bit_cast(_Float16, s16);
    c.y = 1.0f / c.S;
    c.z = 0;
    if constexpr (!SYM) c.z = (int)fminf(fmaxf(rintf(-lo / c.S), 0.0f), 15.0f);
    return c;
}

// Code of weight v under candidate c, in the signed domain q (asym: [0,15], sym: [-8,7]).
template <bool SYM, int DT>
__device__ __forceinline__ int code(float v, const Cand& c) {
    constexpr int q_min = SYM ? -8 : 0, q_max = SYM ? 7 : 15;
    if constexpr (DT == 0) {
        const float qf = rintf(v / c.S) + (float)c.z;
        return (int)fminf(fmaxf(qf, (float)q_min), (float)q_max);
    } else {
        return min(max(rne_small(quot16(v, c.S, c.y)) + c.z, q_min), q_max);
    }
}

__device__ __forceinline__ double xor_add(double v, int m) {
    return v + __shfl_xor(v, m, 64);
}

template <int G, bool SYM, int DT>
__global__ __launch_bounds__(256) void quant_mse_kernel(const void* __restrict__ w, int n, int k,
                                                        uint32_t* __restrict__ qweight,
                                                        uint16_t* __restrict__ scales,
                                                        uint32_t* __restrict__ zeros) {
    constexpr int E = G / 8;
    constexpr uint32_t EB = DT == 0 ? 4 : 2;
    constexpr uint32_t kOff = 0xFFFFFFF0u;
    const int lane = threadIdx.x & 63;
    const int waves = (int)gridDim.x * (int)(blockDim.x >> 6);
    const int gw = (int)blockIdx.x * (int)(blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 3;
    const int t = lane & 7;
    const int n_groups = k / G;
    const int zwords = (n_groups + 7) >> 3;
    const int Z = zwords < waves ? zwords : waves;
    const int R = waves / Z < n ? waves / Z : n;
    const int r0 = gw / Z, z0 = gw - r0 * Z;
    if (r0 >= R) return;  // wave-uniform

    for (int row = r0; row < n; row += R) {
        const q4::rsrc rw = q4::make_rsrc(reinterpret_cast<const char*>(w) + (int64_t)row * k * EB,
                                          (uint32_t)k * EB);
        const q4::rsrc rq = q4::make_rsrc(qweight + (int64_t)row * (k / 8), (uint32_t)k / 2u);
        const q4::rsrc rs = q4::make_rsrc(scales + (int64_t)row * n_groups, (uint32_t)n_groups * 2u);
        const q4::rsrc rz = q4::make_rsrc(zeros + (int64_t)row * zwords, (uint32_t)zwords * 4u);
        for (int zw = z0; zw < zwords; zw += Z) {
            const int gidx = zw * 8 + grp;
            const bool valid = gidx < n_groups;
            const uint32_t elem = (uint32_t)gidx * G + (uint32_t)t * E;
            float v[E];
            load_slice<E, DT>(rw, valid ? elem * EB : kOff, v);
            double v64[E];
#pragma unroll
            for (int e = 0; e < E; ++e) v64[e] = (double)v[e];

            // the group's statistics, once for all candidates
            float amax = 0.0f, x_min = 0.0f, x_max = 0.0f;
            if constexpr (SYM) {
#pragma unroll
                for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
                amax = xor_max(amax, 1);
                amax = xor_max(amax, 2);
                amax = xor_max(amax, 4);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    x_min = fminf(x_min, v[e]);
                    x_max = fmaxf(x_max, v[e]);
                }
                x_min = xor_min(x_min, 1); x_max = xor_max(x_max, 1);
                x_min = xor_min(x_min, 2); x_max = xor_max(x_max, 2);
                x_min = xor_min(x_min, 4); x_max = xor_max(x_max, 4);
            }

            // the search: every candidate's error, the first smallest kept
            int best = 0;
            double best_err = 0.0;
#pragma unroll
            for (int i = 0; i < kCandidates; ++i) {
                constexpr float kTwenty = 20.0f;
                const float alpha = (float)(20 - i) / kTwenty;  // folded to a constant
                const Cand c = candidate<SYM>(alpha, amax, x_min, x_max);
                double acc = 0.0;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int q = code<SYM, DT>(v[e], c);
                    const double xhat = (double)c.S * (double)(q - c.z);
                    const double d = v64[e] - xhat;
                    acc = acc + d * d;
                }
                acc = xor_add(acc, 1);
                acc = xor_add(acc, 2);
                acc = xor_add(acc, 4);
                const bool take = i == 0 || acc < best_err;
                best = take ? i : best;
                best_err = take ? acc : best_err;
            }

            // the winner's codes, scale and zero point
            const float alpha = (float)(20 - best) / 20.0f;  // correctly rounded, as the table
            const Cand c = candidate<SYM>(alpha, amax, x_min, x_max);
            uint32_t packed[(E + 7) / 8];
#pragma unroll
            for (int j = 0; j < (E + 7) / 8; ++j) packed[j] = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int q = code<SYM, DT>(v[e], c);
                packed[e / 8] |= (uint32_t)(SYM ? q + 8 : q) << (4 * (e % 8));
            }
            const uint32_t qoff = valid ? elem / 2u : kOff;
            if constexpr (E == 16) {
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(q4::u32x2, q4::u32x2{packed[0], packed[1]}),
                                                      rq, (int)qoff, 0, 0);
            } else if constexpr (E == 8) {
                __builtin_amdgcn_raw_buffer_store_b32(packed[0], rq, (int)qoff, 0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)packed[0], rq, (int)qoff, 0, 0);
            }
            __builtin_amdgcn_raw_buffer_store_b16(c.s16, rs, (int)(valid && t == 0 ? (uint32_t)gidx * 2u : kOff), 0, 0);
            if constexpr (!SYM) {
                uint32_t zn = valid ? ((uint32_t)c.z << (4 * grp)) : 0u;
                zn |= __shfl_xor(zn, 8, 64);
                zn |= __shfl_xor(zn, 16, 64);
                zn |= __shfl_xor(zn, 32, 64);
                __builtin_amdgcn_raw_buffer_store_b32(zn, rz, (int)(lane == 0 ? (uint32_t)zw * 4u : kOff), 0, 0);
            }
        }
    }
}

template <int G, bool SYM>
hipError_t launch(const void* w, int dt, int64_t n, int64_t k, uint32_t* qw, uint16_t* sc,
                  uint32_t* zr, hipStream_t st, const char** kname) {
    const int num_cus = q4k_device_cus();
    const int64_t cap = (int64_t)num_cus * 32;  // 8 waves per SIMD
    const int64_t tasks = n * ((k / G + 7) / 8);
    const int64_t waves = tasks < cap ? tasks : cap;
    const int64_t blocks = (waves + 3) / 4;
    static const char* names[3] = {"q4_quant_mse_f32", "q4_quant_mse_f16", "q4_quant_mse_bf16"};
    *kname = names[dt];
    const dim3 grid((unsigned)blocks), block(256);
    const int ni = (int)n, ki = (int)k;
    if (dt == 0)
        hipLaunchKernelGGL((quant_mse_kernel<G, SYM, 0>), grid, block, 0, st, w, ni, ki, qw, sc, zr);
    else if (dt == 1)
        hipLaunchKernelGGL((quant_mse_kernel<G, SYM, 1>), grid, block, 0, st, w, ni, ki, qw, sc, zr);
    else
        hipLaunchKernelGGL((quant_mse_kernel<G, SYM, 2>), grid, block, 0, st, w, ni, ki, qw, sc, zr);
    return q4k_launched(*kname);
}

}  // namespace

hipError_t q4k_quant_mse(const void* w, int w_dtype, int64_t n, int64_t k, int g, int sym,
                         uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                         hipStream_t stream, const char** kname) {
    switch (g * 2 + (sym ? 1 : 0)) {
    case 64: return launch<32, false>(w, w_dtype, n, k, qweight, scales, zeros, stream, kname);
    case 65: return launch<32, true>(w, w_dtype, n, k, qweight, scales, zeros, stream, kname);
    case 128: return launch<64, false>(w, w_dtype, n, k, qweight, scales, zeros, stream, kname);
    case 129: return launch<64, true>(w, w_dtype, n, k, qweight, scales, zeros, stream, kname);
    case 256: return launch<128, false>(w, w_dtype, n, k, qweight, scales, zeros, stream, kname);
    default: return launch<128, true>(w, w_dtype, n, k, qweight, scales, zeros, stream, kname);
    }
}
