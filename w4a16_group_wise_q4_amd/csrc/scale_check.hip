// scale_check.hip — corrupted scale detection for a packed weight.
//
// The runtime checks of a quantized artifact include detecting corrupted scales ("LLM
// Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)", §Quantized Artifact Security,
// Runtime).  In this format every stored scale S is an fp16 value >= 0: (max - min)/15 or
// max|w|/7 of a group (§Asymmetric, §Symmetric), rounded, and 0 (or -0) for a group of
// zeros.  A scale that is an infinity, a NaN, or negative (sign set with a nonzero
// magnitude) cannot come from the quantizer and would turn its whole group's products into
// garbage, so it is reported.
//
// Three launches: one thread clears the result, a grid-stride scan counts bad scales (one
// reduction per wave, then one atomic add per count and one atomic minimum of the first
// bad index: integer results that do not depend on the order of the atomics), and one
// thread turns "none found" into -1.  No memset, so the call can sit in a captured graph.
#include "q4_launch.h"

#include <climits>

namespace {

constexpr int kThreads = 256;

__global__ void clear_kernel(int64_t* __restrict__ result) {
    result[0] = 0;
    result[1] = 0;
    result[2] = LLONG_MAX;
}

__global__ __launch_bounds__(kThreads) void scan_kernel(const uint16_t* __restrict__ scales, int64_t count,
                                                        int64_t* __restrict__ result) {
    int64_t nonfinite = 0, negative = 0, first = LLONG_MAX;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride) {
        const uint32_t b = scales[i];
        const bool nf = (b & 0x7C00u) == 0x7C00u;                  // exponent all ones
        const bool neg = !nf && (b & 0x8000u) && (b & 0x7FFFu);    // below zero
        nonfinite += nf;
        negative += neg;
        if ((nf || neg) && i < first) first = i;
    }
    // the wave's totals and minimum
    for (int off = 32; off > 0; off >>= 1) {
        nonfinite += __shfl_xor(nonfinite, off);
        negative += __shfl_xor(negative, off);
        const int64_t o = __shfl_xor(first, off);
        first = o < first ? o : first;
    }
    if ((threadIdx.x & 63) == 0) {
        if (nonfinite) atomicAdd(reinterpret_cast<unsigned long long*>(&result[0]), (unsigned long long)nonfinite);
        if (negative) atomicAdd(reinterpret_cast<unsigned long long*>(&result[1]), (unsigned long long)negative);
        if (first != LLONG_MAX) atomicMin(reinterpret_cast<long long*>(&result[2]), (long long)first);
    }
}

__global__ void finish_kernel(int64_t* __restrict__ result) {
    if (result[2] == LLONG_MAX) result[2] = -1;
}

}  // namespace

hipError_t q4k_check_scales(const uint16_t* scales, int64_t count, int64_t* result, hipStream_t stream,
                            const char** kname) {
    *kname = "q4_check_scales";
    hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, stream, result);
    hipError_t e = q4k_launched("q4_check_scales_clear");
    if (e != hipSuccess) return e;
    // enough workgroups to cover the CUs a few times; each thread then strides the array
    const int64_t need = (count + kThreads - 1) / kThreads;
    const int64_t cap = 8 * (int64_t)q4k_device_cus();
    const int blocks = (int)(need < 1 ? 1 : (need < cap ? need : cap));
    hipLaunchKernelGGL(scan_kernel, dim3(blocks), dim3(kThreads), 0, stream, scales, count, result);
    if ((e = q4k_launched("q4_check_scales")) != hipSuccess) return e;
    hipLaunchKernelGGL(finish_kernel, dim3(1), dim3(1), 0, stream, result);
    return q4k_launched("q4_check_scales_finish");
}
