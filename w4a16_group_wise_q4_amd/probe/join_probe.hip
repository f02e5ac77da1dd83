// join_probe.hip — what it costs to join partial sums across workgroups within one launch,
// the step a split-K decode GEMV would need.  Not part of the library's interface
// (include/q4.h); built into libq4probe.so beside the read probe, loaded only by bench.py.
//
// A launch of rb * s workgroups of 512 threads: workgroup b is split b % s of row block
// b / s and writes 512 partial sums (value (split + 1) * it, so every launch's totals
// differ); the last workgroup of each row block to arrive adds the s partials in split
// order into y[it][row block][512] and sets the block's arrival counter back to zero.
//   mode 0: the partial stores only (no join: the cost of a trivial launch);
//   mode 1: a device-scope release fence before, and an acquire fence after, one
//           device-scope counter increment per workgroup (the plain C++ memory model);
//   mode 2: partials stored with device-scope relaxed atomic stores, their completion
//           waited for before the workgroup barrier, one relaxed device-scope counter
//           increment, and the last arriver's reads as device-scope atomic loads.
// The counters must be zero before the first launch; every launch leaves them zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kMaxSplits = 16;

template <int MODE>
__global__ __launch_bounds__(kThreads) void join_kernel(float* __restrict__ part, uint32_t* __restrict__ cnt,
                                                        float* __restrict__ y, int s, int it) {
    const int rb = blockIdx.x / s, sp = blockIdx.x % s;
    const int rbs = gridDim.x / s;
    float* p = part + ((size_t)rb * s + sp) * kThreads + threadIdx.x;
    const float v = (float)((sp + 1) * it);
    if constexpr (MODE == 0) {
        *p = v;
        return;
    } else {
        __shared__ int last;
        if constexpr (MODE == 1) {
            *p = v;
        } else {
            __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);  // every counter: the store has completed
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            if constexpr (MODE == 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const uint32_t old = __hip_atomic_fetch_add(cnt + rb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = old == (uint32_t)(s - 1);
            if (last) {
                if constexpr (MODE == 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                __hip_atomic_store(cnt + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
        if (last) {
            if constexpr (MODE == 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const float* q = part + (size_t)rb * s * kThreads + threadIdx.x;
            float pv[kMaxSplits];
#pragma unroll
            for (int i = 0; i < kMaxSplits; ++i)  // every load issued before the first add
                pv[i] = i < s ? (MODE == 1 ? q[(size_t)i * kThreads]
                                           : __hip_atomic_load(q + (size_t)i * kThreads, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT))
                              : 0.f;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < kMaxSplits; ++i)
                if (i < s) acc += pv[i];
            y[((size_t)it * rbs + rb) * kThreads + threadIdx.x] = acc;
        }
    }
}

}  // namespace

extern "C" {

// Floats of part and counters of cnt a launch of rb row blocks x s splits uses; y holds
// (it + 1) * rb * 512 floats for launch numbers up to it.  -1 for an unsupported shape.
int64_t q4probe_join_part_floats(int rb, int s) {
    if (rb < 1 || s < 1 || s > kMaxSplits) return -1;
    return (int64_t)rb * s * kThreads;
}

// One launch of rb * s workgroups in mode 0, 1 or 2 (above); it >= 1 numbers the launch.
// 0 on success.
int q4probe_join(float* part, uint32_t* cnt, float* y, int rb, int s, int mode, int it, hipStream_t stream) {
    if (rb < 1 || s < 1 || s > kMaxSplits || it < 1 || mode < 0 || mode > 2) return 1;
    const dim3 grid((unsigned)(rb * s)), block(kThreads);
    if (mode == 0) hipLaunchKernelGGL(join_kernel<0>, grid, block, 0, stream, part, cnt, y, s, it);
    if (mode == 1) hipLaunchKernelGGL(join_kernel<1>, grid, block, 0, stream, part, cnt, y, s, it);
    if (mode == 2) hipLaunchKernelGGL(join_kernel<2>, grid, block, 0, stream, part, cnt, y, s, it);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
