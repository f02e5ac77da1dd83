// read_probe.hip — a plain streaming read, the ceiling the benchmark reports the
// bandwidth-bound kernels against.  Not part of the library's interface (include/q4.h);
// built into its own small library (libq4probe.so) that only bench.py loads.
//
// A workgroup of T threads reads one chunk of T * L * 16 bytes: each thread issues L
// independent 16-byte loads at strides of T * 16 bytes (so a wave reads 1 KiB contiguous
// per load) and folds them with XOR; a word is stored only if the fold hits a value the
// benchmark's all-ones buffers never give, so the loads cannot be dropped and nothing else
// runs.  A buffer of B bytes is one launch of ceil(B / chunk) workgroups, every byte read
// once; bytes past the end read zero through the buffer range check.  Several (T, L)
// shapes are built, with the default cache policy and with the non-temporal (streaming)
// policy: small buffers read fastest in small chunks spread over every CU, large ones in
// larger chunks; the benchmark takes the fastest at each size.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// AUX: the buffer load's cache-policy bits (0 default, 2 non-temporal)
template <int T, int L, int AUX>
__global__ __launch_bounds__(T) void read_kernel(const uint8_t* __restrict__ p, int64_t bytes,
                                                 uint32_t* __restrict__ sink) {
    constexpr int64_t kChunk = int64_t(T) * L * 16;
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    const int64_t left = bytes - base;
    const uint32_t size = left < kChunk ? (uint32_t)left : (uint32_t)kChunk;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p + base), (short)0, (int)size,
                                                      0x00020000);
    u32x4 v[L];
#pragma unroll
    for (int i = 0; i < L; ++i)
        v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, (int)((i * T + threadIdx.x) * 16), 0, AUX));
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

struct Shape {
    int threads, loads, aux;
};
constexpr Shape kShapes[] = {{128, 8, 0}, {256, 8, 0}, {256, 16, 0}, {512, 16, 0},
                             {128, 8, 2}, {256, 8, 2}, {256, 16, 2}, {256, 32, 2}};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

template <int T, int L, int AUX>
void launch(const void* p, int64_t bytes, uint32_t* sink, int64_t blocks, hipStream_t st) {
    hipLaunchKernelGGL((read_kernel<T, L, AUX>), dim3((unsigned)blocks), dim3(T), 0, st,
                       static_cast<const uint8_t*>(p), bytes, sink);
}

}  // namespace

extern "C" {

int q4probe_shapes(void) { return kNumShapes; }

// Threads per workgroup, loads per thread and cache-policy bits of shape s.
int q4probe_shape(int s, int* threads, int* loads, int* aux) {
    if (s < 0 || s >= kNumShapes) return 1;
    *threads = kShapes[s].threads;
    *loads = kShapes[s].loads;
    *aux = kShapes[s].aux;
    return 0;
}

// Words of sink a read of bytes bytes with shape s may write (one per workgroup).
int64_t q4probe_sink_words(int64_t bytes, int s) {
    if (s < 0 || s >= kNumShapes || bytes < 1) return -1;
    const int64_t chunk = int64_t(kShapes[s].threads) * kShapes[s].loads * 16;
    return (bytes + chunk - 1) / chunk;
}

// Reads bytes bytes at p (device memory) once with shape s; sink holds
// q4probe_sink_words(bytes, s) words.  0 on success.
int q4probe_read(const void* p, int64_t bytes, uint32_t* sink, int s, hipStream_t stream) {
    const int64_t blocks = q4probe_sink_words(bytes, s);
    if (!p || !sink || blocks < 1 || blocks > (int64_t(1) << 31) - 1) return 1;
    switch (s) {
    case 0: launch<128, 8, 0>(p, bytes, sink, blocks, stream); break;
    case 1: launch<256, 8, 0>(p, bytes, sink, blocks, stream); break;
    case 2: launch<256, 16, 0>(p, bytes, sink, blocks, stream); break;
    case 3: launch<512, 16, 0>(p, bytes, sink, blocks, stream); break;
    case 4: launch<128, 8, 2>(p, bytes, sink, blocks, stream); break;
    case 5: launch<256, 8, 2>(p, bytes, sink, blocks, stream); break;
    case 6: launch<256, 16, 2>(p, bytes, sink, blocks, stream); break;
    default: launch<256, 32, 2>(p, bytes, sink, blocks, stream); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
