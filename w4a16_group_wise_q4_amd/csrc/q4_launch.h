// q4_launch.h — host-side launchers of libq4's kernels and the argument types of the
// quantize launch.  Implemented in the .hip files, called by the C ABI after validation.
// Each returns the hipError_t of its launch and writes the launched kernel's name.
#pragma once

#include "q4_device.h"

namespace q4 {
// One matrix of a grouped quantize/pack launch, and the launch's problems.  With
// heads > 0 the input rows are (token, head) pairs r = t * heads + h of new KV-cache
// entries and output row r goes to cache row h * t_cap + t0 + t (a head-major cache).
struct QuantProblem {
    const void* w;
    uint32_t* qweight;
    uint16_t* scales;
    uint32_t* zeros;
    int n;
    int k;
    int heads;
    int t_cap;
    int t0;
};
struct QuantBatch {
    QuantProblem p[kMaxGroup];
    int count;
};
}  // namespace q4

hipError_t q4k_quant_pack(const void* w, int w_dtype, int64_t n, int64_t k, int g, int sym,
                          uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                          hipStream_t stream, const char** kname);
// Several matrices sharing dtype, group size and mode quantized in one launch.
hipError_t q4k_quant_pack_grouped(const q4::QuantProblem* problems, int count, int w_dtype, int g,
                                  int sym, hipStream_t stream, const char** kname);
// New tokens of a KV cache: kv [t_new][heads][d] quantized per (token, head) group of g
// along d into the head-major packed cache at token positions t0 .. t0 + t_new - 1.
hipError_t q4k_kv_quantize(const void* kv, int dtype, int64_t t_new, int64_t heads, int64_t d, int g,
                           int sym, int64_t t_cap, int64_t t0, uint32_t* qcache, uint16_t* scache,
                           uint32_t* zcache, hipStream_t stream, const char** kname);
// Decode attention over INT4 K/V caches: the chunk split (chunks per head; loads per wave,
// a chunk being 4 waves x loads x 2048/d tokens; never more than max_chunks per head) and
// the two launches (per-chunk partials into workspace, then the combine).
void q4k_kv_attention_shape(int64_t heads, int64_t d, int64_t n_tok, int* chunks, int* loads);
int64_t q4k_kv_max_chunks(int64_t d, int64_t n_tok);
hipError_t q4k_kv_attention(const void* q, int q_dtype, const uint32_t* kq, const uint16_t* ks,
                            const uint32_t* kz, const uint32_t* vq, const uint16_t* vs,
                            const uint32_t* vz, int64_t heads, int64_t d, int64_t n_tok,
                            int64_t t_cap, int g, int sym, float scale, float* out,
                            float* workspace, int chunks, int loads, hipStream_t stream,
                            const char** kname);
// Compute units of the current device, looked up once per device (256 if the query
// fails); safe to call from several threads.
int q4k_device_cus();
// Corrupted scale detection over count fp16 scales: result (3 int64, device) = non-finite
// count, negative count, first bad index or -1.
hipError_t q4k_check_scales(const uint16_t* scales, int64_t count, int64_t* result, hipStream_t stream,
                            const char** kname);

// The fixed per-device scratch of the no-allocation attention entry point: its size in
// bytes, and its device address on the current device (looked up once per device; a
// failed lookup returns the runtime's error and leaves *ptr NULL).
constexpr int64_t kKvScratchBytes = int64_t(16) << 20;
hipError_t q4k_kv_scratch(void** ptr);
hipError_t q4k_quant_mse(const void* w, int w_dtype, int64_t n, int64_t k, int g, int sym,
                         uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                         hipStream_t stream, const char** kname);
hipError_t q4k_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                       int64_t n, int64_t k, int g, int sym, void* out, int out_dtype,
                       hipStream_t stream, const char** kname);
// y: fp32, fp16 or bf16 elements (ydt = 0, 1, 2: the q4_dtype codes), rounded from the fp32
// accumulators in the kernel's epilogue.
hipError_t q4k_gemv(const void* x, int x_dtype, int m, const uint32_t* qweight,
                    const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k, int g,
                    int sym, void* y, int ydt, hipStream_t stream, const char** kname);
// Decode tile kernels for one group size (32, 64 or 128): UPW units per wave, `waves` waves
// per 16-row tile, one workgroup per tile of the batch; wide != 0 selects the kernel for
// m up to 16 that streams the activations instead of staging them.
hipError_t q4k_gemv_tile_g32(int sym, int x_dtype, int m, int k, int upw, int waves, int wide,
                             const q4::GemvBatch& batch, int tiles, hipStream_t stream,
                             const char** kname);
hipError_t q4k_gemv_tile_g64(int sym, int x_dtype, int m, int k, int upw, int waves, int wide,
                             const q4::GemvBatch& batch, int tiles, hipStream_t stream,
                             const char** kname);
hipError_t q4k_gemv_tile_g128(int sym, int x_dtype, int m, int k, int upw, int waves, int wide,
                              const q4::GemvBatch& batch, int tiles, hipStream_t stream,
                              const char** kname);
// Runs count problems (shared m <= 16, k, g, sym, dtype) in one launch when their
// activations fit the streaming kernel; returns hipErrorNotSupported (enqueuing nothing)
// otherwise, so the caller runs them one by one.
hipError_t q4k_gemv_grouped(const q4::GemvProblem* problems, int count, int x_dtype, int m,
                            int64_t k, int g, int sym, int ydt, hipStream_t stream, const char** kname);
// Prefill GEMM; with a workspace (floats) a product that leaves CUs idle splits its K range
// (partials in the workspace, then an ordered reduction into y).  q4k_gemm_workspace_floats
// gives the size it would use, 0 when it would not split.
int64_t q4k_gemm_workspace_floats(int64_t m, int64_t n, int64_t k);
hipError_t q4k_gemm(const void* x, int x_dtype, int64_t m, const uint32_t* qweight,
                    const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k, int g,
                    int sym, void* y, int ydt, float* workspace, int64_t workspace_floats,
                    hipStream_t stream, const char** kname);
// GPTQ error-feedback quantization (static RTN group quantizers, codes chosen against the
// calibration Hessian); workspace: k*k + n*k + 256*n floats, and with act_order (columns
// swept by descending activation energy) 3*k + n*k/4 more.
int64_t q4k_gptq_workspace_floats(int64_t n, int64_t k);
int64_t q4k_gptq_act_order_workspace_floats(int64_t n, int64_t k);
hipError_t q4k_gptq(const void* w, int w_dtype, int64_t n, int64_t k, const void* x, int x_dtype,
                    int64_t tokens, int g, int sym, float damp, uint32_t* qweight, uint16_t* scales,
                    uint32_t* zeros, float* workspace, int act_order, hipStream_t stream,
                    const char** kname);
