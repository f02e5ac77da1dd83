// q4_abi.cpp — the C ABI of libq4 (declared in include/q4.h).
//
// Validates every argument on the host before anything is enqueued, picks the kernel
// (decode GEMV for m <= 16, the GEMV on 16-row chunks for narrow grids up to m = 256,
// prefill GEMM otherwise), launches it on the caller's stream
// and records the launched kernel's name per thread, so a caller can check which kernel
// ran ("LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)", §Silent Fallback:
// verify the selected kernel and that nothing fell back).  There is no fallback path.
#include "q4.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>
#include <string>

#include "q4_launch.h"

#ifndef Q4_SOURCE_DIGEST
#error "Q4_SOURCE_DIGEST (the digest of the sources, computed by the build) must be defined"
#endif

namespace {

thread_local const char* g_last_kernel = "";

// The kernels enqueued by the calling thread's current entry-point call (distinct names in
// launch order, and the number of launches), and those of its last successful call.
struct LaunchLog {
    const char* names[32];
    int distinct;
    int64_t count;
};
thread_local LaunchLog g_cur_log = {{}, 0, 0};
thread_local LaunchLog g_last_log = {{}, 0, 0};
thread_local std::string g_last_names;

void begin_call() {
    g_cur_log.distinct = 0;
    g_cur_log.count = 0;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// The matmul kernels address one tile's activations (up to 256 rows of k bf16 values)
// and their outputs with 32-bit offsets: k <= 2^22, n <= 2^25 and m*n <= 2^38 keep every
// offset in range.
constexpr int64_t kMaxMatmulK = int64_t(1) << 22;
constexpr int64_t kMaxMatmulOut = int64_t(1) << 38;
// The GEMV addresses y (at most 16 rows of n fp32) with 32-bit buffer offsets.
constexpr int64_t kMaxMatmulN = int64_t(1) << 25;

bool group_ok(int32_t g) { return g == 32 || g == 64 || g == 128; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

q4_status check_layout(int64_t n, int64_t k, int32_t g) {
    if (!group_ok(g)) return Q4_ERR_GROUP;
    if (n < 1 || k < 1 || n > kMaxDim || k > kMaxDim) return Q4_ERR_SHAPE;
    if (k % g != 0) return Q4_ERR_SHAPE;
    if (n > kMaxElems / k) return Q4_ERR_SHAPE;
    return Q4_OK;
}

q4_status check_packed(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                       int32_t symmetric) {
    if (!qweight || !scales || (!symmetric && !zeros)) return Q4_ERR_NULL;
    if (!aligned(qweight, 16) || !aligned(scales, 2) || (!symmetric && !aligned(zeros, 4)))
        return Q4_ERR_ALIGN;
    return Q4_OK;
}

// A row of w is addressed with 32-bit byte offsets (up to 4 bytes per weight).
constexpr int64_t kMaxQuantK = int64_t(1) << 28;

// The size, dtype, pointer and alignment rules of q4_quantize_pack for one matrix.
q4_status check_quant(const void* w, q4_dtype w_dtype, int64_t n, int64_t k, int32_t group_size,
                      int32_t symmetric, const uint32_t* qweight, const uint16_t* scales,
                      const uint32_t* zeros) {
    q4_status st = check_layout(n, k, group_size);
    if (st != Q4_OK) return st;
    if (k > kMaxQuantK) return Q4_ERR_SHAPE;
    if (w_dtype != Q4_F32 && w_dtype != Q4_F16 && w_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (!w) return Q4_ERR_NULL;
    if ((st = check_packed(qweight, scales, zeros, symmetric)) != Q4_OK) return st;
    if (!aligned(w, 16)) return Q4_ERR_ALIGN;
    return Q4_OK;
}

q4_status finish(hipError_t e, const char* name) {
    if (e != hipSuccess) return Q4_ERR_LAUNCH;
    g_last_kernel = name;
    g_last_log = g_cur_log;
    g_last_names.clear();
    for (int i = 0; i < g_last_log.distinct; ++i) {
        if (i) g_last_names += ",";
        g_last_names += g_last_log.names[i];
    }
    return Q4_OK;
}

}  // namespace

void q4k_record(const char* name) {
    ++g_cur_log.count;
    for (int i = 0; i < g_cur_log.distinct; ++i)
        if (std::strcmp(g_cur_log.names[i], name) == 0) return;
    if (g_cur_log.distinct < 32) g_cur_log.names[g_cur_log.distinct++] = name;
}

extern "C" {

q4_status q4_quantize_pack(const void* w, q4_dtype w_dtype, int64_t n, int64_t k,
                           int32_t group_size, int32_t symmetric, uint32_t* qweight,
                           uint16_t* scales, uint32_t* zeros, hipStream_t stream) {
    begin_call();
    q4_status st = check_quant(w, w_dtype, n, k, group_size, symmetric, qweight, scales, zeros);
    if (st != Q4_OK) return st;
    const char* name = "";
    hipError_t e = q4k_quant_pack(w, (int)w_dtype, n, k, group_size, symmetric ? 1 : 0, qweight,
                                  scales, zeros, stream, &name);
    return finish(e, name);
}

q4_status q4_quantize_pack_mse(const void* w, q4_dtype w_dtype, int64_t n, int64_t k,
                               int32_t group_size, int32_t symmetric, uint32_t* qweight,
                               uint16_t* scales, uint32_t* zeros, hipStream_t stream) {
    begin_call();
    q4_status st = check_quant(w, w_dtype, n, k, group_size, symmetric, qweight, scales, zeros);
    if (st != Q4_OK) return st;
    const char* name = "";
    hipError_t e = q4k_quant_mse(w, (int)w_dtype, n, k, group_size, symmetric ? 1 : 0, qweight,
                                 scales, zeros, stream, &name);
    return finish(e, name);
}

q4_status q4_quantize_pack_grouped(const q4_quant_problem* problems, int32_t count,
                                   q4_dtype w_dtype, int32_t group_size, int32_t symmetric,
                                   hipStream_t stream) {
    begin_call();
    if (!problems) return Q4_ERR_NULL;
    if (count < 1 || count > q4::kMaxGroup) return Q4_ERR_SHAPE;
    q4::QuantProblem qp[q4::kMaxGroup];
    for (int i = 0; i < count; ++i) {
        const q4_quant_problem& p = problems[i];
        const q4_status st = check_quant(p.w, w_dtype, p.n, p.k, group_size, symmetric, p.qweight,
                                         p.scales, p.zeros);
        if (st != Q4_OK) return st;
        qp[i] = q4::QuantProblem{p.w, p.qweight, p.scales, symmetric ? nullptr : p.zeros, (int)p.n,
                                 (int)p.k};
    }
    const char* name = "";
    const hipError_t e = q4k_quant_pack_grouped(qp, count, (int)w_dtype, group_size,
                                                symmetric ? 1 : 0, stream, &name);
    return finish(e, name);
}

q4_status q4_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                     int64_t n, int64_t k, int32_t group_size, int32_t symmetric, void* w_out,
                     q4_dtype out_dtype, hipStream_t stream) {
    begin_call();
    q4_status st = check_layout(n, k, group_size);
    if (st != Q4_OK) return st;
    if (out_dtype != Q4_F32 && out_dtype != Q4_F16 && out_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if ((st = check_packed(qweight, scales, zeros, symmetric)) != Q4_OK) return st;
    if (!w_out) return Q4_ERR_NULL;
    if (!aligned(w_out, 16)) return Q4_ERR_ALIGN;
    const char* name = "";
    hipError_t e = q4k_dequant(qweight, scales, zeros, n, k, group_size, symmetric ? 1 : 0, w_out,
                               (int)out_dtype, stream, &name);
    return finish(e, name);
}

q4_status q4_check_scales(const uint16_t* scales, int64_t n, int64_t k, int32_t group_size,
                          int64_t* result, hipStream_t stream) {
    begin_call();
    const q4_status st = check_layout(n, k, group_size);
    if (st != Q4_OK) return st;
    if (!scales || !result) return Q4_ERR_NULL;
    if (!aligned(scales, 2) || !aligned(result, 8)) return Q4_ERR_ALIGN;
    const char* name = "";
    const hipError_t e = q4k_check_scales(scales, n * (k / group_size), result, stream, &name);
    return finish(e, name);
}

}  // extern "C"

// Compute units per device.  Threads that race on the first lookup store the same value.
int q4k_device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

extern "C" {

namespace {

// One W4A16 product, validated.  m <= 16: the decode GEMV.  16 < m <= 256: the GEMV on
// 16-row chunks of x sharing the weight (full chunks in grouped launches of up to 8, the
// rest alone) when that is faster than the prefill GEMM, else the GEMM.  A GEMM grid of
// 128 x 256 tiles that fits in one round (at most 2 workgroups per CU) takes about
// k x 20.7 ns on MI355X whatever m and n, while the chunks stream chunks x n x k/2 bytes of
// codes at about 3.5 TB/s (the grouped chunks share the weight through the caches); so the
// chunks win while chunks x n stays under about 144K rows.
// ([FL7] §Batch와 Context에 따라 속도가 달라진다: decode batches sit between the
// bandwidth-bound and the compute-bound regime.)
bool chunked_gemv(int64_t m, int64_t n, int cus) {
    if (m <= 16 || m > 256) return false;
    const int64_t chunks = (m + 15) / 16;
    const int64_t gemm_wgs = ((m + 127) / 128) * ((n + 255) / 256);
    return gemm_wgs <= 2 * (int64_t)cus && chunks * n < 144 * 1024;
}

// Whether a product with a workspace runs as the split-K GEMM (rather than as below): where
// the GEMM's tiles leave CUs idle, from m > 64 on (below that the chunked GEMV is as fast or
// faster on the 7B projections), and from m > 32 on for matrices of 2^27 weights and more
// (the 70B projection at m = 64: 94 against 114 us).
bool splitk_gemm(int64_t m, int64_t n, int64_t k) {
    if (m <= 32 || (m <= 64 && n * k < (int64_t(1) << 27))) return false;
    return q4k_gemm_workspace_floats(m, n, k) > 0;
}

hipError_t run_product(const void* x, int xd, int64_t m, const uint32_t* qw, const uint16_t* sc,
                       const uint32_t* zr, int64_t n, int64_t k, int g, int sym, void* y, int ydt,
                       float* ws, int64_t ws_floats, hipStream_t st, const char** name) {
    if (m <= 16) return q4k_gemv(x, xd, (int)m, qw, sc, zr, n, k, g, sym, y, ydt, st, name);
    if (ws != nullptr && splitk_gemm(m, n, k))
        return q4k_gemm(x, xd, m, qw, sc, zr, n, k, g, sym, y, ydt, ws, ws_floats, st, name);
    if (!chunked_gemv(m, n, q4k_device_cus()))
        return q4k_gemm(x, xd, m, qw, sc, zr, n, k, g, sym, y, ydt, nullptr, 0, st, name);
    const int64_t full = m / 16, rem = m % 16;
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    char* yb = static_cast<char*>(y);
    const int64_t ye = ydt == Q4_F32 ? 4 : 2;  // bytes per y element
    for (int64_t c0 = 0; c0 < full; c0 += q4::kMaxGroup) {
        const int64_t cnt = full - c0 < q4::kMaxGroup ? full - c0 : q4::kMaxGroup;
        q4::GemvProblem gp[q4::kMaxGroup];
        for (int64_t c = 0; c < cnt; ++c)
            gp[c] = q4::GemvProblem{xs + (c0 + c) * 16 * k, qw, sc, zr, yb + (c0 + c) * 16 * n * ye, (int)n, 0};
        hipError_t e = hipErrorNotSupported;
        if (cnt > 1) e = q4k_gemv_grouped(gp, (int)cnt, xd, 16, k, g, sym, ydt, st, name);
        if (e == hipErrorNotSupported) {
            for (int64_t c = 0; c < cnt; ++c) {
                e = q4k_gemv(gp[c].x, xd, 16, qw, sc, zr, n, k, g, sym, gp[c].y, ydt, st, name);
                if (e != hipSuccess) return e;
            }
        } else if (e != hipSuccess) {
            return e;
        }
    }
    if (rem > 0)
        return q4k_gemv(xs + full * 16 * k, xd, (int)rem, qw, sc, zr, n, k, g, sym, yb + full * 16 * n * ye,
                        ydt, st, name);
    return hipSuccess;
}

// The size, dtype, pointer and alignment rules of q4_w4a16_gemm_out for one problem.
q4_status check_matmul(const void* x, q4_dtype x_dtype, int64_t m, const uint32_t* qweight,
                       const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k,
                       int32_t group_size, int32_t symmetric, const void* y, q4_dtype y_dtype) {
    q4_status st = check_layout(n, k, group_size);
    if (st != Q4_OK) return st;
    if (k > kMaxMatmulK || n > kMaxMatmulN) return Q4_ERR_SHAPE;
    if (m < 1 || m > kMaxDim || m > kMaxElems / k || m > kMaxMatmulOut / n) return Q4_ERR_SHAPE;
    if (x_dtype != Q4_F16 && x_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (y_dtype != Q4_F32 && y_dtype != Q4_F16 && y_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (!x || !y) return Q4_ERR_NULL;
    if ((st = check_packed(qweight, scales, zeros, symmetric)) != Q4_OK) return st;
    if (!aligned(x, 16) || !aligned(y, y_dtype == Q4_F32 ? 4 : 2)) return Q4_ERR_ALIGN;
    return Q4_OK;
}
}  // namespace

q4_status q4_w4a16_gemm_grouped_out(const q4_gemm_problem* problems, int32_t count,
                                    q4_dtype x_dtype, int64_t m, int64_t k, int32_t group_size,
                                    int32_t symmetric, q4_dtype y_dtype, hipStream_t stream) {
    begin_call();
    if (!problems) return Q4_ERR_NULL;
    if (count < 1 || count > q4::kMaxGroup) return Q4_ERR_SHAPE;
    int64_t rows = 0;
    for (int32_t i = 0; i < count; ++i) {
        const q4_gemm_problem& p = problems[i];
        const q4_status st = check_matmul(p.x, x_dtype, m, p.qweight, p.scales, p.zeros, p.n, k,
                                          group_size, symmetric, p.y, y_dtype);
        if (st != Q4_OK) return st;
        rows += (p.n + 15) / 16 * 16;
    }
    const char* name = "";
    if (m <= 16 && count > 1 && rows <= kMaxMatmulN) {
        q4::GemvProblem gp[q4::kMaxGroup];
        for (int32_t i = 0; i < count; ++i)
            gp[i] = q4::GemvProblem{problems[i].x, problems[i].qweight, problems[i].scales,
                                    symmetric ? nullptr : problems[i].zeros, problems[i].y,
                                    (int)problems[i].n, 0};
        const hipError_t e = q4k_gemv_grouped(gp, count, (int)x_dtype, (int)m, k, group_size,
                                              symmetric ? 1 : 0, (int)y_dtype, stream, &name);
        if (e != hipErrorNotSupported) return finish(e, name);
    }
    for (int32_t i = 0; i < count; ++i) {  // one product at a time
        const q4_gemm_problem& p = problems[i];
        const hipError_t e = run_product(p.x, (int)x_dtype, m, p.qweight, p.scales,
                                         symmetric ? nullptr : p.zeros, p.n, k, group_size,
                                         symmetric ? 1 : 0, p.y, (int)y_dtype, nullptr, 0, stream, &name);
        if (e != hipSuccess) return Q4_ERR_LAUNCH;
    }
    return finish(hipSuccess, name);
}

q4_status q4_w4a16_gemm_grouped(const q4_gemm_problem* problems, int32_t count,
                                q4_dtype x_dtype, int64_t m, int64_t k, int32_t group_size,
                                int32_t symmetric, hipStream_t stream) {
    return q4_w4a16_gemm_grouped_out(problems, count, x_dtype, m, k, group_size, symmetric, Q4_F32,
                                     stream);
}

q4_status q4_w4a16_gemm_out(const void* x, q4_dtype x_dtype, int64_t m, const uint32_t* qweight,
                            const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k,
                            int32_t group_size, int32_t symmetric, void* y, q4_dtype y_dtype,
                            hipStream_t stream) {
    return q4_w4a16_gemm_ws(x, x_dtype, m, qweight, scales, zeros, n, k, group_size, symmetric, y,
                            y_dtype, nullptr, 0, stream);
}

int64_t q4_w4a16_gemm_workspace(int64_t m, int64_t n, int64_t k, int32_t group_size) {
    if (check_layout(n, k, group_size) != Q4_OK || k > kMaxMatmulK || n > kMaxMatmulN) return -1;
    if (m < 1 || m > kMaxDim || m > kMaxElems / k || m > kMaxMatmulOut / n) return -1;
    return splitk_gemm(m, n, k) ? q4k_gemm_workspace_floats(m, n, k) * (int64_t)sizeof(float) : 0;
}

q4_status q4_w4a16_gemm_ws(const void* x, q4_dtype x_dtype, int64_t m, const uint32_t* qweight,
                           const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k,
                           int32_t group_size, int32_t symmetric, void* y, q4_dtype y_dtype,
                           void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    begin_call();
    const q4_status st = check_matmul(x, x_dtype, m, qweight, scales, zeros, n, k, group_size,
                                      symmetric, y, y_dtype);
    if (st != Q4_OK) return st;
    int64_t ws_floats = 0;
    if (workspace != nullptr) {
        if (!aligned(workspace, 16)) return Q4_ERR_ALIGN;
        if (workspace_bytes < q4_w4a16_gemm_workspace(m, n, k, group_size)) return Q4_ERR_SHAPE;
        ws_floats = workspace_bytes / (int64_t)sizeof(float);
    }
    const char* name = "";
    const hipError_t e = run_product(x, (int)x_dtype, m, qweight, scales, symmetric ? nullptr : zeros, n,
                                     k, group_size, symmetric ? 1 : 0, y, (int)y_dtype,
                                     static_cast<float*>(workspace), ws_floats, stream, &name);
    return finish(e, name);
}

q4_status q4_w4a16_gemm(const void* x, q4_dtype x_dtype, int64_t m, const uint32_t* qweight,
                        const uint16_t* scales, const uint32_t* zeros, int64_t n, int64_t k,
                        int32_t group_size, int32_t symmetric, float* y, hipStream_t stream) {
    return q4_w4a16_gemm_out(x, x_dtype, m, qweight, scales, zeros, n, k, group_size, symmetric, y,
                             Q4_F32, stream);
}

namespace {
constexpr int64_t kMaxKvHeads = 65536;
constexpr int64_t kMaxKvTokens = int64_t(1) << 24;
constexpr int64_t kMaxKvDim = 65536;

// Sizes shared by both KV entry points: head-major cache rows heads * t_cap index as int.
q4_status check_kv_sizes(int64_t heads, int64_t head_dim, int32_t g, int64_t t_cap) {
    if (!group_ok(g)) return Q4_ERR_GROUP;
    if (heads < 1 || head_dim < 1 || t_cap < 1 || head_dim > kMaxKvDim) return Q4_ERR_SHAPE;
    if (head_dim % g != 0) return Q4_ERR_SHAPE;
    if (t_cap > kMaxDim / heads) return Q4_ERR_SHAPE;
    return Q4_OK;
}

bool kv_attention_dims_ok(int64_t heads, int64_t head_dim, int64_t n_tok) {
    return (head_dim == 64 || head_dim == 128 || head_dim == 256) && heads >= 1 &&
           heads <= kMaxKvHeads && n_tok >= 1 && n_tok <= kMaxKvTokens;
}
}  // namespace

q4_status q4_kv_quantize(const void* kv, q4_dtype kv_dtype, int64_t t_new, int64_t heads,
                         int64_t head_dim, int32_t group_size, int32_t symmetric, int64_t t_cap,
                         int64_t t0, uint32_t* qcache, uint16_t* scache, uint32_t* zcache,
                         hipStream_t stream) {
    begin_call();
    q4_status st = check_kv_sizes(heads, head_dim, group_size, t_cap);
    if (st != Q4_OK) return st;
    if (t_new < 1 || t0 < 0 || t0 > t_cap - t_new) return Q4_ERR_SHAPE;
    st = check_quant(kv, kv_dtype, t_new * heads, head_dim, group_size, symmetric, qcache, scache,
                     zcache);
    if (st != Q4_OK) return st;
    const char* name = "";
    const hipError_t e = q4k_kv_quantize(kv, (int)kv_dtype, t_new, heads, head_dim, group_size,
                                         symmetric ? 1 : 0, t_cap, t0, qcache, scache,
                                         symmetric ? nullptr : zcache, stream, &name);
    return finish(e, name);
}

int64_t q4_kv_attention_workspace(int64_t heads, int64_t head_dim, int64_t n_tok) {
    if (!kv_attention_dims_ok(heads, head_dim, n_tok)) return -1;
    return heads * q4k_kv_max_chunks(head_dim, n_tok) * (head_dim + 2) * (int64_t)sizeof(float);
}

q4_status q4_kv_attention(const void* q, q4_dtype q_dtype, int64_t heads, int64_t head_dim,
                          int64_t n_tok, int64_t t_cap, const uint32_t* kq, const uint16_t* ks,
                          const uint32_t* kz, const uint32_t* vq, const uint16_t* vs,
                          const uint32_t* vz, int32_t group_size, int32_t symmetric, float scale,
                          float* out, void* workspace, int64_t workspace_bytes,
                          hipStream_t stream) {
    begin_call();
    q4_status st = check_kv_sizes(heads, head_dim, group_size, t_cap);
    if (st != Q4_OK) return st;
    if (!kv_attention_dims_ok(heads, head_dim, n_tok) || n_tok > t_cap) return Q4_ERR_SHAPE;
    if (q_dtype != Q4_F16 && q_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (!q || !out || !workspace) return Q4_ERR_NULL;
    if ((st = check_packed(kq, ks, kz, symmetric)) != Q4_OK) return st;
    if ((st = check_packed(vq, vs, vz, symmetric)) != Q4_OK) return st;
    if (!aligned(q, 16) || !aligned(out, 4) || !aligned(workspace, 16)) return Q4_ERR_ALIGN;
    if (workspace_bytes < q4_kv_attention_workspace(heads, head_dim, n_tok)) return Q4_ERR_SHAPE;
    int chunks = 0, loads = 0;
    q4k_kv_attention_shape(heads, head_dim, n_tok, &chunks, &loads);
    const char* name = "";
    const hipError_t e = q4k_kv_attention(
        q, (int)q_dtype, kq, ks, symmetric ? nullptr : kz, vq, vs, symmetric ? nullptr : vz, heads,
        head_dim, n_tok, t_cap, group_size, symmetric ? 1 : 0, scale, out,
        static_cast<float*>(workspace), chunks, loads, stream, &name);
    return finish(e, name);
}

q4_status q4_kv_attention_noalloc(const void* q, q4_dtype q_dtype, int64_t heads, int64_t head_dim,
                                  int64_t n_tok, int64_t t_cap, const uint32_t* kq,
                                  const uint16_t* ks, const uint32_t* kz, const uint32_t* vq,
                                  const uint16_t* vs, const uint32_t* vz, int32_t group_size,
                                  int32_t symmetric, float scale, float* out, hipStream_t stream) {
    begin_call();
    q4_status st = check_kv_sizes(heads, head_dim, group_size, t_cap);
    if (st != Q4_OK) return st;
    if (!kv_attention_dims_ok(heads, head_dim, n_tok) || n_tok > t_cap) return Q4_ERR_SHAPE;
    if (q_dtype != Q4_F16 && q_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (!q || !out) return Q4_ERR_NULL;
    if ((st = check_packed(kq, ks, kz, symmetric)) != Q4_OK) return st;
    if ((st = check_packed(vq, vs, vz, symmetric)) != Q4_OK) return st;
    if (!aligned(q, 16) || !aligned(out, 4)) return Q4_ERR_ALIGN;
    int chunks = 0, loads = 0;
    q4k_kv_attention_shape(heads, head_dim, n_tok, &chunks, &loads);
    if (heads * chunks * (head_dim + 2) * (int64_t)sizeof(float) > kKvScratchBytes) return Q4_ERR_SCRATCH;
    void* ws = nullptr;
    if (q4k_kv_scratch(&ws) != hipSuccess || ws == nullptr) return Q4_ERR_LAUNCH;
    const char* name = "";
    const hipError_t e = q4k_kv_attention(
        q, (int)q_dtype, kq, ks, symmetric ? nullptr : kz, vq, vs, symmetric ? nullptr : vz, heads,
        head_dim, n_tok, t_cap, group_size, symmetric ? 1 : 0, scale, out, static_cast<float*>(ws),
        chunks, loads, stream, &name);
    return finish(e, name);
}

int64_t q4_kv_attention_noalloc_max_bytes(void) { return kKvScratchBytes; }

namespace {
constexpr int64_t kMaxGptqK = 32768;   // the k x k Hessian: at most 4 GiB of fp32
}  // namespace

int64_t q4_gptq_workspace(int64_t n, int64_t k, int32_t group_size) {
    if (check_layout(n, k, group_size) != Q4_OK || k > kMaxGptqK) return -1;
    return q4k_gptq_workspace_floats(n, k) * (int64_t)sizeof(float);
}

int64_t q4_gptq_act_order_workspace(int64_t n, int64_t k, int32_t group_size) {
    if (check_layout(n, k, group_size) != Q4_OK || k > kMaxGptqK) return -1;
    return q4k_gptq_act_order_workspace_floats(n, k) * (int64_t)sizeof(float);
}

namespace {
q4_status gptq_call(const void* w, q4_dtype w_dtype, int64_t n, int64_t k, const void* x,
                    q4_dtype x_dtype, int64_t tokens, int32_t group_size, int32_t symmetric,
                    float damp, uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                    void* workspace, int64_t workspace_bytes, int act_order, hipStream_t stream) {
    begin_call();
    q4_status st = check_quant(w, w_dtype, n, k, group_size, symmetric, qweight, scales, zeros);
    if (st != Q4_OK) return st;
    if (k > kMaxGptqK || tokens < 1 || tokens > kMaxDim || tokens > kMaxElems / k) return Q4_ERR_SHAPE;
    if (!(damp > 0.0f) || !(damp <= 1.0f)) return Q4_ERR_SHAPE;
    if (x_dtype != Q4_F16 && x_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (!x || !workspace) return Q4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(workspace, 16)) return Q4_ERR_ALIGN;
    const int64_t need = act_order ? q4_gptq_act_order_workspace(n, k, group_size)
                                   : q4_gptq_workspace(n, k, group_size);
    if (workspace_bytes < need) return Q4_ERR_SHAPE;
    const char* name = "";
    const hipError_t e = q4k_gptq(w, (int)w_dtype, n, k, x, (int)x_dtype, tokens, group_size,
                                  symmetric ? 1 : 0, damp, qweight, scales, symmetric ? nullptr : zeros,
                                  static_cast<float*>(workspace), act_order, stream, &name);
    return finish(e, name);
}
}  // namespace

q4_status q4_gptq_quantize(const void* w, q4_dtype w_dtype, int64_t n, int64_t k, const void* x,
                           q4_dtype x_dtype, int64_t tokens, int32_t group_size, int32_t symmetric,
                           float damp, uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                           void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return gptq_call(w, w_dtype, n, k, x, x_dtype, tokens, group_size, symmetric, damp, qweight,
                     scales, zeros, workspace, workspace_bytes, 0, stream);
}

q4_status q4_gptq_quantize_act_order(const void* w, q4_dtype w_dtype, int64_t n, int64_t k,
                                     const void* x, q4_dtype x_dtype, int64_t tokens,
                                     int32_t group_size, int32_t symmetric, float damp,
                                     uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                                     void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return gptq_call(w, w_dtype, n, k, x, x_dtype, tokens, group_size, symmetric, damp, qweight,
                     scales, zeros, workspace, workspace_bytes, 1, stream);
}

int64_t q4_qweight_words(int64_t n, int64_t k) {
    if (n < 1 || k < 1 || k % 8 != 0) return -1;
    return n * (k / 8);
}

int64_t q4_scale_count(int64_t n, int64_t k, int32_t group_size) {
    if (check_layout(n, k, group_size) != Q4_OK) return -1;
    return n * (k / group_size);
}

int64_t q4_zero_words(int64_t n, int64_t k, int32_t group_size) {
    if (check_layout(n, k, group_size) != Q4_OK) return -1;
    return n * ((k / group_size + 7) / 8);
}

const char* q4_status_str(q4_status s) {
    switch (s) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "shape out of range (n, k, m >= 1; k a multiple of group_size)";
    case Q4_ERR_GROUP: return "group_size must be 32, 64 or 128";
    case Q4_ERR_DTYPE: return "dtype not accepted by this entry point";
    case Q4_ERR_ALIGN: return "pointer misaligned (w/x/qweight/w_out 16 B, zeros/y 4 B, scales 2 B)";
    case Q4_ERR_LAUNCH: return "kernel launch failed";
    case Q4_ERR_SCRATCH: return "sizes need more than the fixed scratch of the no-allocation entry point";
    default: break;
    }
    return "unknown status";
}

const char* q4_last_kernel(void) { return g_last_kernel; }

const char* q4_last_kernels(void) { return g_last_names.c_str(); }

int64_t q4_last_launch_count(void) { return g_last_log.count; }

const char* q4_source_digest(void) { return Q4_SOURCE_DIGEST; }

int32_t q4_layout_version(void) { return 1; }

}  // extern "C"
