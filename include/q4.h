/* q4.h — C ABI of the MI355X (gfx950) group-wise INT4 weight-only (W4A16) library.
 *
 * What the operations are (pages cited by title and section):
 *   [FL7] "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)", blog.ruahverce.com
 *   [QA1] "Quantization Algorithms 단권화", brianyu43.github.io (V10)
 *   [YJ]  "최신 LLM 양자화 기술 총정리 — GPTQ·AWQ부터 FP8·MXFP4·KV 캐시 양자화까지",
 *         youngju.dev (Korean and English versions)
 *
 * Packed format (canonical, layout version 1).  W is [n][k] row-major: n output features,
 * k input features.  A group is g consecutive input columns of one row ([FL7] §Per-group),
 * G = k / g groups per row.
 *   qweight : uint32 [n][k/8]; the 4-bit code of column 8j+i is bits 4i..4i+3 of word j.
 *   scales  : fp16 bit patterns [n][G], the scale S of each group.  The matmul and
 *             dequant entry points take any finite S; a group with S = 0 contributes 0.
 *   zeros   : uint32 [n][ceil(G/8)]; zero point of group 8j+i in bits 4i..4i+3 of word j,
 *             unused pad nibbles are 0.  Asymmetric mode only.
 * Asymmetric codes are q in [0,15] stored as is; symmetric codes q in [-8,7] are stored
 * as u = q + 8 (an implicit zero point of 8) ([QA1] §Signed ↔ Unsigned gives the ranges).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are device memory owned by the caller.  No call allocates or frees
 *     anything, and none synchronizes: work is enqueued on `stream` (NULL = the default
 *     stream) and the call returns.  The only memory the library holds itself is the
 *     fixed scratch of q4_kv_attention_noalloc (below).
 *   - Arguments are validated on the host before anything is enqueued; an invalid call
 *     returns a non-zero q4_status and touches no memory.  A launch failure reported by
 *     the runtime returns Q4_ERR_LAUNCH.  Faults during execution surface at the
 *     caller's next synchronization, as for any asynchronous HIP work.
 *   - Sizes: 1 <= n, 1 <= k, k % group_size == 0, group_size in {32, 64, 128}, and
 *     n*k < 2^40 (so every element index fits comfortably in 64 bits).
 *   - Alignment: w, x, qweight and w_out 16 bytes; zeros and y 4 bytes; scales 2 bytes.
 *   - There is no fallback path: each call runs the hand-written kernel named by
 *     q4_last_kernel(), or fails.
 */
#ifndef Q4_H
#define Q4_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,    /* a required pointer is NULL */
    Q4_ERR_SHAPE = 2,   /* n, k or m out of range, or k not a multiple of group_size */
    Q4_ERR_GROUP = 3,   /* group_size not in {32, 64, 128} */
    Q4_ERR_DTYPE = 4,   /* dtype not accepted by this entry point */
    Q4_ERR_ALIGN = 5,   /* a pointer misses its required alignment */
    Q4_ERR_LAUNCH = 6,  /* the HIP runtime rejected the kernel launch */
    Q4_ERR_SCRATCH = 7, /* the sizes need more scratch than q4_kv_attention_noalloc holds */
    /* never returned: they make every int32 a value of the type, so a code or dtype
     * outside the list above (which the library rejects) is still a valid argument */
    Q4_STATUS_INT_MIN_ = -2147483647 - 1,
    Q4_STATUS_INT_MAX_ = 2147483647
} q4_status;

typedef enum {
    Q4_F32 = 0,
    Q4_F16 = 1,
    Q4_BF16 = 2,
    Q4_DTYPE_INT_MIN_ = -2147483647 - 1, /* never accepted; see q4_status */
    Q4_DTYPE_INT_MAX_ = 2147483647
} q4_dtype;

/* RTN quantize-and-pack of W [n][k] (F32, F16 or BF16) into the packed format.
 *   q = clamp(round(w/s) + z, q_min, q_max)      [FL7] §Affine Quantization
 * with, per group, computed in fp32:
 *   asymmetric: s = (max(x_max,0) - min(x_min,0)) / 15, z = clamp(round(-min(x_min,0)/S), 0, 15)
 *               ([FL7] §Symmetric과 Asymmetric, zero kept exactly representable);
 *   symmetric:  s = max|x| / 7, z = 0, q in [-8, 7] stored as q + 8.
 * S is s rounded to fp16 (round-to-nearest-even); S = 0 is replaced by 1.0 and S = inf by
 * 65504; the codes are computed with S, round() is round-half-to-even, the division is
 * IEEE fp32.  Codes, scales and zeros are bit-identical to the CPU definition.
 * zeros may be NULL when symmetric != 0 (it is not written then).  Beyond the shared size
 * rules, k <= 2^28 (a row is addressed with 32-bit byte offsets). */
q4_status q4_quantize_pack(const void* w, q4_dtype w_dtype, int64_t n, int64_t k,
                           int32_t group_size, int32_t symmetric,
                           uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                           hipStream_t stream);

/* Quantize-and-pack with the clipping threshold chosen per group to minimize the
 * reconstruction error ([FL7] §Clipping Trade-off: a clipped range trades a larger error
 * on the few outliers for a finer grid on the rest; the MSE-optimal criterion
 * argmin ||x - x_dq||^2 of [QA1] §MSE-optimal).  Each group tries the clip ratios
 * alpha_i = (20 - i) / 20, i = 0..10, in that order: the q4_quantize_pack computation with
 * the range scaled by alpha (asymmetric [alpha*min(x_min,0), alpha*max(x_max,0)], the zero
 * point from -alpha*min(x_min,0) / S; symmetric alpha*max|x|), weights outside the
 * clipped range saturating at the end codes.  A candidate's error is the sum of
 * (x - S(q - z))^2 in IEEE fp64: each lane adds its g/8 consecutive weights in order and
 * the 8 lanes' sums are combined in a tree, ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)); the
 * first smallest error wins, so alpha = 1 (the q4_quantize_pack result) is kept unless
 * clipping strictly lowers the error.  Output is the same packed format: each group is
 * exactly the quantization at its chosen ratio, and that ratio's error is the smallest
 * up to the fp64 rounding of the sums (another summation order may break a near-tie the
 * other way).  Arguments, limits and errors as for q4_quantize_pack.  The search costs
 * about a dozen fp32/fp64 operations per weight and candidate: it is bound by ALU
 * throughput, not memory. */
q4_status q4_quantize_pack_mse(const void* w, q4_dtype w_dtype, int64_t n, int64_t k,
                               int32_t group_size, int32_t symmetric,
                               uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                               hipStream_t stream);

/* One matrix of a grouped quantize/pack call. */
typedef struct {
    const void* w;        /* [n][k] weights, in the dtype of the call */
    int64_t n;            /* rows (output features) */
    int64_t k;            /* columns (input features), a multiple of group_size */
    uint32_t* qweight;    /* [n][k/8] packed codes (written) */
    uint16_t* scales;     /* [n][k/g] fp16 bit patterns (written) */
    uint32_t* zeros;      /* [n][ceil(k/g/8)] zero points (written); may be NULL when symmetric */
} q4_quant_problem;

/* Quantize/pack of several matrices that share dtype, group size and mode (e.g. the seven
 * linear layers of one decoder layer) in one launch, each exactly as q4_quantize_pack
 * would: same codes, scales and zero points, bit for bit ([FL7] §Per-group, applied per
 * matrix).  Each matrix may have its own n and k.  One launch streams all of them, so
 * small matrices do not each pay a launch's ramp-up and tail.  problems is a host array
 * of 1 <= count <= 8 entries; every entry is validated as for q4_quantize_pack before
 * anything is enqueued. */
q4_status q4_quantize_pack_grouped(const q4_quant_problem* problems, int32_t count,
                                   q4_dtype w_dtype, int32_t group_size, int32_t symmetric,
                                   hipStream_t stream);

/* Path B of [FL7] §Kernel이 없으면 압축 이점이 사라진다 (full dequantization):
 *   w_out[n][k] = S * (u - z),   x_hat = s(q - z)   [FL7] §Affine Quantization
 * with z = 8 in symmetric mode.  F32 output is exact; F16 and BF16 outputs are one
 * round-to-nearest-even of the exact value. */
q4_status q4_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                     int64_t n, int64_t k, int32_t group_size, int32_t symmetric,
                     void* w_out, q4_dtype out_dtype, hipStream_t stream);

/* Path A of the same section (fused load / dequant / matmul, higher-precision
 * accumulation); W4A16 as in [YJ] §Notation (4-bit weights, 16-bit activations):
 *   y[m][n] = sum_k x[m][k] * S[n][k/g] * (u[n][k] - z[n][k/g])
 * x is [m][k] F16 or BF16; y is [m][n] fp32, accumulated in fp32.  m >= 1, and beyond
 * the shared size rules k <= 2^22, n <= 2^25 and m*n <= 2^38 (Q4_ERR_SHAPE otherwise).
 * m <= 16 runs the decode GEMV kernel.  16 < m <= 256 runs the decode GEMV on 16-row
 * chunks of x (the full chunks in grouped launches of up to 8, the rest in one more) when
 * the prefill GEMM's grid of 128 x 256 tiles fits in one round (at most 2 workgroups per
 * compute unit) and ceil(m/16) * n < 147456: then the chunks stream the weight faster
 * than the under-filled GEMM covers it.  Otherwise the prefill GEMM kernel runs.  Every
 * path meets the same accuracy bound. */
q4_status q4_w4a16_gemm(const void* x, q4_dtype x_dtype, int64_t m,
                        const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                        int64_t n, int64_t k, int32_t group_size, int32_t symmetric,
                        float* y, hipStream_t stream);

/* q4_w4a16_gemm with the output written as y_dtype: Q4_F32 (identical to q4_w4a16_gemm),
 * or Q4_F16 / Q4_BF16, the 16-bit activations that the next W4A16 layer takes ([YJ]
 * §Notation: W4A16 is 4-bit weights with 16-bit activations).  The same kernels accumulate
 * in fp32 and round each element once, to nearest even, as they store it (the output
 * epilogue): a 16-bit y is exactly the rounding of the fp32 y this call would give with
 * Q4_F32.  Accuracy: the bound above plus half an ulp of the 16-bit type (relative 2^-8
 * for bf16, 2^-11 for fp16); fp16 outputs beyond 65504 become infinities.  y alignment: 4
 * bytes for Q4_F32, 2 bytes otherwise; another y_dtype is Q4_ERR_DTYPE. */
q4_status q4_w4a16_gemm_out(const void* x, q4_dtype x_dtype, int64_t m,
                            const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                            int64_t n, int64_t k, int32_t group_size, int32_t symmetric,
                            void* y, q4_dtype y_dtype, hipStream_t stream);

/* q4_w4a16_gemm_out with a workspace for products that would leave compute units idle
 * (mid-size batches on narrow weights, [FL7] §Batch와 Context에 따라 속도가 달라진다: between
 * the bandwidth-bound decode and the compute-bound prefill).  When the product runs as the
 * GEMM and its 128 x 128 tiles number fewer than the device's compute units, its K range
 * is split into up to 16 parts of at least 512 columns: each part's fp32 partial sums go to
 * the workspace, then one pass adds the parts in a fixed order (one fp32 rounding per
 * addition, the same every call) and writes y in y_dtype.  The accuracy bound is that of
 * q4_w4a16_gemm.  workspace: device memory of at least q4_w4a16_gemm_workspace(m, n, k,
 * group_size) bytes, 16-byte aligned, contents ignored; NULL runs the product unsplit
 * (exactly as q4_w4a16_gemm_out); a non-NULL workspace that is too small is Q4_ERR_SHAPE.
 * Other arguments, rules and errors as q4_w4a16_gemm_out. */
q4_status q4_w4a16_gemm_ws(const void* x, q4_dtype x_dtype, int64_t m,
                           const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                           int64_t n, int64_t k, int32_t group_size, int32_t symmetric,
                           void* y, q4_dtype y_dtype, void* workspace, int64_t workspace_bytes,
                           hipStream_t stream);
/* Bytes of workspace q4_w4a16_gemm_ws uses for this product (m*n*4 per part), 0 when it
 * would not split it, -1 for sizes the entry points reject. */
int64_t q4_w4a16_gemm_workspace(int64_t m, int64_t n, int64_t k, int32_t group_size);

/* One problem of a grouped call: y = x . x_hat^T for one packed weight. */
typedef struct {
    const void* x;            /* [m][k] activations, in the dtype of the call */
    const uint32_t* qweight;  /* [n][k/8] packed codes */
    const uint16_t* scales;   /* [n][k/g] fp16 bit patterns */
    const uint32_t* zeros;    /* [n][ceil(k/g/8)] zero points; may be NULL when symmetric */
    int64_t n;                /* output features of this problem */
    void* y;                  /* [m][n] output: fp32 for q4_w4a16_gemm_grouped, y_dtype for
                                 q4_w4a16_gemm_grouped_out */
} q4_gemm_problem;

/* Several independent W4A16 products that share m, k, group_size, symmetry and the
 * activation dtype, e.g. the q, k, v or the gate and up projections of one decoder layer.
 * Decode is bandwidth-bound ([FL7] §Batch와 Context에 따라 속도가 달라진다), and a small
 * projection pays a launch's ramp-up and tail for little data; with m <= 16 all problems
 * run in one launch of the decode GEMV kernel when their activations fit its on-chip
 * staging, otherwise (and for m > 16) one after another.  Each y meets the same accuracy
 * bound as a q4_w4a16_gemm call on that problem (the order of the fp32 sums may differ).
 * problems is a host array of 1 <= count <= 8 entries; every entry is validated as for
 * q4_w4a16_gemm before anything is enqueued. */
q4_status q4_w4a16_gemm_grouped(const q4_gemm_problem* problems, int32_t count,
                                q4_dtype x_dtype, int64_t m, int64_t k, int32_t group_size,
                                int32_t symmetric, hipStream_t stream);

/* q4_w4a16_gemm_grouped with every y written as y_dtype (the output epilogue of
 * q4_w4a16_gemm_out; the same rules per problem). */
q4_status q4_w4a16_gemm_grouped_out(const q4_gemm_problem* problems, int32_t count,
                                    q4_dtype x_dtype, int64_t m, int64_t k, int32_t group_size,
                                    int32_t symmetric, q4_dtype y_dtype, hipStream_t stream);

/* ---- INT4 KV cache ([QA1] KV-cache chapter: §KV cache의 bandwidth 부담, §Per-token scale
 * 수식, §asym 선택 이유, §Attention에서의 결합, §INT4 group scheme; [FL7] §KV Cache
 * Quantization).  One layer's K cache, and separately its V cache, for `heads` heads of
 * head_dim d with room for t_cap tokens, is head-major: token t of head h is row
 * h * t_cap + t of the packed format above with n = heads * t_cap and k = d, i.e. groups
 * of g consecutive head dimensions with one fp16 scale and one zero point per
 * (token, head, group):
 *   qcache uint32 [heads*t_cap][d/8], scache fp16 [heads*t_cap][d/g],
 *   zcache uint32 [heads*t_cap][ceil(d/g/8)] (asymmetric only, may be NULL otherwise).
 * The pages' scheme is asymmetric with g = 32 and d = 128; symmetric codes are accepted
 * too. */

/* Append t_new tokens to a cache: kv [t_new][heads][d] (F32, F16 or BF16, the new tokens'
 * K or V as the projection produces them) is quantized per (token, head) exactly as
 * q4_quantize_pack quantizes one row, scales and zero points recomputed for every token,
 * into rows h * t_cap + t0 + t, t = 0 .. t_new-1.  A prefill writes its prompt in one call,
 * a decode step its one token.  No other row is touched.  Requires t_new >= 1, t0 >= 0,
 * t0 + t_new <= t_cap, d % group_size == 0, d <= 2^16 and heads * t_cap < 2^31 (else
 * Q4_ERR_SHAPE); dtype, pointer and alignment rules as q4_quantize_pack (kv and qcache
 * 16 bytes). */
q4_status q4_kv_quantize(const void* kv, q4_dtype kv_dtype, int64_t t_new, int64_t heads,
                         int64_t head_dim, int32_t group_size, int32_t symmetric, int64_t t_cap,
                         int64_t t0, uint32_t* qcache, uint16_t* scache, uint32_t* zcache,
                         hipStream_t stream);

/* Bytes of workspace q4_kv_attention needs for (heads, head_dim, n_tok): head_dim + 2
 * floats for each of at most ceil(n_tok * head_dim / 8192) chunks per head.  Never smaller
 * for a larger n_tok, so one workspace sized for the cache capacity serves every decode
 * step.  -1 for sizes q4_kv_attention rejects. */
int64_t q4_kv_attention_workspace(int64_t heads, int64_t head_dim, int64_t n_tok);

/* Decode attention, one query per head, over tokens 0 .. n_tok-1 of a quantized K and V
 * cache (same heads, head_dim, group_size, symmetric and t_cap):
 *   out[h][i] = sum_t softmax_t(scale * q[h] . K_hat[h][t]) * V_hat[h][t][i],
 *   K_hat = S (u - z) per group (z = 8 when symmetric), V_hat alike,
 * with the dequantization inside the kernel, so the cache is read once at 4 bits
 * ([QA1] §Attention에서의 결합).  q [heads][head_dim] F16 or BF16; out fp32
 * [heads][head_dim]; scale is the caller's (usually 1/sqrt(head_dim)).  The tokens of a
 * head are split into chunks (a rule that depends on heads, head_dim and n_tok alone, so
 * results repeat bit for bit), each reduced in `workspace` to a reference maximum, its sum
 * of exponentials and its unnormalized output; a second kernel combines each head's
 * chunks in chunk order.  workspace: device memory of at least q4_kv_attention_workspace
 * bytes, 16-byte aligned, contents on entry ignored; calls that share a workspace must
 * not run concurrently.  Arithmetic is fp32: with u = 2^-24, gamma(n) = n*u/(1-n*u) and
 * L = ceil(n_tok * head_dim / 8192) + 32 (a bound on the longest chain of fp32 additions),
 * the score error is at most delta = gamma(64) |scale| max_t sum_i |q_i| 30 S_K(t, i), and
 * |out - exact| <= 2 (delta + gamma(L + 8)) max_t |V_hat[t][i]| + gamma(L) 60 max_t S_V(t, i)
 * (exact = the same formula in exact arithmetic on the stored codes).
 * Requires head_dim in {64, 128, 256}, group_size <= head_dim, 1 <= heads <= 65536,
 * 1 <= n_tok <= t_cap, n_tok <= 2^24, heads * t_cap < 2^31 (else Q4_ERR_SHAPE; a short
 * workspace is Q4_ERR_SHAPE too); alignment: q, kq, vq, workspace 16 bytes, kz, vz, out
 * 4 bytes, ks, vs 2 bytes. */
q4_status q4_kv_attention(const void* q, q4_dtype q_dtype, int64_t heads, int64_t head_dim,
                          int64_t n_tok, int64_t t_cap, const uint32_t* kq, const uint16_t* ks,
                          const uint32_t* kz, const uint32_t* vq, const uint16_t* vs,
                          const uint32_t* vz, int32_t group_size, int32_t symmetric, float scale,
                          float* out, void* workspace, int64_t workspace_bytes,
                          hipStream_t stream);

/* q4_kv_attention for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and rules as q4_kv_attention without workspace and workspace_bytes (the same kernels,
 * chunking and summation order, so the output is bit-identical).  The per-chunk partials
 * go to a fixed scratch array of q4_kv_attention_noalloc_max_bytes() bytes (16 MiB) that
 * the library holds in device memory, one per GPU, from its first call on that GPU until
 * the process ends; the call itself allocates and frees nothing.  The partials need
 * heads * chunks * (head_dim + 2) * 4 bytes with chunks <= ceil(n_tok * head_dim / 8192)
 * (e.g. 1.06 MB for 32 heads of 128 over 4096 tokens); sizes that need more return
 * Q4_ERR_SCRATCH before anything is enqueued.  Every call on a GPU shares that GPU's
 * scratch: calls that may overlap on one GPU (other streams, other threads) race and must
 * be serialized by the caller.  The scratch needs no clearing: each call writes every
 * partial it reads. */
q4_status q4_kv_attention_noalloc(const void* q, q4_dtype q_dtype, int64_t heads, int64_t head_dim,
                                  int64_t n_tok, int64_t t_cap, const uint32_t* kq,
                                  const uint16_t* ks, const uint32_t* kz, const uint32_t* vq,
                                  const uint16_t* vs, const uint32_t* vz, int32_t group_size,
                                  int32_t symmetric, float scale, float* out, hipStream_t stream);
int64_t q4_kv_attention_noalloc_max_bytes(void);

/* ---- GPTQ ([QA1] GPTQ chapter: §Hessian 정의, §OBQ single-step 수식, §GPTQ block-wise,
 * §알고리즘 개요, §설정 grid; [FL7] §GPTQ: Approximate Second-order Weight Quantization).
 * Quantize W [n][k] (F32, F16 or BF16) into the packed format with the quantization
 * error of each column carried into the columns not yet quantized, weighted by the
 * calibration Hessian H = 2 X^T X of x [tokens][k] (F16 or BF16 activations):
 *   - the group scales and zero points are q4_quantize_pack's on the original W (fixed
 *     before the sweep, "static groups"; the format's groups are g consecutive columns);
 *   - H's diagonal is scaled by 1 + damp (the pages use damp = 0.01); a zero diagonal entry
 *     (a feature never active) becomes 1 first; 0 < damp <= 1;
 *   - columns are taken in natural order (q4_gptq_quantize_act_order below takes them by
 *     activation energy); column j is quantized at w_j + sum_{i<j} d_i U_ij / U_jj,
 *     d_i = w_i - w_hat_i, H = U U^T with U upper triangular: the pages' update
 *     err_j = (w'_j - w_hat_j) / L_jj, w'_l -= err_j L_jl with H^-1 = L^T L, without the
 *     inverse.
 * All arithmetic is fp32 (Hessian, Cholesky factor, updates); a code can differ from an
 * exact-arithmetic sweep where the updated weight falls within rounding of a code
 * boundary.  workspace: device memory of at least q4_gptq_workspace(n, k, group_size)
 * bytes (k*k + n*k + 256*n floats), 16-byte aligned, contents ignored; k <= 32768.  Other
 * rules as q4_quantize_pack; x 16-byte aligned.  Runs about 5k/64 kernels on `stream`. */
int64_t q4_gptq_workspace(int64_t n, int64_t k, int32_t group_size);
q4_status q4_gptq_quantize(const void* w, q4_dtype w_dtype, int64_t n, int64_t k, const void* x,
                           q4_dtype x_dtype, int64_t tokens, int32_t group_size, int32_t symmetric,
                           float damp, uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                           void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* GPTQ with act-order ([QA1] GPTQ chapter, §설정 grid: the columns whose activations have
 * the largest |X|^2 are quantized first, so less error accumulates on them): as
 * q4_gptq_quantize, but the sweep takes the columns by descending energy
 * e_i = sum_t x_ti^2 (fp32, summed over slices of 32 tokens and then across slices; equal
 * energies by the lower column index; a feature never active comes last).  Every column
 * keeps its own group's scale and zero point (the static RTN quantizers), so the output
 * format and its group layout are unchanged; only the order in which codes are chosen and
 * errors carried differs.  workspace: at least q4_gptq_act_order_workspace(n, k, group_size)
 * bytes (the q4_gptq_workspace floats, 3*k more, and n*k bytes of codes).  Other arguments,
 * rules and errors as q4_gptq_quantize.  About 5k/64 + 6 kernels on `stream`. */
int64_t q4_gptq_act_order_workspace(int64_t n, int64_t k, int32_t group_size);
q4_status q4_gptq_quantize_act_order(const void* w, q4_dtype w_dtype, int64_t n, int64_t k,
                                     const void* x, q4_dtype x_dtype, int64_t tokens,
                                     int32_t group_size, int32_t symmetric, float damp,
                                     uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                                     void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* Element counts of the three packed arrays (payload + metadata, [FL7] §Memory 계산은
 * Payload와 Metadata로 나눈다): n*k/8 words, n*(k/g) scales, n*ceil((k/g)/8) words.
 * Return -1 for arguments the entry points would reject. */
/* Corrupted scale detection ([FL7] §Quantized Artifact Security, Runtime: a loaded
 * quantized artifact is checked, not trusted).  Every scale this format stores is an fp16
 * value >= 0 (a group's range over 15 or its largest magnitude over 7, rounded; 0 or -0 for
 * a group of zeros), so a scale that is infinite, NaN or negative (sign set, nonzero
 * magnitude) marks a corrupted artifact.  scales: [n][k/group_size] fp16 bits, 2-byte
 * aligned.  result: device memory of 3 int64, 8-byte aligned, overwritten (no clearing
 * needed): [0] the number of non-finite scales, [1] the number of negative scales, [2] the
 * flat index n*(k/g)+g of the first bad scale, or -1 when there is none.  Asynchronous on
 * stream, like the other calls; the values are exact integers whatever the launch order.
 * Errors: Q4_ERR_GROUP, Q4_ERR_SHAPE (as q4_dequant), Q4_ERR_NULL, Q4_ERR_ALIGN. */
q4_status q4_check_scales(const uint16_t* scales, int64_t n, int64_t k, int32_t group_size,
                          int64_t* result, hipStream_t stream);

int64_t q4_qweight_words(int64_t n, int64_t k);
int64_t q4_scale_count(int64_t n, int64_t k, int32_t group_size);
int64_t q4_zero_words(int64_t n, int64_t k, int32_t group_size);

/* Static description of a status code. */
const char* q4_status_str(q4_status s);

/* Name of the kernel the calling thread's last successful entry-point call enqueued
 * ("" before any), so callers can verify which kernel ran ([FL7] §Silent Fallback). */
const char* q4_last_kernel(void);

/* Every kernel the calling thread's last successful entry-point call enqueued: their
 * distinct names in launch order, comma-separated (a multi-launch call, such as a chunked
 * mid-m product, attention's partial and combine kernels or GPTQ, lists each), and the
 * number of launches.  "" and 0 before any call.  [FL7] §Silent Fallback asks to check the
 * selected kernel and that nothing fell back. */
const char* q4_last_kernels(void);
int64_t q4_last_launch_count(void);

/* Version of the packed layout described above (1). */
int32_t q4_layout_version(void);

/* Digest of the sources this library was built from (the first 16 hex digits of a SHA-256
 * over the kernel sources and this header, as the build computes it), so a loader can
 * refuse a library built from other sources ([FL7] lists the quantizer code version among
 * what a deployment must be able to reproduce). */
const char* q4_source_digest(void);

#ifdef __cplusplus
}
#endif
#endif
