/* q4_oracle.h — plain, slow CPU oracle for group-wise affine INT4 (W4A16).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  It shares no source, header, table or helper
 * with the GPU library, and the GPU library never calls it.
 *
 * Sources (the pages this follows; sections named, no line numbers):
 *   [FL7]  "LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)", blog.ruahverce.com
 *          §Affine Quantization, §Bit 수와 Level 수 (bits and levels),
 *          §Symmetric과 Asymmetric, §Granularity / Per-group,
 *          §Memory 계산은 Payload와 Metadata로 나눈다 (payload + metadata),
 *          §Group Scale Overhead 예, §어떤 Tensor를 Quantize하는가 / Weight-only,
 *          §Kernel이 없으면 압축 이점이 사라진다 (path A fused / path B full dequant).
 *   [QA1]  "Quantization Algorithms 단권화", brianyu43.github.io (V10)
 *          §Uniform Symmetric, §Signed ↔ Unsigned (INT4 ranges), §Calibration-free (RTN),
 *          §MSE-optimal; KV-cache chapter: §KV cache의 bandwidth 부담, §Per-token scale 수식,
 *          §asym 선택 이유, §Attention에서의 결합, §INT4 group scheme.
 *
 * Parity status: every function here is pinned by tests (hand-worked groups, closed
 * forms, invariants, brute force, an independent fp16 converter); none is
 * "parity unpinned".
 *
 * Layout produced (row-major, n output rows, k input columns, groups of g consecutive
 * columns within one row, G = k/g):
 *   qweight : uint32 [n][k/8]; code of column 8j+i sits in bits 4i..4i+3 of word j.
 *   scales  : fp16 bit patterns [n][G].
 *   zeros   : uint32 [n][ceil(G/8)]; zero point of group 8j+i in bits 4i..4i+3 of word
 *             j; pad nibbles 0.  Asymmetric only (left untouched when symmetric).
 * Stored code u: asymmetric u = q in [0,15]; symmetric u = q + 8 with q in [-8,7].
 */
#ifndef Q4_ORACLE_H
#define Q4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* fp32 -> fp16 with round-to-nearest-even, subnormals kept, overflow to +-inf,
 * NaN kept NaN.  Written from the IEEE 754 binary16 definition. */
uint16_t orc_f32_to_f16_rne(float f);
/* Exact widenings. */
float orc_f16_to_f32(uint16_t h);
float orc_bf16_to_f32(uint16_t b);

/* onesided[n*G] (diagnostics, may be NULL) = 1 when the group's literal range excludes
 * zero (all values > 0 or all < 0), i.e. the zero-extended asymmetric range differs
 * from the literal [x_min, x_max]. */
/* Returns 0 on success, -1 on bad arguments (k % g != 0, k % 8 != 0, g < 1). */
int orc_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g,
                      int symmetric, uint32_t* qweight, uint16_t* scales,
                      uint32_t* zeros, uint8_t* onesided);

/* MSE-optimal clip search ([FL7] §Clipping Trade-off; [QA1] §MSE-optimal): per group, the
 * RTN quantization of the range scaled by each clip ratio alpha_i = (20 - i) / 20,
 * i = 0..10, scored by the fp64 squared reconstruction error summed in column order; the
 * first smallest error wins (alpha = 1 is plain RTN).
 * Same packed layout as orc_quantize_pack.  choice[n*G] (may be NULL) receives i.
 * Returns 0 on success, -1 on bad arguments (also g % 8 != 0). */
int orc_quantize_pack_mse(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g,
                          int symmetric, uint32_t* qweight, uint16_t* scales,
                          uint32_t* zeros, uint8_t* choice);

/* The same quantization with the clip ratio given per group instead of searched:
 * ratio[n*G] holds i (alpha = (20 - i) / 20), i < 11.  -1 on bad arguments or ratio. */
int orc_quantize_pack_clip(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g,
                           int symmetric, const uint8_t* ratio, uint32_t* qweight,
                           uint16_t* scales, uint32_t* zeros);

/* Every candidate's error of the clip search, errors[n][G][11] (i = 0..10 in order), each
 * summed as orc_quantize_pack_mse sums it.  -1 on bad arguments. */
int orc_mse_errors(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g, int symmetric,
                   double* errors);

/* x_hat[n][k] = S * (u - z) in fp64 (exact), z = stored zero (asym) or 8 (sym). */
int orc_dequant_f64(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                    int64_t n, int64_t k, int64_t g, int symmetric, double* out);

/* y[mi][ni] = sum_k x[m][k] * x_hat[n][k] in fp64 for every (m, n) in rows x cols,
 * where m = rows[mi], n = cols[ni] (pass rows=NULL / cols=NULL for all of [0,m) / [0,n)).
 * yabs gets sum_k |x[m][k]| * |x_hat[n][k]| (the tolerance reference), may be NULL.
 * x is [m][k] in x_dtype (F32, F16 or BF16). */
int orc_linear_f64(const void* x, int x_dtype, int64_t m, const int64_t* rows, int64_t n_rows,
                   const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                   int64_t n, int64_t k, int64_t g, int symmetric,
                   const int64_t* cols, int64_t n_cols, double* y, double* yabs);

/* KV cache ([QA1] KV-cache chapter, §INT4 group scheme): kv [t_new][heads][d] (new tokens)
 * quantized per (token, head) in groups of g along d, as orc_quantize_pack does for one row,
 * into rows h * t_cap + t0 + t of a head-major cache in the packed layout with k = d
 * (qcache [heads*t_cap][d/8], scache [heads*t_cap][d/g], zcache [heads*t_cap][ceil(d/g/8)],
 * zcache untouched and may be NULL when symmetric).  Other rows are left as they are.
 * Returns 0, or -1 on bad arguments (t0 + t_new > t_cap, d % g != 0, ...). */
int orc_kv_quantize(const void* kv, int dtype, int64_t t_new, int64_t heads, int64_t d, int64_t g,
                    int symmetric, int64_t t_cap, int64_t t0, uint32_t* qcache,
                    uint16_t* scache, uint32_t* zcache);

/* Decode attention over the first n_tok tokens of that cache, fp64:
 * out[h][i] = sum_t softmax_t(scale * q[h] . K_hat[h][t]) V_hat[h][t][i], q [heads][d] in
 * q_dtype.  score_abs[heads] = max_t |scale| sum_i |q_i K_hat_ti| and v_abs[heads][d] =
 * max_t |V_hat_ti| (both may be NULL) are the tolerance references. */
int orc_kv_attention_f64(const void* q, int q_dtype, int64_t heads, int64_t d, int64_t n_tok,
                         int64_t t_cap, const uint32_t* kq, const uint16_t* ks, const uint32_t* kz,
                         const uint32_t* vq, const uint16_t* vs, const uint32_t* vz, int64_t g,
                         int symmetric, double scale, double* out, double* score_abs,
                         double* v_abs);

/* Sizes of the three arrays, in elements of their own type. */
int64_t orc_qweight_words(int64_t n, int64_t k);
int64_t orc_scale_count(int64_t n, int64_t k, int64_t g);
int64_t orc_zero_words(int64_t n, int64_t k, int64_t g);

#ifdef __cplusplus
}
#endif
#endif
