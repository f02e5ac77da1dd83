/* q4_oracle.c — plain, slow CPU oracle for group-wise affine INT4 (W4A16).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the benchmark's
 * CPU-baseline leg, never by the GPU library.  Built with gcc -O2 -ffp-contract=off and
 * no fast-math, so every float operation below is one IEEE binary32 (or binary64)
 * operation in round-to-nearest-even, in the order written.
 *
 * Page names are abbreviated as in q4_oracle.h ([FL7], [QA1]).
 *
 * Readings taken where the pages leave a step open (each listed in the design notes):
 *   R1 group = g consecutive input columns of one output row ([FL7] §Per-group);
 *   R2 round() is round-half-to-even in fp32 (rintf in the default rounding mode);
 *   R3 q = clamp(round(x/s) + z): round first, then add the integer zero point, exactly
 *      as the affine formula of [FL7] §Affine Quantization is written;
 *   R4 the scale used to quantize is the stored fp16 one (S), so dequantization uses
 *      exactly the scale the codes were computed against;
 *   R5 asymmetric range is zero-extended [min(x_min,0), max(x_max,0)] so zero is exactly
 *      representable, which [FL7] §Asymmetric asks the rounding and clamping to ensure;
 *   R6 symmetric: s = max|x| / 7, q clamped to [-8, 7] ([FL7] §Symmetric with q_max = 7;
 *      [QA1] §Signed ↔ Unsigned gives INT4 signed [-8, 7]); stored as u = q + 8;
 *   R7 degenerate scales: fp16(s) == 0 -> 1.0, fp16(s) == +inf -> 65504;
 *   R8 layout: little-endian nibbles in uint32 words, row-major.
 */
#include "q4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 / bf16 */

uint16_t orc_f32_to_f16_rne(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t exp32 = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;
    if (exp32 == 0xFFu) /* inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    int32_t e = (int32_t)exp32 - 127 + 15; /* binary16 biased exponent */
    if (e >= 31) return (uint16_t)(sign | 0x7C00u);
    if (e >= 1) {
        /* normal: keep 10 mantissa bits, round the 13 dropped bits to nearest even */
        uint32_t h = ((uint32_t)e << 10) | (man >> 13);
        uint32_t rem = man & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* carry may reach inf */
        return (uint16_t)(sign | h);
    }
    /* subnormal (or zero) in binary16: value = mm * 2^(exp32-150), unit 2^-24 */
    if (exp32 == 0) return (uint16_t)sign; /* fp32 zero/subnormal is < 2^-126: rounds to 0 */
    uint32_t mm = man | 0x800000u;             /* 24-bit significand */
    int32_t shift = 126 - (int32_t)exp32;      /* = 14 - e, >= 14 */
    if (shift > 25) return (uint16_t)sign;     /* |f| < 2^-25: below half the smallest step */
    uint32_t h = mm >> shift;
    uint32_t rem = mm & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) h += 1u; /* may become the min normal */
    return (uint16_t)(sign | h);
}

float orc_f16_to_f32(uint16_t h) {
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = ((uint32_t)h >> 10) & 0x1Fu;
    uint32_t m = (uint32_t)h & 0x3FFu;
    float mag;
    if (e == 0) {
        mag = ldexpf((float)m, -24); /* subnormal (exact) */
    } else if (e == 31) {
        mag = m ? NAN : INFINITY;
    } else {
        mag = ldexpf((float)(m | 0x400u), (int)e - 25);
    }
    uint32_t bits;
    memcpy(&bits, &mag, 4);
    bits |= sign;
    float out;
    memcpy(&out, &bits, 4);
    return out;
}

float orc_bf16_to_f32(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float out;
    memcpy(&out, &bits, 4);
    return out;
}

static float load_elem(const void* p, int dtype, int64_t idx) {
    switch (dtype) {
    case ORC_F32: return ((const float*)p)[idx];
    case ORC_F16: return orc_f16_to_f32(((const uint16_t*)p)[idx]);
    default:      return orc_bf16_to_f32(((const uint16_t*)p)[idx]);
    }
}

/* ---------------------------------------------------------------- sizes */

int64_t orc_qweight_words(int64_t n, int64_t k) { return n * (k / 8); }
int64_t orc_scale_count(int64_t n, int64_t k, int64_t g) { return n * (k / g); }
int64_t orc_zero_words(int64_t n, int64_t k, int64_t g) { return n * ((k / g + 7) / 8); }

/* ---------------------------------------------------------------- quantize + pack */

static float clampf(float v, float lo, float hi) {
    /* fmaxf/fminf return the non-NaN operand, so a NaN quotient lands on lo. */
    return fminf(fmaxf(v, lo), hi);
}

int orc_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g,
                      int symmetric, uint32_t* qweight, uint16_t* scales,
                      uint32_t* zeros, uint8_t* onesided) {
    if (n < 0 || k < 0 || g < 1 || k % g != 0 || k % 8 != 0) return -1;
    const int64_t G = k / g;
    const int64_t zw = (G + 7) / 8;
    /* integer code range of the format ([QA1] §Signed ↔ Unsigned, INT4) */
    const float q_min = symmetric ? -8.0f : 0.0f;
    const float q_max = symmetric ? 7.0f : 15.0f;

    memset(qweight, 0, (size_t)(n * (k / 8)) * sizeof(uint32_t));
    if (!symmetric) memset(zeros, 0, (size_t)(n * zw) * sizeof(uint32_t));

    float* v = (float*)malloc((size_t)g * sizeof(float));
    if (!v) return -1;
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t j = 0; j < G; ++j) {
            /* the group: g consecutive input columns of this row (R1) */
            for (int64_t t = 0; t < g; ++t) v[t] = load_elem(w, w_dtype, row * k + j * g + t);

            float s;           /* scale before storage, fp32 */
            float x_min = 0.0f, x_max = 0.0f; /* zero-extended range (R5) */
            float lit_min = v[0], lit_max = v[0]; /* literal range, diagnostics only */
            if (symmetric) {
                /* s = max|x| / q_max ([FL7] §Symmetric) */
                float amax = 0.0f;
                for (int64_t t = 0; t < g; ++t) amax = fmaxf(amax, fabsf(v[t]));
                s = amax / 7.0f;
            } else {
                /* s = (x_max - x_min) / (q_max - q_min) ([FL7] §Asymmetric) */
                for (int64_t t = 0; t < g; ++t) {
                    x_min = fminf(x_min, v[t]);
                    x_max = fmaxf(x_max, v[t]);
                    lit_min = fminf(lit_min, v[t]);
                    lit_max = fmaxf(lit_max, v[t]);
                }
                s = (x_max - x_min) / 15.0f;
            }
            /* stored fp16 scale, degenerate values replaced (R7) */
            uint16_t s16 = orc_f32_to_f16_rne(s);
            if ((s16 & 0x7FFFu) == 0) s16 = 0x3C00u;  /* 1.0 */
            if (s16 == 0x7C00u) s16 = 0x7BFFu;        /* 65504 */
            const float S = orc_f16_to_f32(s16);      /* the scale the codes use (R4) */
            scales[row * G + j] = s16;

            /* zero point z ≈ q_min - x_min / s, rounded and clamped ([FL7] §Asymmetric) */
            int z = 0;
            if (!symmetric) {
                float zf = clampf(rintf(-x_min / S), q_min, q_max);
                z = (int)zf;
                zeros[row * zw + j / 8] |= (uint32_t)z << (4 * (j % 8));
                if (onesided) onesided[row * G + j] = (uint8_t)(lit_min > 0.0f || lit_max < 0.0f);
            } else if (onesided) {
                onesided[row * G + j] = 0;
            }

            for (int64_t t = 0; t < g; ++t) {
                /* q = clamp(round(x / s) + z, q_min, q_max) ([FL7] §Affine Quantization) */
                float qf = clampf(rintf(v[t] / S) + (float)z, q_min, q_max);
                int q = (int)qf;
                uint32_t u = (uint32_t)(symmetric ? q + 8 : q); /* stored code (R6) */
                int64_t col = j * g + t;
                qweight[row * (k / 8) + col / 8] |= u << (4 * (col % 8));
            }
        }
    }
    free(v);
    return 0;
}

/* ---------------------------------------------------------------- MSE-optimal clipping */

/* Clip search per group ([FL7] §Clipping Trade-off: pick the clipping threshold that
 * minimizes the local reconstruction error; [QA1] §MSE-optimal: argmin ||x - x_dq||^2).
 * Readings where the pages leave the search open:
 *   M1 candidates: clip ratios alpha_i = (20 - i) / 20 in fp32, i = 0..10 (1.0 down to 0.5),
 *      tried in that order;
 *   M2 a candidate quantizes exactly as RTN does (R1-R8) with its range scaled by alpha:
 *      asymmetric [alpha*min(x_min,0), alpha*max(x_max,0)], symmetric alpha*max|x|, each
 *      product one fp32 rounding; the zero point divides -alpha*min(x_min,0) by S in fp32;
 *      weights outside the clipped range saturate at the end codes;
 *   M3 the error of a candidate is sum over the group of (x - S*(q - z))^2 in IEEE binary64,
 *      each difference and square one binary64 rounding, the terms added one by one in
 *      column order: the plain definition, no blocking;
 *   M4 the candidate with the smallest error wins; an equal error keeps the earlier
 *      (larger) ratio, so alpha = 1 (plain RTN) wins unless clipping strictly helps. */
#define ORC_MSE_CANDIDATES 11

/* scale, zero point and codes of one group for clip ratio alpha; returns the error (M3) */
static double mse_candidate(const float* v, int64_t g, int symmetric, float alpha,
                            uint16_t* s16_out, int* z_out, int* q_out) {
    float s, lo = 0.0f;
    if (symmetric) {
        float amax = 0.0f;
        for (int64_t t = 0; t < g; ++t) amax = fmaxf(amax, fabsf(v[t]));
        s = (alpha * amax) / 7.0f;
    } else {
        float x_min = 0.0f, x_max = 0.0f;
        for (int64_t t = 0; t < g; ++t) {
            x_min = fminf(x_min, v[t]);
            x_max = fmaxf(x_max, v[t]);
        }
        lo = alpha * x_min;
        const float hi = alpha * x_max;
        s = (hi - lo) / 15.0f;
    }
    uint16_t s16 = orc_f32_to_f16_rne(s);
    if ((s16 & 0x7FFFu) == 0) s16 = 0x3C00u;
    if (s16 == 0x7C00u) s16 = 0x7BFFu;
    const float S = orc_f16_to_f32(s16);
    const float q_min = symmetric ? -8.0f : 0.0f;
    const float q_max = symmetric ? 7.0f : 15.0f;
    int z = 0;
    if (!symmetric) z = (int)clampf(rintf(-lo / S), q_min, q_max);
    double err = 0.0;
    for (int64_t t = 0; t < g; ++t) {
        const int q = (int)clampf(rintf(v[t] / S) + (float)z, q_min, q_max);
        if (q_out) q_out[t] = q;
        const double xhat = (double)S * (double)(q - z);
        const double d = (double)v[t] - xhat;
        err = err + d * d;
    }
    *s16_out = s16;
    *z_out = z;
    return err;
}

/* The clip search over a whole matrix.  ratio == NULL: each group scans the ratios (M1, M4);
 * otherwise group (row, j) is quantized at ratio index ratio[row*G + j] without a search.
 * errors (may be NULL) receives every candidate's error, [n][G][ORC_MSE_CANDIDATES]. */
static int mse_matrix(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g, int symmetric,
                      const uint8_t* ratio, uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                      uint8_t* choice, double* errors) {
    if (n < 0 || k < 0 || g < 8 || g % 8 != 0 || k % g != 0 || k % 8 != 0) return -1;
    const int64_t G = k / g;
    const int64_t zw = (G + 7) / 8;
    if (qweight) memset(qweight, 0, (size_t)(n * (k / 8)) * sizeof(uint32_t));
    if (zeros && !symmetric) memset(zeros, 0, (size_t)(n * zw) * sizeof(uint32_t));
    float* v = (float*)malloc((size_t)g * sizeof(float));
    int* q = (int*)malloc((size_t)g * sizeof(int));
    if (!v || !q) {
        free(v);
        free(q);
        return -1;
    }
    int rc = 0;
    for (int64_t row = 0; row < n && rc == 0; ++row) {
        for (int64_t j = 0; j < G; ++j) {
            for (int64_t t = 0; t < g; ++t) v[t] = load_elem(w, w_dtype, row * k + j * g + t);
            int best = 0;
            if (ratio) {
                best = ratio[row * G + j];
                if (best >= ORC_MSE_CANDIDATES) {
                    rc = -1;
                    break;
                }
            }
            if (!ratio || errors) {
                /* M1, M4: scan the ratios, keep the first smallest error */
                double best_err = 0.0;
                for (int i = 0; i < ORC_MSE_CANDIDATES; ++i) {
                    const float alpha = (float)(20 - i) / 20.0f;
                    uint16_t s16;
                    int z;
                    const double e = mse_candidate(v, g, symmetric, alpha, &s16, &z, NULL);
                    if (errors) errors[(row * G + j) * ORC_MSE_CANDIDATES + i] = e;
                    if (!ratio && (i == 0 || e < best_err)) {
                        best = i;
                        best_err = e;
                    }
                }
            }
            if (choice) choice[row * G + j] = (uint8_t)best;
            if (!qweight) continue;
            uint16_t s16;
            int z;
            mse_candidate(v, g, symmetric, (float)(20 - best) / 20.0f, &s16, &z, q);
            scales[row * G + j] = s16;
            if (!symmetric) zeros[row * zw + j / 8] |= (uint32_t)z << (4 * (j % 8));
            for (int64_t t = 0; t < g; ++t) {
                const uint32_t u = (uint32_t)(symmetric ? q[t] + 8 : q[t]);
                const int64_t col = j * g + t;
                qweight[row * (k / 8) + col / 8] |= u << (4 * (col % 8));
            }
        }
    }
    free(v);
    free(q);
    return rc;
}

int orc_quantize_pack_mse(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g,
                          int symmetric, uint32_t* qweight, uint16_t* scales, uint32_t* zeros,
                          uint8_t* choice) {
    return mse_matrix(w, w_dtype, n, k, g, symmetric, NULL, qweight, scales, zeros, choice, NULL);
}

int orc_quantize_pack_clip(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g,
                           int symmetric, const uint8_t* ratio, uint32_t* qweight,
                           uint16_t* scales, uint32_t* zeros) {
    if (!ratio) return -1;
    return mse_matrix(w, w_dtype, n, k, g, symmetric, ratio, qweight, scales, zeros, NULL, NULL);
}

int orc_mse_errors(const void* w, int w_dtype, int64_t n, int64_t k, int64_t g, int symmetric,
                   double* errors) {
    if (!errors) return -1;
    return mse_matrix(w, w_dtype, n, k, g, symmetric, NULL, NULL, NULL, NULL, NULL, errors);
}

/* ---------------------------------------------------------------- dequant */

static double xhat_elem(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                        int64_t row, int64_t col, int64_t k, int64_t g, int symmetric) {
    const int64_t G = k / g;
    const int64_t zw = (G + 7) / 8;
    const int64_t j = col / g;
    uint32_t u = (qweight[row * (k / 8) + col / 8] >> (4 * (col % 8))) & 0xFu;
    uint32_t z = symmetric ? 8u : (zeros[row * zw + j / 8] >> (4 * (j % 8))) & 0xFu;
    double S = (double)orc_f16_to_f32(scales[row * G + j]);
    /* x_hat = s (q - z) ([FL7] §Affine Quantization, dequantization) */
    return S * ((double)u - (double)z);
}

int orc_dequant_f64(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                    int64_t n, int64_t k, int64_t g, int symmetric, double* out) {
    if (n < 0 || k < 0 || g < 1 || k % g != 0 || k % 8 != 0) return -1;
    for (int64_t row = 0; row < n; ++row)
        for (int64_t col = 0; col < k; ++col)
            out[row * k + col] = xhat_elem(qweight, scales, zeros, row, col, k, g, symmetric);
    return 0;
}

/* ---------------------------------------------------------------- linear */

int orc_linear_f64(const void* x, int x_dtype, int64_t m, const int64_t* rows, int64_t n_rows,
                   const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                   int64_t n, int64_t k, int64_t g, int symmetric,
                   const int64_t* cols, int64_t n_cols, double* y, double* yabs) {
    if (m < 0 || n < 0 || k < 0 || g < 1 || k % g != 0 || k % 8 != 0) return -1;
    const int64_t nr = rows ? n_rows : m;
    const int64_t nc = cols ? n_cols : n;
    double* wrow = (double*)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
    if (!wrow) return -1;
    for (int64_t ci = 0; ci < nc; ++ci) {
        const int64_t col_n = cols ? cols[ci] : ci;
        if (col_n < 0 || col_n >= n) { free(wrow); return -1; }
        for (int64_t kk = 0; kk < k; ++kk)
            wrow[kk] = xhat_elem(qweight, scales, zeros, col_n, kk, k, g, symmetric);
        for (int64_t ri = 0; ri < nr; ++ri) {
            const int64_t row_m = rows ? rows[ri] : ri;
            if (row_m < 0 || row_m >= m) { free(wrow); return -1; }
            /* y = x · x_hat^T, accumulated in fp64 */
            double acc = 0.0, aabs = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) {
                double xv = (double)load_elem(x, x_dtype, row_m * k + kk);
                acc += xv * wrow[kk];
                aabs += fabs(xv) * fabs(wrow[kk]);
            }
            y[ri * nc + ci] = acc;
            if (yabs) yabs[ri * nc + ci] = aabs;
        }
    }
    free(wrow);
    return 0;
}

/* ---------------------------------------------------------------- KV cache */

/* [QA1] KV-cache chapter, §INT4 group scheme and §asym 선택 이유: the K (or V) row of one
 * token and one head, d values, is quantized in groups of g consecutive head dimensions,
 * each group with its own scale and zero point, recomputed for every token as it arrives
 * (per-token scales, §Per-token scale 수식).  The group quantizer is the RTN of
 * orc_quantize_pack.  Reading K1: one layer's cache is head-major, token t of head h in row
 * h * t_cap + t of the packed layout with k = d. */
int orc_kv_quantize(const void* kv, int dtype, int64_t t_new, int64_t heads, int64_t d, int64_t g,
                    int symmetric, int64_t t_cap, int64_t t0, uint32_t* qcache,
                    uint16_t* scache, uint32_t* zcache) {
    if (t_new < 0 || heads < 1 || d < 1 || g < 1 || d % g != 0 || d % 8 != 0) return -1;
    if (t0 < 0 || t0 + t_new > t_cap) return -1;
    const int64_t G = d / g;
    const int64_t zw = (G + 7) / 8;
    const size_t esize = dtype == ORC_F32 ? 4 : 2;
    for (int64_t t = 0; t < t_new; ++t) {
        for (int64_t h = 0; h < heads; ++h) {
            const char* src = (const char*)kv + (size_t)((t * heads + h) * d) * esize;
            const int64_t r = h * t_cap + t0 + t;
            const int rc = orc_quantize_pack(src, dtype, 1, d, g, symmetric, qcache + r * (d / 8),
                                             scache + r * G, symmetric ? NULL : zcache + r * zw,
                                             NULL);
            if (rc != 0) return rc;
        }
    }
    return 0;
}

/* Decode attention over the quantized cache, in fp64 ([QA1] KV-cache chapter, §Attention에서의
 * 결합: the dequantized K and V enter the attention matmuls).  For each head h, with the
 * cached tokens t = 0 .. n_tok-1 dequantized as in orc_dequant_f64 (x_hat = S (u - z)):
 *   s_t = scale * sum_i q[h][i] K_hat[h][t][i]
 *   out[h][i] = sum_t exp(s_t - M) V_hat[h][t][i] / sum_t exp(s_t - M),  M = max_t s_t
 * (softmax; subtracting M changes nothing mathematically and keeps exp in range).
 * score_abs[h] (may be NULL) = max_t |scale| sum_i |q[h][i]| |K_hat[h][t][i]| and
 * v_abs[h][i] (may be NULL) = max_t |V_hat[h][t][i]|: the tolerance references. */
int orc_kv_attention_f64(const void* q, int q_dtype, int64_t heads, int64_t d, int64_t n_tok,
                         int64_t t_cap, const uint32_t* kq, const uint16_t* ks, const uint32_t* kz,
                         const uint32_t* vq, const uint16_t* vs, const uint32_t* vz, int64_t g,
                         int symmetric, double scale, double* out, double* score_abs,
                         double* v_abs) {
    if (heads < 1 || d < 1 || n_tok < 1 || n_tok > t_cap || g < 1 || d % g != 0 || d % 8 != 0)
        return -1;
    double* s = (double*)malloc((size_t)n_tok * sizeof(double));
    double* qh = (double*)malloc((size_t)d * sizeof(double));
    if (!s || !qh) { free(s); free(qh); return -1; }
    for (int64_t h = 0; h < heads; ++h) {
        for (int64_t i = 0; i < d; ++i) qh[i] = (double)load_elem(q, q_dtype, h * d + i);
        double M = -HUGE_VAL, sabs_max = 0.0;
        for (int64_t t = 0; t < n_tok; ++t) {
            const int64_t r = h * t_cap + t;
            double acc = 0.0, aabs = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                const double kh = xhat_elem(kq, ks, kz, r, i, d, g, symmetric);
                acc += qh[i] * kh;
                aabs += fabs(qh[i]) * fabs(kh);
            }
            s[t] = scale * acc;
            if (s[t] > M) M = s[t];
            if (fabs(scale) * aabs > sabs_max) sabs_max = fabs(scale) * aabs;
        }
        double l = 0.0;
        for (int64_t t = 0; t < n_tok; ++t) {
            s[t] = exp(s[t] - M);  /* now the unnormalized probability */
            l += s[t];
        }
        for (int64_t i = 0; i < d; ++i) {
            double acc = 0.0, vmax = 0.0;
            for (int64_t t = 0; t < n_tok; ++t) {
                const double vh = xhat_elem(vq, vs, vz, h * t_cap + t, i, d, g, symmetric);
                acc += s[t] * vh;
                if (fabs(vh) > vmax) vmax = fabs(vh);
            }
            out[h * d + i] = acc / l;
            if (v_abs) v_abs[h * d + i] = vmax;
        }
        if (score_abs) score_abs[h] = sabs_max;
    }
    free(s);
    free(qh);
    return 0;
}
