"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle's C source, plants one plausible mistake (a wrong rounding
order, a dropped term, a wrong sign or index, a swapped operand ...), compiles the copy
on the CPU and runs every pin against it.  At least one pin has to fail; a mutant that
passes every pin would mean the pins cannot tell that mistake from the real definition.
"""
import os

import pytest

import oracle
import pins

MUTANTS = [
    ("add_then_round", "float qf = clampf(rintf(v[t] / S) + (float)z,",
     "float qf = clampf(rintf(v[t] / S + (float)z),"),
    ("quantize_with_fp32_scale", "float qf = clampf(rintf(v[t] / S) + (float)z,",
     "float qf = clampf(rintf(v[t] / s) + (float)z,"),
    ("no_zero_extension", "float x_min = 0.0f, x_max = 0.0f; /* zero-extended range (R5) */",
     "float x_min = v[0], x_max = v[0];"),
    ("sym_divides_by_8", "s = amax / 7.0f;", "s = amax / 8.0f;"),
    ("sym_uses_signed_max", "amax = fmaxf(amax, fabsf(v[t]));\n                s = amax / 7.0f;",
     "amax = fmaxf(amax, v[t]);\n                s = amax / 7.0f;"),
    ("asym_divides_by_16", "s = (x_max - x_min) / 15.0f;", "s = (x_max - x_min) / 16.0f;"),
    ("nibbles_reversed", "                int64_t col = j * g + t;\n                qweight[row * (k / 8) + col / 8] |= u << (4 * (col % 8));",
     "                int64_t col = j * g + t;\n                qweight[row * (k / 8) + col / 8] |= u << (4 * (7 - col % 8));"),
    ("zero_point_sign", "rintf(-x_min / S)", "rintf(x_min / S)"),
    ("zero_word_index", "zeros[row * zw + j / 8] |= (uint32_t)z << (4 * (j % 8));\n                if (onesided)",
     "zeros[row * zw + j / 8] |= (uint32_t)z << (4 * (j / 8));\n                if (onesided)"),
    ("fp16_truncates", "if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;", ""),
    ("fp16_ties_away", "(rem == 0x1000u && (h & 1u))", "(rem == 0x1000u)"),
    ("fp16_subnormal_exponent", "mag = ldexpf((float)m, -24);", "mag = ldexpf((float)m, -25);"),
    ("degenerate_scale_zero", "s16 = 0x3C00u;  /* 1.0 */", "s16 = 0x0000u;"),
    ("sym_stores_twos_complement", "symmetric ? q + 8 : q", "symmetric ? (q & 15) : q"),
    ("asym_range_0_14", "const float q_max = symmetric ? 7.0f : 15.0f;\n\n    memset",
     "const float q_max = symmetric ? 7.0f : 14.0f;\n\n    memset"),
    ("dequant_drops_zero", "return S * ((double)u - (double)z);", "return S * (double)u;"),
    ("dequant_group_index", "const int64_t j = col / g;", "const int64_t j = col / 8;"),
    ("linear_drops_first_term", "acc += xv * wrow[kk];", "if (kk) acc += xv * wrow[kk];"),
    ("linear_transposed_x", "load_elem(x, x_dtype, row_m * k + kk)",
     "load_elem(x, x_dtype, kk * m + row_m)"),
    ("bf16_widening_shift", "uint32_t bits = (uint32_t)b << 16;",
     "uint32_t bits = (uint32_t)b << 15;"),
    ("zero_rows_padding", "return n * ((k / g + 7) / 8);", "return n * ((k / g) / 8);"),
    ("mse_ties_keep_later", "(i == 0 || e < best_err)", "(i == 0 || e <= best_err)"),
    ("mse_grid_step", "const float alpha = (float)(20 - i) / 20.0f;",
     "const float alpha = (float)(20 - i) / 21.0f;"),
    ("mse_error_drops_zero_point", "const double xhat = (double)S * (double)(q - z);",
     "const double xhat = (double)S * (double)q;"),
    ("mse_clips_low_end_only", "const float hi = alpha * x_max;", "const float hi = x_max;"),
    ("mse_picks_largest_error", "(i == 0 || e < best_err)", "(i == 0 || e > best_err)"),
    ("mse_error_drops_first_term", "err = err + d * d;", "if (t) err = err + d * d;"),
    ("mse_error_absolute", "err = err + d * d;", "err = err + fabs(d);"),
    ("mse_error_in_fp32", "err = err + d * d;", "err = (float)(err + d * d);"),
    ("mse_clip_ratio_ignored", "best = ratio[row * G + j];", "best = 0;"),
    ("mse_zero_point_unclipped", "if (!symmetric) z = (int)clampf(rintf(-lo / S), q_min, q_max);",
     "if (!symmetric) z = (int)clampf(rintf(-lo / S) + 1.0f, q_min, q_max);"),
    ("mse_sym_range_unscaled", "s = (alpha * amax) / 7.0f;", "s = amax / 7.0f;"),
    ("kv_cache_token_major", "const int64_t r = h * t_cap + t0 + t;",
     "const int64_t r = (t0 + t) * heads + h;"),
    ("kv_cache_ignores_t0", "const int64_t r = h * t_cap + t0 + t;", "const int64_t r = h * t_cap + t;"),
    ("kv_input_head_major", "(size_t)((t * heads + h) * d) * esize",
     "(size_t)((h * t_new + t) * d) * esize"),
    ("kv_attn_token_major", "const int64_t r = h * t_cap + t;\n            double acc",
     "const int64_t r = t * heads + h;\n            double acc"),
    ("kv_attn_value_token_shift", "xhat_elem(vq, vs, vz, h * t_cap + t, i",
     "xhat_elem(vq, vs, vz, h * t_cap + (t + 1) % n_tok, i"),
    ("kv_attn_keys_as_values", "xhat_elem(vq, vs, vz,", "xhat_elem(kq, ks, kz,"),
    ("kv_attn_value_scales_from_keys", "xhat_elem(vq, vs, vz,", "xhat_elem(vq, ks, vz,"),
    ("kv_attn_no_scale", "s[t] = scale * acc;", "s[t] = acc;"),
    ("kv_attn_unnormalized", "out[h * d + i] = acc / l;", "out[h * d + i] = acc;"),
    ("kv_attn_exp_sign", "s[t] = exp(s[t] - M);", "s[t] = exp(M - s[t]);"),
    ("kv_attn_query_of_head0", "load_elem(q, q_dtype, h * d + i)", "load_elem(q, q_dtype, i)"),
    ("kv_attn_drops_last_token", "for (int64_t t = 0; t < n_tok; ++t) {\n            s[t] = exp",
     "for (int64_t t = 0; t < n_tok; ++t) {\n            if (t == n_tok - 1 && t) { s[t] = 0; continue; }\n            s[t] = exp"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new), encoding="utf-8")
    lib = oracle.compile_source(str(path), str(tmp_path / "libmutant.so"),
                                include_dir=os.path.dirname(oracle.SOURCE))
    o = oracle.Oracle(lib)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(o)
        except Exception as exc:  # AssertionError, or a crash-free error from bad output
            caught.append(f"{check.__name__}: {type(exc).__name__}")
    assert caught, f"mutant {name} passed every pin"
