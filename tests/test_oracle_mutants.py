"""Plant plausible mistakes in a private copy of the oracle (CPU only) and
check that every one of them is caught by at least one pin.

Each mutation is a textual edit of oracle.c compiled to a temporary library;
the real oracle is never modified.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "ln_unbiased_variance": ("double var = or_acc_sum(&a2) / (double)N;",
                             "double var = or_acc_sum(&a2) / (double)(N - 1);"),
    "ln_eps_outside_sqrt": ("double rs = 1.0 / sqrt(var + deps);", "double rs = 1.0 / sqrt(var) + deps;"),
    "ln_mean_wrong_count": ("double mu = or_acc_sum(&a1) / (double)N;",
                            "double mu = or_acc_sum(&a1) / (double)(N + 1);"),
    "ln_gamma_beta_swapped": ("- mu) * rs * g + b;", "- mu) * rs * b + g;"),
    "ln_gamma_reversed": ("or_load(dtype, gamma, j)", "or_load(dtype, gamma, N - 1 - j)"),
    "ln_beta_dropped": ("double b = beta ? or_load(dtype, beta, j) : 0.0;", "double b = 0.0;"),
    "rms_no_mean": ("1.0 / sqrt(or_acc_sum(&acc) / (double)N + deps);", "1.0 / sqrt(or_acc_sum(&acc) + deps);"),
    "rms_weight_first_only": ("or_load(dtype, w, j)", "or_load(dtype, w, 0)"),
    "rms_eps_dropped": ("sqrt(or_acc_sum(&acc) / (double)N + deps)", "sqrt(or_acc_sum(&acc) / (double)N)"),
    "softmax_no_shift": ("double e = exp(v - m);", "double e = exp(v);"),
    "softmax_dropped_term": ("or_acc_add(&acc, e);", "or_acc_add(&acc, (j > 0) ? e : 0.0);"),
    "sum_compensation_dropped": ("    return isfinite(a->s) ? a->s + a->c : a->s;", "    return a->s;"),
    "sum_compensation_wrong_branch": ("        if (fabs(a->s) >= fabs(v))", "        if (fabs(a->s) < fabs(v))"),
    "softmax_exp2": ("double e = exp(v - m);", "double e = exp2(v - m);"),
    "softmax_multiply": ("yr[j] = yr[j] / s;", "yr[j] = yr[j] * s;"),
    "softmax_max_is_min": ("else if (v > m) m = v;\n        }\n        or_acc acc", "else if (v < m || m == -INFINITY) m = v;\n        }\n        or_acc acc"),
    "f16_bias_off_by_one": ("expo - 25", "expo - 24"),
    "f16_subnormal_scale": ("ldexp((double)mant, -24)", "ldexp((double)mant, -25)"),
    "bf16_shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "online_no_rescale": ("l_prev = l_prev * alpha + psum;", "l_prev = l_prev + psum;"),
    "online_alpha_sign": ("exp(m_prev - m_new)", "exp(m_new - m_prev)"),
    "online_final_uses_first_max": ("m_prev = m_new;", "m_prev = (m_prev == -INFINITY) ? m_new : m_prev;"),
    "add_subtracts": ("h[i] = or_load(dtype, x, i) + or_load(dtype, r, i);",
                      "h[i] = or_load(dtype, x, i) - or_load(dtype, r, i);"),
    "add_drops_residual": ("h[i] = or_load(dtype, x, i) + or_load(dtype, r, i);", "h[i] = or_load(dtype, x, i);"),
    "causal_drops_diagonal": ("int64_t vis = q + offset + 1;", "int64_t vis = q + offset;"),
    "causal_ignores_offset": ("int64_t vis = q + offset + 1;", "int64_t vis = q + 1;"),
    "causal_query_is_row": ("int64_t q = r % queries;", "int64_t q = r;"),
    "causal_scale_dropped": ("double v = sc * or_load(dtype, x, base + k);", "double v = or_load(dtype, x, base + k);"),
    "causal_masked_outputs_uniform": ("for (int64_t k = vis; k < N; ++k) y[base + k] = 0.0;",
                                      "for (int64_t k = vis; k < N; ++k) y[base + k] = 1.0 / (double)N;"),
    "add_residual_shifted": ("h[i] = or_load(dtype, x, i) + or_load(dtype, r, i);",
                             "h[i] = or_load(dtype, x, i) + or_load(dtype, r, i > 0 ? i - 1 : i);"),
    "attn_no_scale": ("s[j] = sc * or_acc_sum(&dot);", "s[j] = or_acc_sum(&dot);"),
    "attn_k_transposed": ("or_load(dtype, k, (b * Lk + j) * D + c)", "or_load(dtype, k, b * Lk * D + c * Lk + j)"),
    "attn_mask_drops_diagonal": ("if (causal && i + offset + 1 < vis) vis = i + offset + 1;",
                                 "if (causal && i + offset < vis) vis = i + offset;"),
    "attn_mask_one_too_many": ("if (causal && i + offset + 1 < vis) vis = i + offset + 1;",
                               "if (causal && i + offset + 2 < vis) vis = i + offset + 2;"),
    "attn_mask_ignores_offset": ("if (causal && i + offset + 1 < vis) vis = i + offset + 1;",
                                 "if (causal && i + 1 < vis) vis = i + 1;"),
    "attn_no_max_shift": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "attn_value_first_column": ("const double vj = or_load(dtype, v, (b * Lk + j) * D + c);",
                                "const double vj = or_load(dtype, v, (b * Lk + j) * D);"),
    "attn_value_of_query_head": ("const double vj = or_load(dtype, v, (b * Lk + j) * D + c);",
                                 "const double vj = or_load(dtype, v, j * D + c);"),
    "attn_abs_drops_weights": ("if (oabs) or_acc_add(&aab, s[j] * fabs(vj));", "if (oabs) or_acc_add(&aab, fabs(vj));"),
    "attn_no_normalization": ("o[n * D + c] = or_acc_sum(&acc) / ls;", "o[n * D + c] = or_acc_sum(&acc);"),
    "attn_online_no_acc_rescale": ("for (int64_t c = 0; c < D; ++c) acc[c] *= alpha;",
                                   "for (int64_t c = 0; c < D; ++c) acc[c] *= 1.0;"),
    "attn_online_no_l_rescale": ("            l_prev = l_prev * alpha + psum;\n            m_prev = m_new;\n        }\n"
                                 "        for (int64_t c = 0; c < D; ++c) o[row * D + c]",
                                 "            l_prev = l_prev + psum;\n            m_prev = m_new;\n        }\n"
                                 "        for (int64_t c = 0; c < D; ++c) o[row * D + c]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))
    failed = []
    # cheap pins first; the first one that fails is enough
    order = sorted(ALL_PINS, key=lambda n: ("torch" in n, "brute" in n, n))
    for pin_name in order:
        try:
            ALL_PINS[pin_name](lib)
        except AssertionError:
            failed.append(pin_name)
        except Exception as e:  # a crash or NaN trap also counts as caught
            failed.append(f"{pin_name} ({type(e).__name__})")
        if failed:
            break
    assert failed, f"mutant {name} passed every pin"
