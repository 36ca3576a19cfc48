"""Planted mistakes in copies of the oracle: every one must fail at least one pin.

Each mutant rewrites one fragment of ``oracle/oracle.c`` in a temporary copy (a dropped term,
a wrong sign, a wrong index or constant, a transposed field layout ...), compiles it with the
same flags and runs the whole pin suite against it.  This shows the pins would catch the
plausible mistakes; the real oracle is never modified.
"""

import os

import pytest

import oracle
import pins

MUTANTS = {
    "gamma_drops_abs": ("sum += fabs((double)W[i]);", "sum += (double)W[i];"),
    "gamma_off_by_one_count": ("sum / (double)count", "sum / (double)(count - 1 + (count == 1))"),
    "gamma_uses_max": ("sum += fabs((double)W[i]);",
                       "sum = fabs((double)W[i]) > sum ? fabs((double)W[i]) : sum;"),
    "tie_rounds_up": ("if (x > 0.5f)\n        return 1;", "if (x >= 0.5f)\n        return 1;"),
    "negative_code_sign": ("if (x < -0.5f)\n        return -1;", "if (x < -0.5f)\n        return 1;"),
    "divides_the_wrong_way": ("float t = W[i] / gamma;", "float t = gamma / W[i];"),
    "pack_minus_one_field": ("field = 3u;", "field = 2u;"),
    "pack_transposed_fields": ("return (unsigned)(8 * b + 2 * i);", "return (unsigned)(8 * i + 2 * b);"),
    "unpack_sign_swap": ("else if (field == 3u)\n                    c = -1;",
                         "else if (field == 3u)\n                    c = 1;"),
    "act_uses_128": ("float inv = 127.0f / a;", "float inv = 128.0f / a;"),
    "act_truncates": ("float v = rintf(u * inv);", "float v = truncf(u * inv);"),
    "act_rounds_half_away": ("float v = rintf(u * inv);", "float v = roundf(u * inv);"),
    "act_scale_inverted": ("*s_x = a / 127.0f;", "*s_x = 127.0f / a;"),
    "norm_drops_g": ("float u = g ? x[k] * g[k] : x[k];\n        float v",
                     "float u = x[k];\n        float v"),
    "norm_drops_eps": ("ss / (double)K + (double)eps", "ss / (double)K"),
    "norm_sum_not_mean": ("ss / (double)K + (double)eps", "ss + (double)eps"),
    "bf16_wrong_shift": ("(uint32_t)X[m * K + k] << 16", "(uint32_t)X[m * K + k] << 15"),
    "matmul_drops_first_term": ("for (int64_t k = 0; k < K; ++k)\n                s += (int64_t)Xq[m * K + k] * (int64_t)C[n * K + k];",
                                "for (int64_t k = 1; k < K; ++k)\n                s += (int64_t)Xq[m * K + k] * (int64_t)C[n * K + k];"),
    "matmul_subtracts": ("s += (int64_t)Xq[m * K + k] * (int64_t)C[n * K + k];",
                         "s -= (int64_t)Xq[m * K + k] * (int64_t)C[n * K + k];"),
    "epilogue_drops_gamma": ("Y[m * N + n] = (float)((double)acc[m * N + n] * (double)gamma * (double)s_x[m]);",
                             "Y[m * N + n] = (float)((double)acc[m * N + n] * (double)s_x[m]);"),
    "epilogue_wrong_row_scale": ("Y[m * N + n] = (float)((double)acc[m * N + n] * (double)gamma * (double)s_x[m]);",
                                 "Y[m * N + n] = (float)((double)acc[m * N + n] * (double)gamma * (double)s_x[0]);"),
    "silu_wrong_sign": ("(1.0 + exp(-(double)x))", "(1.0 + exp((double)x))"),
    "swiglu_drops_up": ("v = ((double)x / (1.0 + exp(-(double)x))) * (double)x2;",
                        "v = ((double)x / (1.0 + exp(-(double)x)));"),
    "relu2_glu_no_square": ("v = r * r * (double)x2;", "v = r * (double)x2;"),
    "relu2_no_square": ("        v = r * r;\n    }", "        v = r;\n    }"),
    "relu2_keeps_negatives": ("        double r = x > 0.0f ? (double)x : 0.0;\n        v = r * r;",
                              "        double r = (double)x;\n        v = r * r;"),
    "residual_dropped": ("Y[m * N + n] = y + R[m * N + n];", "Y[m * N + n] = y;"),
    "residual_subtracted": ("Y[m * N + n] = y + R[m * N + n];", "Y[m * N + n] = y - R[m * N + n];"),
    "wonly_transposed_codes": ("s += (double)X[m * K + k] * (double)C[n * K + k];",
                               "s += (double)X[m * K + k] * (double)C[k * N + n];"),
    "wonly_drops_gamma": ("Y[m * N + n] = (float)((double)gamma * s);", "Y[m * N + n] = (float)s;"),
    "grad_input_untransposed": ("s += (double)dY[m * N + n] * (double)C[n * K + k];",
                                "s += (double)dY[m * N + n] * (double)C[k * N + n];"),
    "grad_input_subtracts": ("s += (double)dY[m * N + n] * (double)C[n * K + k];",
                             "s -= (double)dY[m * N + n] * (double)C[n * K + k];"),
    "grad_input_drops_gamma": ("dX[m * K + k] = (float)((double)gamma * s);", "dX[m * K + k] = (float)s;"),
    "ste_hard_strict": ("return fabsf(t) <= 1.0f ? 1.0 : 0.0;", "return fabsf(t) < 1.0f ? 1.0 : 0.0;"),
    "ste_soft_no_beta": ("cosh(beta * (double)t)", "cosh((double)t)"),
    "ste_soft_fp32_tanh": ("return 1.0 / (c * c);",
                           "return (double)(1.0f - tanhf((float)(beta * t)) * tanhf((float)(beta * t)));"),
    "ste_multiplies": ("const float t = gamma == 0.0f ? 0.0f : w / gamma;",
                       "const float t = gamma == 0.0f ? 0.0f : w * gamma;"),
    "grad_weight_drops_row_scale": ("(double)Xq[m * K + k] * (double)s_x[m] : (double)Xf",
                                    "(double)Xq[m * K + k] : (double)Xf"),
    "grad_weight_first_row_scale": ("(double)Xq[m * K + k] * (double)s_x[m] : (double)Xf",
                                    "(double)Xq[m * K + k] * (double)s_x[0] : (double)Xf"),
    "grad_weight_mask_transposed": ("oracle_ste_scale(kind, W[n * K + k], gamma, beta)",
                                    "oracle_ste_scale(kind, W[k * N + n], gamma, beta)"),
    "grad_weight_dy_transposed": ("s += (double)dY[m * N + n] * xh;", "s += (double)dY[n * M + m] * xh;"),
    "b3_digit_without_offset": ("v += (unsigned)(c + 1) * p;", "v += (unsigned)(c + 3) % 3 * p;"),
    "b3_plane_mapping": ("return 80 * j + (i < 4 ? 4 * b + i : 64 + b);", "return 80 * j + 16 * i + b;"),
    "b3_last_digit_mapping": ("return 80 * j + (i < 4 ? 4 * b + i : 64 + b);", "return 80 * j + (i < 4 ? 4 * b + i : 79 - b);"),
    "b3_base_four": ("p *= 3;", "p *= 4;"),
    "b3_unpack_sign": ("codes[n * K + k] = (int8_t)((int)(v % 3) - 1);", "codes[n * K + k] = (int8_t)(1 - (int)(v % 3));"),
    "b3_padding_minus_one": ("                    int c = 0;\n                    if (k < K) {", "                    int c = -1;\n                    if (k < K) {"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutant {name}: fragment not found in oracle.c"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new, 1))
    lib = oracle.build(str(path), str(tmp_path / "liboracle_mutant.so"), ["-w"])
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except (ValueError, OverflowError, ZeroDivisionError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
