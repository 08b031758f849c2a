"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/bitlinear_oracle.c, makes one plausible mistake in the
copy (a dropped term, a wrong constant, a transposed index, another rounding
rule), builds it with gcc in a temporary folder and runs the pin suite against
it in a subprocess.  The suite must fail on every copy.  All of this runs on
the CPU; the real oracle source is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "round_half_away": ("float v = rintf(W[i] / gamma_c);", "float v = roundf(W[i] / gamma_c);"),
    "ternary_sign_dropped": ("float v = rintf(W[i] / gamma_c);", "float v = rintf(fabsf(W[i]) / gamma_c);"),
    "gamma_divides_by_k": ("double count = (double)N * (double)K;", "double count = (double)K;"),
    "gamma_float_sum": ("double r = 0.0;", "float r = 0.0f;"),
    "gamma_no_guard": ("*gamma_c = g > ORACLE_EPS ? g : ORACLE_EPS;", "*gamma_c = g;"),
    "acts_qb_128": ("float qs = 127.0f / a_c;", "float qs = 128.0f / a_c;"),
    "acts_scale_reciprocal": ("*s_x = a_c / 127.0f;", "*s_x = 1.0f / qs;"),
    "acts_sign_dropped": ("float v = rintf(x[k] * qs);", "float v = rintf(fabsf(x[k]) * qs);"),
    "acts_truncate": ("float v = rintf(x[k] * qs);", "float v = truncf(x[k] * qs);"),
    "bf16_widen_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "pack_field_from_byte": ("*shift = (int)(2 * field);", "*shift = (int)(2 * byte_in_word);"),
    "pack_chunk_transposed": ("int64_t chunk = sub * 16 + row_in_tile;",
                              "int64_t chunk = row_in_tile * 4 + sub;"),
    "matmul_wrong_row": ("s += (int32_t)qx[m * K + k] * (int32_t)qw[n * K + k];",
                         "s += (int32_t)qx[m * K + k] * (int32_t)qw[((n + 1) % N) * K + k];"),
    "rescale_drops_gamma": ("y[mn] = t * gamma_c;", "y[mn] = t;"),
    "rescale_other_order": ("float t = (float)acc[mn] * s_x[mn / N];\n    y[mn] = t * gamma_c;",
                            "float t = (float)acc[mn] * gamma_c;\n    y[mn] = t * s_x[mn / N];"),
    "relu_dropped": ("float r = y[i] > 0.0f ? y[i] : 0.0f;", "float r = y[i];"),
    "norm_gain_dropped": ("    u[k] = x[k] * g[k];", "    u[k] = x[k];"),
    "norm_sum_not_mean": ("float r = (float)(1.0 / sqrt(S / (double)K + (double)eps_n));",
                          "float r = (float)(1.0 / sqrt(S + (double)eps_n));"),
    "norm_no_sqrt": ("float r = (float)(1.0 / sqrt(S / (double)K + (double)eps_n));",
                     "float r = (float)(1.0 / (S / (double)K + (double)eps_n));"),
    "norm_eps_outside": ("float r = (float)(1.0 / sqrt(S / (double)K + (double)eps_n));",
                         "float r = (float)(1.0 / (sqrt(S / (double)K) + (double)eps_n));"),
    "norm_scale_missing": ("  *s_x = *s_x * r;", "  (void)r;"),
    "glu_halves_swapped": ("      float g = y[m * N + f];", "      float g = y[m * N + F + f];"),
    "glu_not_squared": ("      float t = r * r;", "      float t = r;"),
    "glu_pack_rows": ("  return i < 8 ? 8 * t + i : N / 2 + 8 * t + (i - 8);",
                      "  return i < 8 ? 16 * t + i : N / 2 + 8 * t + (i - 8);"),
    # other orders of the same float operations (R4, R2, R12, R8)
    "acts_x127_over_a": ("float v = rintf(x[k] * qs);", "float v = rintf(x[k] * 127.0f / a_c);"),
    "acts_x_over_scale": ("float v = rintf(x[k] * qs);",
                          "float v = rintf(x[k] / (a_c / 127.0f));"),
    "ternary_reciprocal": ("float v = rintf(W[i] / gamma_c);",
                           "float v = rintf(W[i] * (1.0f / gamma_c));"),
    "glu_other_association": ("      float t = r * r;\n      h[m * F + f] = t * y[m * N + F + f];",
                              "      float t = r * y[m * N + F + f];\n      h[m * F + f] = r * t;"),
    "norm_factor_in_float": ("float r = (float)(1.0 / sqrt(S / (double)K + (double)eps_n));",
                             "float r = 1.0f / sqrtf((float)(S / (double)K) + eps_n);"),
    # base-3 layout (R13)
    "b3_digit_order_reversed": ("  *digit = (int)(u / 4);", "  *digit = (int)(4 - u / 4);"),
    "b3_columns_grouped_by_five": (
        "  int64_t byte_in_word = u % 4;\n  int64_t chunk = quarter * 16 + row_in_tile;\n"
        "  int64_t tile = tile_row * (Kp / 320) + kblock;\n  *digit = (int)(u / 4);",
        "  int64_t byte_in_word = u / 5;\n  int64_t chunk = quarter * 16 + row_in_tile;\n"
        "  int64_t tile = tile_row * (Kp / 320) + kblock;\n  *digit = (int)(u % 5);"),
    "b3_chunk_transposed": ("  int64_t chunk = quarter * 16 + row_in_tile;",
                            "  int64_t chunk = row_in_tile * 4 + quarter;"),
    "b3_padding_not_zero": ("  memset(packed, 0, (size_t)(N * Kp / 5));",
                            "  memset(packed, 1, (size_t)(N * Kp / 5));"),
    "b3_pad_to_256": ("static int64_t b3_padded_k(int64_t K) { return (K + 319) / 320 * 320; }",
                      "static int64_t b3_padded_k(int64_t K) { return (K + 255) / 256 * 256; }"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant_src), str(tmp_path / "libmutant.so"), extra_flags=["-w"])
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"pins did not catch {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
