"""The oracle's pins must fail when a plausible mistake is planted in it.

Each case copies oracle.c, applies one textual mutation (a dropped term, a
wrong sign, a transposed operand, double rounding, ties away from zero, a wrong
padding test, ...), builds the copy on the CPU into a temporary library and runs
the pin suite against it in a subprocess.  The suite must fail for every mutant;
a mutant that survives means some part of the oracle is not pinned.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_last_term": ("s[j] = 0.0, ab[j] = 0.0;\n    for (int64_t r = 0; r < red; ++r) {",
                          "s[j] = 0.0, ab[j] = 0.0;\n    for (int64_t r = 0; r < red - 1; ++r) {"),
    "fp8_dropped_last_term": ("g[j] = 0.0;\n    for (int64_t r = 0; r < red; ++r) {",
                              "g[j] = 0.0;\n    for (int64_t r = 0; r < red - 1; ++r) {"),
    "bias_sign": ("s[j] += c->B[j], ab[j] += fabs(c->B[j]);",
                  "s[j] -= c->B[j], ab[j] += fabs(c->B[j]);"),
    "forward_transposed_w": ("row_dot(c->X + r * c->k, c->k, c->W, c->n, 1, c->n, s, ab);",
                             "row_dot(c->X + r * c->k, c->k, c->W, 1, c->k, c->n, s, ab);"),
    "dx_untransposed_w": ("row_dot(c->DY + r * c->n, c->n, c->W, 1, c->n, c->k, s, ab);",
                          "row_dot(c->DY + r * c->n, c->n, c->W, c->k, 1, c->k, s, ab);"),
    "double_rounding_via_f32": ("case ORC_BF16: ((uint16_t *)base)[i] = orc_rne_bf16(v); break;",
                                "case ORC_BF16: ((uint16_t *)base)[i] = orc_rne_bf16((float)v); break;"),
    "ties_away_from_zero": ("double r = rint(ax / q) * q;", "double r = round(ax / q) * q;"),
    "padding_bound_off_by_one": ("if ((int64_t)ex >= c->e) {", "if ((int64_t)ex > c->e) {"),
    "e4m3_exponent_bias": ("v = ldexp((double)(8 + frac), ex - 10);",
                           "v = ldexp((double)(8 + frac), ex - 9);"),
    "f16_subnormal_quantum": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "fp8_missing_b_scale": ("double v = s[j] * c->da * c->db;", "double v = s[j] * c->da;"),
    "abs_scale_signed": ("ab[j] += fabs(p);\n        }\n    }\n}",
                         "ab[j] += p;\n        }\n    }\n}"),
    "dweights_wrong_expert_test": ("if ((int64_t)c->row_experts[mm] != ee) continue;",
                                   "if ((int64_t)c->row_experts[mm] > ee) continue;"),
    "dw_reads_dy_transposed": ("row_dot(arow, c->m, c->DY, c->n, 1, c->n, s, ab);",
                               "row_dot(arow, c->m, c->DY, 1, c->m, c->n, s, ab);"),
    "e5m2_exponent_bias": ("v = ldexp((double)(4 + frac), ex - 17);",
                           "v = ldexp((double)(4 + frac), ex - 16);"),
    "e5m2_no_saturation": ("if (isinf(r)) r = 57344.0;", "if (isinf(r)) r = 49152.0;"),
    "quantize_product_in_double": ("return fmt == ORC_E5M2 ? orc_rne_e5m2_sat((double)v) : orc_rne_e4m3_sat((double)v);",
                                   "return fmt == ORC_E5M2 ? orc_rne_e5m2_sat((double)raw * scale_inv) : orc_rne_e4m3_sat((double)raw * scale_inv);"),
    "quantize_ignores_format": ("return fmt == ORC_E5M2 ? orc_rne_e5m2_sat((double)v) : orc_rne_e4m3_sat((double)v);",
                                "return orc_rne_e4m3_sat((double)v);"),
    "transpose_quantize_not_transposed": ("dst[c * rows + r] = quant_code(fmt, src[r * cols + c], scale_inv);",
                                          "dst[r * cols + c] = quant_code(fmt, src[r * cols + c], scale_inv);"),
    "amax_signed": ("const float a = fabsf((float)orc_decode_bf16(src[i]));",
                    "const float a = (float)orc_decode_bf16(src[i]);"),
    "fp8_linear_bias_dropped": ("if (c->B) v += c->B[j], a += fabs(c->B[j]);",
                                "if (c->B) a += fabs(c->B[j]);"),
    "fp8_linear_dx_w_untransposed": ("row_dot_g8(c->QG + r * c->n, c->n, c->QW, c->k, 1, c->k, s, ab, g);",
                                     "row_dot_g8(c->QG + r * c->n, c->n, c->QW, 1, c->n, c->k, s, ab, g);"),
    "fp8_linear_dw_wrong_scale": ("c.sa = (double)sg, c.sb = which == 1 ? (double)sw : (double)sx, c.rows = rows;",
                                  "c.sa = (double)sg, c.sb = (double)sw, c.rows = rows;"),
    "fp8_group_of_16": ("if (r % 8 == 7 || r == red - 1)", "if (r % 16 == 15 || r == red - 1)"),
    "bias_grad_row_stride": ("const double v = orc_decode(dt, dy, i * n + j);",
                             "const double v = orc_decode(dt, dy, j * m + i);"),
    "f16_overflow_saturates": ("double r = round_mag(fabs(x), 11, -14, 65504.0);\n    uint16_t mag;\n    if (isinf(r)) {\n        mag = 0x7c00;",
                               "double r = round_mag(fabs(x), 11, -14, 65504.0);\n    uint16_t mag;\n    if (isinf(r)) {\n        mag = 0x7bff;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-pthread", str(mut), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
