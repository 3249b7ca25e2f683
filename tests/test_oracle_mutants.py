"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle.c, plants one plausible mistake (a swapped nibble, a
wrong tie rule, a dropped scale, a wrong block index, ...), builds it with
gcc on the CPU, and runs the pin suite against that build in a fresh
process: the suite has to fail.  The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "unpack_nibble_swap": ("(k % 2 == 0) ? (byte & 0xf) : (byte >> 4)",
                           "(k % 2 == 0) ? (byte >> 4) : (byte & 0xf)"),
    "pack_nibble_swap": ("(code[2 * j] | (code[2 * j + 1] << 4))",
                         "(code[2 * j + 1] | (code[2 * j] << 4))"),
    "tie_to_upper": ("if ((double)w[k] > mid[i] * s) ++c;",
                     "if ((double)w[k] >= mid[i] * s) ++c;"),
    "codes_against_fp32_absmax": ("if ((double)w[k] > mid[i] * s) ++c;",
                                  "if ((double)w[k] > mid[i] * (double)amax) ++c;"),
    "negative_grid_8": ("(p_top - 0.5) / 7.0", "(p_top - 0.5) / 8.0"),
    "dropped_scale": ("double w = (double)cb[code_at(codes, K, m, k)] * s;",
                      "double w = (double)cb[code_at(codes, K, m, k)];"),
    "block_index_32": ("double s = oracle_f16_to_f64(scales[m * (K / 64) + k / 64]);\n            double w",
                       "double s = oracle_f16_to_f64(scales[m * (K / 64) + k / 128]);\n            double w"),
    "f16_tie_up": ("r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0; /* tie: to even */", "r = fl + 1.0;"),
    "argmax_last_tie": ("if (!isnan(y[i]) && (best < 0 || y[i] > y[best])) best = i;\n    return best;\n}\n\nint64_t oracle_argmax_f32",
                        "if (!isnan(y[i]) && (best < 0 || y[i] >= y[best])) best = i;\n    return best;\n}\n\nint64_t oracle_argmax_f32"),
    "abs_sum_signed": ("mag += fabs(t);", "mag += t;"),
    "zero_block_code_0": ("code[k] = 7;\n                    continue;", "code[k] = 0;\n                    continue;"),
    "silu_exponent_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "swiglu_operands_swapped": ("v = oracle_silu(a) * b;", "v = oracle_silu(b) * a;"),
    "bias_after_silu": ("        double v = a;\n        if (swiglu) {", "        double v = a;\n        if (swiglu && bias0) a -= (double)bias0[i];\n        if (swiglu) {"),
    "bf16_precision_7_bits": ("q = ldexp(1.0, ex - 1 - 7);", "q = ldexp(1.0, ex - 1 - 6);"),
    "bf16_tie_away": ("r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;\n    double u = r * q; /* the rounded magnitude */",
                      "r = fl + 1.0;\n    double u = r * q; /* the rounded magnitude */"),
    "bf16_truncate": ("    if (frac > 0.5)\n        r = fl + 1.0;\n    else if (frac < 0.5)\n        r = fl;\n    else\n        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;\n    double u = r * q; /* the rounded magnitude */",
                      "    r = fl;\n    double u = r * q; /* the rounded magnitude */"),
    "gather_ignores_ids": ("const int64_t m = ids[i];", "const int64_t m = i;"),
    "gather_bad_row_untouched": ("                    ((float *)out)[i * K + k] = 0.0f;",
                                 "                    (void)0;"),
    "gather_accepts_id_M": ("if (m < 0 || m >= M) {", "if (m < 0 || m > M) {"),
    "gather_fp32_via_bf16": ("((float *)out)[i * K + k] = (float)w;",
                             "((float *)out)[i * K + k] = (float)oracle_bf16_to_f64(oracle_f64_to_bf16_rne(w));"),
    "affine_zero_sign": ("What[m * K + k] = ((double)code_at(codes, K, m, k) - oracle_f16_to_f64(zeros[g])) *",
                         "What[m * K + k] = ((double)code_at(codes, K, m, k) + oracle_f16_to_f64(zeros[g])) *"),
    "affine_range_without_zero": ("float lo = 0.0f, hi = 0.0f;", "float lo = w[0], hi = w[0];"),
    "affine_scale_over_16": ("((double)hi - (double)lo) / 15.0", "((double)hi - (double)lo) / 16.0"),
    "affine_zero_tie_up": ("if (-(double)lo > ((double)j + 0.5) * s) ++z;",
                           "if (-(double)lo >= ((double)j + 0.5) * s) ++z;"),
    "affine_code_tie_up": ("if ((double)w[k] > ((double)(j - z) + 0.5) * s) ++c;",
                           "if ((double)w[k] >= ((double)(j - z) + 0.5) * s) ++c;"),
    "affine_gemv_ignores_zero": ("const double w = ((double)code_at(codes, K, m, k) - oracle_f16_to_f64(zeros[g])) *",
                                 "const double w = ((double)code_at(codes, K, m, k)) *"),
    "f16_via_f32": ("    if (isnan(v)) return (uint16_t)(sign | 0x7e00);\n    double a = fabs(v);",
                    "    if (isnan(v)) return (uint16_t)(sign | 0x7e00);\n    double a = fabs((double)(float)v);"),
    "e4m3_bias_8": ("v = ldexp(8.0 + m, e - 10); /* (1 + m / 8) 2^(e - 7) */", "v = ldexp(8.0 + m, e - 11);"),
    "e2m1_top_5": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};\n    const double v = mag[c & 7];",
                   "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0};\n    const double v = mag[c & 7];"),
    "grid_ties_to_odd": ("if (a > mid || (a == mid && (i & 1))) {", "if (a > mid || (a == mid && !(i & 1))) {"),
    "tensor_scale_2048": ("return (float)(amax / 2688.0);", "return (float)(amax / 2048.0);"),
    "nvfp4_sign_dropped": ("c[h] = (uint8_t)(mag | (signbit(wv) ? 8 : 0));", "c[h] = (uint8_t)mag;"),
    "nvfp4_block_32": ("oracle_e4m3_to_f64(scales[m * (K / 16) + k / 16]) * (double)s;\n}",
                       "oracle_e4m3_to_f64(scales[m * (K / 16) + k / 32]) * (double)s;\n}"),
    "nvfp4_gemv_drops_tensor_scale": ("oracle_e4m3_to_f64(scales[m * (K / 16) + k / 16]) * (double)s;\n            const double prod",
                                      "oracle_e4m3_to_f64(scales[m * (K / 16) + k / 16]);\n            const double prod"),
    "x8_ties_up": ("if (a > mid || (a == mid && (j & 1))) ++j;", "if (a >= mid) ++j;"),
    "x8_scale_128": ("const float db = (float)(amax / 127.0);", "const float db = (float)(amax / 128.0);"),
    "x8_second_word_256": ("a2 = nearest_int_127(fabs(r), (double)db / 128.0);",
                           "a2 = nearest_int_127(fabs(r), (double)db / 256.0);"),
    "x8_second_word_sign": ("if (r < 0) a2 = -a2;", "if (v < 0) a2 = -a2;"),
    "x8_gemv_second_word_256": ("const double xv = (double)d[k / 32] * ((double)q1[k] + (q2 ? (double)q2[k] / 128.0 : 0.0));",
                                "const double xv = (double)d[k / 32] * ((double)q1[k] + (q2 ? (double)q2[k] / 256.0 : 0.0));"),
    "residual_dropped": ("if (residual) v += (double)residual[i];", "if (residual && !swiglu) v += (double)residual[i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(mpath), str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, Q4_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
