"""The oracle's pins must catch plausible mistakes (CPU only).

Each case below plants one mistake in a private copy of the oracle's C source
(a dropped term, a wrong sign, a swapped operand, a transposed store, a wrong
rounding rule ...), builds it, and runs the pin tests against it in a child
process.  The pins pass on the real oracle; every mutant must make at least
one of them fail.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "siluquant_oracle.c")
PINS = ["tests/test_oracle_pipeline.py", "tests/test_oracle_quant.py",
        "tests/test_oracle_elementwise.py", "tests/test_oracle_sigmoid.py", "tests/test_oracle_forward.py",
        "tests/test_oracle_fp8.py", "tests/test_oracle_gemm.py", "tests/test_oracle_q8_1.py"]

MUTANTS = {
    "sigmoid_sign": ("exp(-(double)g)", "exp((double)g)"),
    "dgate_one_minus_s": ("float c = 1.0f - s;", "float c = s;"),
    "dgate_dropped_term": ("float m = 1.0f + k;", "float m = 1.0f;"),
    "dup_uses_up": ("*d_up = d * silu;", "*d_up = d * u;"),
    "y_missing_up": ("*y = silu * u;", "*y = silu;"),
    "bf16_truncates": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "no_bf16_round_trip": ("Y[t * H + h] = bf16_round(y);", "Y[t * H + h] = y;"),
    "ties_away_from_zero": ("float r = nearbyintf(p);", "float r = roundf(p);"),
    "exact_product_rounded": ("float p = x * inv;       /* one fp32 rounding (no contraction: -ffp-contract=off) */\n"
                              "      float r = nearbyintf(p);",
                              "double p = (double)x * (double)inv;\n      float r = (float)nearbyint(p);"),
    "quotient_not_inverse": ("float p = x * inv;", "float p = x / scale;"),
    "scale_over_128": ("amax / 127.0f", "amax / 128.0f"),
    "amax_without_abs": ("float a = fabsf(v[i * stride]);", "float a = v[i * stride];"),
    "zero_group_scale_zero": ("(amax == 0.0f) ? 1.0f : amax / 127.0f", "(amax == 0.0f) ? 0.0f : amax / 127.0f"),
    "fp8_zero_group_scale_zero": ("(amax == 0.0f) ? 1.0f : amax / 448.0f", "(amax == 0.0f) ? 0.0f : amax / 448.0f"),
    "gate_up_swapped": ("float g = oracle_bf16_to_f32(x[t * 2 * H + h]);\n"
                        "      float u = oracle_bf16_to_f32(x[t * 2 * H + H + h]);\n      float d",
                        "float g = oracle_bf16_to_f32(x[t * 2 * H + H + h]);\n"
                        "      float u = oracle_bf16_to_f32(x[t * 2 * H + h]);\n      float d"),
    "forward_gate_up_swapped": ("float g = oracle_bf16_to_f32(x[t * 2 * H + h]);\n"
                                "      float u = oracle_bf16_to_f32(x[t * 2 * H + H + h]);\n      float s",
                                "float g = oracle_bf16_to_f32(x[t * 2 * H + H + h]);\n"
                                "      float u = oracle_bf16_to_f32(x[t * 2 * H + h]);\n      float s"),
    "yqt_not_transposed": ("oracle_quant_group(&Y[t0 * H + h], n, H, &y_q_t[h * T + t0], 1)",
                           "oracle_quant_group(&Y[t0 * H + h], n, H, &y_q_t[t0 * H + h], H)"),
    "fp8_yqt_not_transposed": ("oracle_quant_group_fp8(&Y[t0 * H + h], n, H, &y_q_t[h * T + t0], 1)",
                               "oracle_quant_group_fp8(&Y[t0 * H + h], n, H, &y_q_t[t0 * H + h], H)"),
    "forward_missing_up": ("float v = silu * u;\n      if (w) v = v * w[t];\n      uint16_t b = oracle_f32_to_bf16(v);\n"
                           "      Y[h] = oracle_bf16_to_f32(b);\n      if (y_bf16)",
                           "float v = silu;\n      if (w) v = v * w[t];\n      uint16_t b = oracle_f32_to_bf16(v);\n"
                           "      Y[h] = oracle_bf16_to_f32(b);\n      if (y_bf16)"),
    "forward_ignores_weight": ("if (w) v = v * w[t];\n      uint16_t b = oracle_f32_to_bf16(v);\n"
                               "      Y[h] = oracle_bf16_to_f32(b);\n      if (y_bf16)",
                               "if (w) v = v + 0.0f * w[t];\n      uint16_t b = oracle_f32_to_bf16(v);\n"
                               "      Y[h] = oracle_bf16_to_f32(b);\n      if (y_bf16)"),
    "forward_weight_after_rounding": ("      Y[h] = oracle_bf16_to_f32(b);\n      if (y_bf16)",
                                      "      Y[h] = oracle_bf16_to_f32(b) * (w ? w[t] : 1.0f);\n      if (y_bf16)"),
    "fp8_scale_over_127": ("(amax == 0.0f) ? 1.0f : amax / 448.0f", "(amax == 0.0f) ? 1.0f : amax / 127.0f"),
    "fp8_truncates": ("double mant = nearbyint(m * 16.0);", "double mant = floor(m * 16.0);"),
    "fp8_subnormal_step": ("double k = nearbyint(a * 512.0);", "double k = nearbyint(a * 256.0);"),
    "fp8_exponent_bias": ("int efield = e - 1 + 7;", "int efield = e - 1 + 8;"),
    "row_groups_skip_up_half": ("  int64_t row_groups = (2 * H + group - 1) / group;\n  for (int64_t t = 0; t < T; ++t) {",
                                "  int64_t row_groups = (H + group - 1) / group;\n  for (int64_t t = 0; t < T; ++t) {"),
    "fp8_row_groups_skip_up_half": ("    int64_t row_groups = (2 * H + group - 1) / group;\n    for (int64_t t = 0; t < T; ++t)\n",
                                    "    int64_t row_groups = (H + group - 1) / group;\n    for (int64_t t = 0; t < T; ++t)\n"),
    "fp8_zero_loses_sign": ("(x == 0.0f) ? oracle_f32_to_e4m3(x)", "(x == 0.0f) ? 0"),
    "gemm_drops_a_scale": ("double term = (double)sA[m * groups + g] * (double)sB",
                           "double term = (double)sB"),
    "gemm_b_scale_group_zero": ("sB[(n / b_rows_per_scale) * groups + g]", "sB[(n / b_rows_per_scale) * groups + 0]"),
    "gemm_b_scale_row_zero": ("sB[(n / b_rows_per_scale) * groups + g]", "sB[g]"),
    "gemm_b_not_transposed": ("(int64_t)B[n * K + k]", "(int64_t)B[k * N + n]"),
    "gemm_group_offset": ("for (int64_t k = g * group; k < (g + 1) * group; ++k)", "for (int64_t k = 0; k < group; ++k)"),
    "row_groups_split_at_halves": ("      int64_t n = (2 * H - c0 < group) ? 2 * H - c0 : group;\n      grad_input_s",
                                   "      int64_t n = (2 * H - c0 < group) ? 2 * H - c0 : group;\n"
                                   "      if (c0 < H && c0 + n > H) n = H - c0;\n      grad_input_s"),
    "f16_truncates": ("double mant = nearbyint(m * 2048.0);", "double mant = floor(m * 2048.0);"),
    "f16_subnormal_step": ("double k = nearbyint(a * ldexp(1.0, 24));", "double k = nearbyint(a * ldexp(1.0, 23));"),
    "f16_exponent_bias": ("int efield = e - 1 + 15;", "int efield = e - 1 + 16;"),
    "q8_1_header_swapped": ("uint16_t d16 = oracle_f32_to_f16(scale), s16 = oracle_f32_to_f16(dequant_sum);",
                            "uint16_t s16 = oracle_f32_to_f16(scale), d16 = oracle_f32_to_f16(dequant_sum);"),
    "q8_1_sum_of_codes": ("float dequant_sum = scale * (float)sum;", "float dequant_sum = (float)sum;"),
    "q8_1_codes_after_header_shift": ("memcpy(blk + 4, qb, 32);", "memcpy(blk + 4, qb + 1, 31);"),
    "kquant_rows_gate_from_up": ("float g = oracle_bf16_to_f32(gate[t * inter + h]);",
                                 "float g = oracle_bf16_to_f32(up[t * inter + h]);"),
    "kquant_rows_weight_dropped": ("      if (w) v = v * w[t];\n      uint16_t b = oracle_f32_to_bf16(v);\n"
                                   "      Y[h] = oracle_bf16_to_f32(b);\n      if (h_bf16)",
                                   "      uint16_t b = oracle_f32_to_bf16(v);\n"
                                   "      Y[h] = oracle_bf16_to_f32(b);\n      if (h_bf16)"),
    "kquant_rows_blocks_rotated": ("oracle_q8_1_block(qb, scale, blocks + (t * nb + b) * 36);",
                                   "oracle_q8_1_block(qb, scale, blocks + (t * nb + (b + 1) % nb) * 36);"),
    "fp8_nan_beyond_range": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 464.0) return sign | 0x7F;"),
}


# The pin file most likely to catch a family of mutants runs first, so that the
# child run (which stops at the first failure) ends early.
FIRST = {"gemm_": "tests/test_oracle_gemm.py", "fp8_": "tests/test_oracle_fp8.py",
         "forward_": "tests/test_oracle_forward.py", "f16_": "tests/test_oracle_q8_1.py",
         "q8_1_": "tests/test_oracle_q8_1.py", "kquant_": "tests/test_oracle_q8_1.py"}


def _run_mutant(name, workdir):
    """Build the mutant and run the pins against it; returns (caught, output)."""
    old, new = MUTANTS[name]
    src = open(SRC).read()
    if src.count(old) != 1:
        return None, "mutation anchor not found once: %r" % old
    mutant = os.path.join(workdir, "mutant_%s.c" % name)
    with open(mutant, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(workdir, "libmutant_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
                    "-fvisibility=hidden", mutant, "-o", lib, "-lm"], check=True)
    first = [f for pre, f in FIRST.items() if name.startswith(pre)]
    pins = first + [f for f in PINS if f not in first]
    env = dict(os.environ, SILUQUANT_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + pins,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode != 0, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Every mutant built and run against the pins, six at a time."""
    from concurrent.futures import ThreadPoolExecutor

    workdir = str(tmp_path_factory.mktemp("mutants"))
    with ThreadPoolExecutor(max_workers=6) as pool:
        futures = {name: pool.submit(_run_mutant, name, workdir) for name in MUTANTS}
        return {name: f.result() for name, f in futures.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, mutant_results):
    caught, out = mutant_results[name]
    assert caught is not None, out
    assert caught, "mutant %s passed every pin:\n%s" % (name, out)
