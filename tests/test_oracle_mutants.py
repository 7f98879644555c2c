"""Each pin set must catch plausible mistakes planted in a copy of the oracle.

Every mutant is a one-line textual change to ``oracle/sgemm_oracle.c`` or
``oracle/attention_oracle.c``
(a dropped term, a wrong sign or index, a transposed operand, a lost factor
in the bound, ...), compiled to a temporary library.  The pins of
tests/oracle_pins.py then run against it in a child process (a mutant may
read out of bounds and crash; a crash also counts as caught).  A mutant that
passes every pin would mean the pins cannot tell that mistake from the
oracle, and the test fails.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sgemm_oracle.c")
SRC_ATT = os.path.join(ROOT, "oracle", "attention_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("drop_beta_term", "if (beta != 0.0f) t += (double)beta * (double)c;", ""),
    ("beta_term_sign", "t += (double)beta * (double)c;", "t -= (double)beta * (double)c;"),
    ("drop_alpha", "double t = (double)alpha * sum;", "double t = sum;"),
    ("subtract_products", "s[j] += p;", "s[j] -= p;"),
    ("drop_last_k", "for (int64_t k = 0; k < K; ++k) {\n                    const double a",
     "for (int64_t k = 0; k < K - 1; ++k) {\n                    const double a"),
    ("skip_first_k", "for (int64_t k = 0; k < K; ++k) {\n                    const double a",
     "for (int64_t k = (K > 1); k < K; ++k) {\n                    const double a"),
    ("transposed_B", "const double p = a * (double)brow[j];",
     "const double p = a * (double)B[j * ldb + k];"),
    ("A_column_for_row", "const double a = (double)A[i * lda + k];",
     "const double a = (double)A[k * lda + i];"),
    ("B_ignores_ld", "const float* brow = B + k * ldb;", "const float* brow = B + k * N;"),
    ("fp32_accumulator", "const double p = a * (double)brow[j];",
     "const double p = (double)(float)(a * (double)brow[j]);"),
    ("bound_factor_1", "return 2.0 * (double)K * ORACLE_U", "return (double)K * ORACLE_U"),
    ("bound_signed_sum", "sa[j] += fabs(p);", "sa[j] += p;"),
    ("bound_drops_beta", "double beta_term = (beta == 0.0f) ? 0.0 : fabs((double)beta * (double)c);",
     "double beta_term = 0.0;"),
    ("C_ignores_ldc", "const float c = (beta != 0.0f) ? C[i * ldc + j] : 0.0f;\n"
     "                    Cref", "const float c = (beta != 0.0f) ? C[i * N + j] : 0.0f;\n"
     "                    Cref"),
    ("A_ignores_lda", "const double a = (double)A[i * lda + k];",
     "const double a = (double)A[i * K + k];"),
    ("alpha_scales_by_beta", "double t = (double)alpha * sum;", "double t = (double)beta * sum;"),
    ("entries_transposed_B", "(double)B[k * ldb + j];", "(double)B[j * ldb + k];"),
    ("entries_drop_beta", "        out[t] = finish(alpha, beta, s, c);\n        if (bnd) bnd[t] = bound_of(K, alpha, beta, sa, c);\n    }\n    return 0;\n}\n\n/*\n * Matrix-core",
     "        out[t] = finish(alpha, 0.0f, s, c);\n        if (bnd) bnd[t] = bound_of(K, alpha, beta, sa, c);\n    }\n    return 0;\n}\n\n/*\n * Matrix-core"),
    # the matrix-core variant
    ("round_ties_away", "nearbyint((double)x / q)", "round((double)x / q)"),
    ("round_truncates", "nearbyint((double)x / q)", "trunc((double)x / q)"),
    ("f16_one_bit_short", "round_to_format(x, 11, -14, 65504.0)",
     "round_to_format(x, 10, -14, 65504.0)"),
    ("no_subnormal_spacing", "if (lead < emin) lead = emin;", ""),
    ("no_overflow_to_inf", "if (fabs(r) > max) return copysign(INFINITY, (double)x);", ""),
    ("exponent_off_by_one", "int lead = e - 1; ", "int lead = e; "),
    ("bf16_rounded_as_f16", "return round_to_format(x, 8, -126, ldexp(255.0, 120));",
     "return round_to_format(x, 11, -14, 65504.0);"),
    ("A_not_rounded", "Ar[i * K + k] = (float)round_fmt(fmt, A[i * lda + k]);",
     "Ar[i * K + k] = A[i * lda + k];"),
    ("B_not_rounded", "Br[k * N + j] = (float)round_fmt(fmt, B[k * ldb + j]);",
     "Br[k * N + j] = B[k * ldb + j];"),
    ("tc_entries_not_rounded",
     "round_fmt(fmt, A[i * lda + k]) * round_fmt(fmt, B[k * ldb + j])",
     "(double)A[i * lda + k] * (double)B[k * ldb + j]"),
]

# mutants of the attention oracle
ATT_MUTANTS = [
    ("att_no_max_subtraction", "w[j] = exp((double)scale * s0[j] - smax);",
     "w[j] = exp((double)scale * s0[j]);"),
    ("att_scale_dropped", "w[j] = exp((double)scale * s0[j] - smax);",
     "w[j] = exp(s0[j] - smax / (double)scale);"),
    ("att_not_normalised", "        o /= l;\n", ""),
    ("att_sum_skips_first_key", "        l += w[j];", "        if (j > 0) l += w[j];"),
    ("att_dot_drops_last_d", "        for (int64_t d = 0; d < D; ++d) {\n            const double p",
     "        for (int64_t d = 0; d + 1 < D; ++d) {\n            const double p"),
    ("att_value_column_of_key", "o += w[j] * (double)V[j * ldv + d];",
     "o += w[j] * (double)V[j * ldv + (d + j) % D];"),
    ("att_query_row_ignored", "const float* q = Q + i * ldq;", "const float* q = Q;"),
    ("att_bound_drops_accumulation", "(5.0 * (double)Nk + 8.0) * ATT_U * mag", "0.0 * mag"),
    ("att_bound_drops_score_error", "(2.0 * (double)D * ATT_U * delta[j] +",
     "(0.0 * delta[j] +"),
]

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
orc = oracle.Oracle({lib!r})
failed = []
for check in oracle_pins.ALL_CHECKS:
    try:
        check(orc)
    except Exception as e:
        failed.append(check.__name__)
print("FAILED_PINS", ",".join(failed))
"""


CASES = [(m, SRC) for m in MUTANTS] + [(m, SRC_ATT) for m in ATT_MUTANTS]


@pytest.mark.parametrize("mutant,path", CASES, ids=[c[0][0] for c in CASES])
def test_mutant_is_caught(tmp_path, mutant, path):
    name, old, new = mutant
    text = open(path).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique or missing"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    lib = str(tmp_path / f"lib_{name}.so")
    if path == SRC:
        oracle.build(src=str(src), out=lib)
    else:
        oracle.build(src_att=str(src), out=lib)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    proc = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, lib=lib)],
                          capture_output=True, text=True, timeout=300, env=env)
    if proc.returncode != 0:
        return  # crashed on a planted out-of-bounds access: caught
    line = [l for l in proc.stdout.splitlines() if l.startswith("FAILED_PINS")][-1]
    failed = [x for x in line.split(" ", 1)[1].split(",") if x]
    assert failed, f"mutant {name} passed every pin"
