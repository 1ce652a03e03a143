"""The oracle's pins must catch plausible mistakes.

Each case copies the C oracle, plants one mistake by a textual edit, compiles the
copy with gcc and runs the pin suite against it in a subprocess; the suite must
fail.  The oracle source itself is never modified.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "w4_oracle.c")

MUTANTS = {
    "nibble_order_reversed": ("(word >> (4 * (k % 8)))", "(word >> (4 * (7 - k % 8)))"),
    "offset_7_not_8": ("w4o_code(codes, K, n, k) - 8)", "w4o_code(codes, K, n, k) - 7)"),
    "step_index_k_over_64": ("steps[n * (K / 32) + k / 32]", "steps[n * (K / 32) + k / 64]"),
    "bound_without_abs": ("mag += fabs(p);\n        }\n        y[n - n0] = acc;\n        if (a)",
                          "mag += p;\n        }\n        y[n - n0] = acc;\n        if (a)"),
    "bound_without_abs_exact_input": ("mag += fabs(p);\n        }\n        y[n - n0] = acc;\n        a[n - n0]",
                                      "mag += p;\n        }\n        y[n - n0] = acc;\n        a[n - n0]"),
    "exact_input_ignores_x": ("double p = w4o_weight(codes, steps, K, n, k) * x[k];",
                              "double p = w4o_weight(codes, steps, K, n, k) * x[0];"),
    "bf16_bias_off_by_one": ("e - 134", "e - 133"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "round_half_up": ("nearbyint(a / quantum)", "floor(a / quantum + 0.5)"),
    "side_input_by_slot": ("row_scale[e * N + n]", "row_scale[a * N + n]"),
    "route_weight_dropped": ("Y[t * N + n] += r * v;", "Y[t * N + n] += v;"),
    "rms_over_k_minus_1": ("sqrt(ss / (double)K)", "sqrt(ss / (double)(K - 1))"),
    "x_index_per_pair_ignored": ("(x_per_pair ? (t * topk + j) : t)", "(t)"),
    "grid_step_always_eighth": ("an > ap ? an / 8.0 : ap / 7.0", "an > ap ? an / 8.0 : ap / 8.0"),
    "grid_tie_to_negative": ("an > ap ? an / 8.0", "an >= ap ? an / 8.0"),
    "grid_clamp_upper_14": ("(q > 15.0 ? 15.0 : q)", "(q > 14.0 ? 14.0 : q)"),
    "grid_truncates": ("nearbyint(v[8 * w + j] / step)", "trunc(v[8 * w + j] / step)"),
    # the quotient as the fp32 product with the step's reciprocal
    "grid_reciprocal_fp32": ("nearbyint(v[8 * w + j] / step)",
                             "nearbyint((double)((float)v[8 * w + j] * (1.0f / (float)step)))"),
    # no search for the group's own grid: always the extreme rule
    "grid_extreme_rule_only": ("j <= jmax && !found", "j <= 0 && !found"),
    # the finest grid that holds the group instead of the coarsest
    "grid_finest_not_coarsest": ("for (int j = 1; j <= jmax && !found; ++j)",
                                 "for (int j = jmax; j >= 1 && !found; --j)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                           "-o", str(so), str(mut), "-lm"])
    env = dict(os.environ, W4O_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
