"""The oracle's pins reject plausible mistakes.

Each case plants one mistake in a copy of ``oracle/rmsnorm_oracle.c`` (on the
CPU, in a temporary directory), compiles it with the oracle's own flags, and
runs the pin battery of ``test_oracle_pins.py`` against it: at least one pin
must fail.  The planted mistakes are the ones a plain reading of the pages
could plausibly produce (sum instead of mean, eps outside the square root,
another summation order, the unrounded residual normalised, ...).
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "rmsnorm_oracle.c")

FUSED_SUM = (
    "float acc = (float)load(partials[0], base + j, dtype);\n"
    "            for (int q = 1; q < k; ++q) acc = acc + (float)load(partials[q], base + j, dtype);\n"
    "            acc = acc + (float)load(residual, base + j, dtype);"
)

MUTANTS = {
    "mean_as_sum": [("double ms = ss / (double)hidden;", "double ms = ss;")],
    "eps_outside_sqrt": [("1.0 / sqrt(ms + (double)eps)", "1.0 / (sqrt(ms) + (double)eps)")],
    "eps_before_mean": [("double ms = ss / (double)hidden;",
                         "double ms = (ss + (double)eps) / (double)hidden;"),
                        ("1.0 / sqrt(ms + (double)eps)", "1.0 / sqrt(ms)")],
    "residual_added_first": [(FUSED_SUM,
                              "float acc = (float)load(residual, base + j, dtype);\n"
                              "            for (int q = 0; q < k; ++q) acc = acc + (float)load(partials[q], base + j, dtype);")],
    "accumulator_seeded_with_plus_zero": [(FUSED_SUM,
                                           "float acc = 0.0f;\n"
                                           "            for (int q = 0; q < k; ++q) acc = acc + (float)load(partials[q], base + j, dtype);\n"
                                           "            acc = acc + (float)load(residual, base + j, dtype);")],
    "partials_summed_in_double": [("float acc = (float)load(partials[0]", "double acc = load(partials[0]")],
    "normalise_unrounded_sum": [("v[j] = r_new;", "v[j] = (double)acc;")],
    "ties_away_from_zero": [("nearbyint(ldexp(a, -qexp))", "round(ldexp(a, -qexp))")],
    "no_subnormal_binade": [("if (e < f->emin) e = f->emin;", "")],
    "double_rounding_via_float": [("store_exact(base, idx, round_to(v, fmt_of(dtype)), dtype);",
                                   "store_exact(base, idx, round_to((double)(float)v, fmt_of(dtype)), dtype);")],
    "gamma_off_by_one": [("* load(gamma, j, gamma_dtype);",
                          "* load(gamma, (j + 1) % hidden, gamma_dtype);")],
    "gamma_read_in_data_dtype": [("* load(gamma, j, gamma_dtype);", "* load(gamma, j, dtype);")],
    "output_rounded_via_data_dtype": [("if (out) store_rounded(out, base + j, y, out_dtype);",
                                       "if (out) store_rounded(out, base + j, round_to(y, f), out_dtype);")],
    "float_sum_of_squares": [("double ss = 0.0;", "float ss = 0.0f;")],
    "last_element_dropped": [("for (int64_t j = 0; j < hidden; ++j) ss += v[j] * v[j];",
                              "for (int64_t j = 0; j + 1 < hidden; ++j) ss += v[j] * v[j];")],
    "sign_lost_in_rounding": [("return copysign(r, v);", "return r;")],
    "overflow_not_to_inf": [("if (r > maxfin) r = INFINITY;", "if (r > maxfin) r = maxfin;")],
}

# cheap, discriminating pins first
ORDER = ["special_cases", "torch_rms_norm", "residual", "scale", "gamma_one", "brute_force",
         "constant_row", "converters", "general_dtypes"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = oracle.load_library(oracle.compile_library(str(path), str(tmp_path / "libmutant.so")))
    caught = None
    with np.errstate(all="ignore"):
        for pin in ORDER:
            try:
                pins.PINS[pin](lib=lib)
            except (AssertionError, RuntimeError) as e:  # noqa: PERF203
                caught = (pin, repr(e)[:120])
                break
    assert caught is not None, f"mutant {name} passed every pin"
