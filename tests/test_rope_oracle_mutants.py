"""The 3D rotary-embedding oracle's pins must catch plausible mistakes.

Each mutant is ``oracle/rope_oracle.c`` with one slip (a sign, a swapped
cosine and sine, an operand used twice, the pairing flag ignored, the
frequency order reversed, a table row stride lost, rounding by truncation or
ties away from even), compiled on the CPU with the other oracle sources
unchanged, swapped in and run against the pins of ``test_rope_oracle.py``:
at least one pin must fail for every mutant.  Every mutant keeps its indices
inside the arrays.  Nothing here touches a GPU.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle.build import ROPE_SRC, build_oracle
import test_rope_oracle as pins

MUTANTS = [
    ("first_sign", "const double y0 = x0 * c - x1 * sv;", "const double y0 = x0 * c + x1 * sv;"),
    ("second_swaps_cos_sin", "const double y1 = x0 * sv + x1 * c;", "const double y1 = x0 * c + x1 * sv;"),
    ("first_uses_sin_twice", "const double y0 = x0 * c - x1 * sv;", "const double y0 = x0 * sv - x1 * sv;"),
    ("second_uses_x0_twice", "const double y1 = x0 * sv + x1 * c;", "const double y1 = x0 * sv + x0 * c;"),
    ("pairing_always_interleaved",
     "const int64_t i0 = interleaved ? off + 2 * p : off + p;\n"
     "                        const int64_t i1 = interleaved ? off + 2 * p + 1 : off + p + half;",
     "const int64_t i0 = off + 2 * p;\n"
     "                        const int64_t i1 = off + 2 * p + 1;"),
    ("frequencies_reversed", "const double c = (double)cs[a][ps[a] * half + p];",
     "const double c = (double)cs[a][ps[a] * half + (half - 1 - p)];"),
    ("sin_row_ignored", "const double sv = (double)sn[a][ps[a] * half + p];",
     "const double sv = (double)sn[a][p];"),
    ("rounding_truncates", "if (dlo < dhi)\n        r = lo;", "if (1)\n        r = lo;"),
    ("ties_away_from_zero", "r = (fmod(n, 2.0) == 0.0) ? lo : hi;", "r = hi;"),
]

PIN_FUNCS = [
    pins.test_round_bf16_matches_brute_force,
    lambda: pins.test_zero_angle_returns_input_bits(True),
    lambda: pins.test_quarter_and_half_turns(True),
    lambda: pins.test_quarter_and_half_turns(False),
    lambda: pins.test_complex_multiplication(True, 128, (44, 42, 42)),
    lambda: pins.test_complex_multiplication(False, 64, (20, 22, 22)),
    pins.test_pair_norm_scales_by_table_norm,
    lambda: pins.test_dot_product_depends_on_position_difference(True),
    pins.test_each_axis_moves_only_its_section,
    pins.test_split_halves_is_a_permuted_interleaving,
    pins.test_outside_tables_and_tail_features_untouched,
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="vdx_rope_mut_")
    yield d
    oracle.use_library(None)
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    src = open(ROPE_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = os.path.join(workdir, f"lib_{name}.so")
    build_oracle(rope_src=path, out=lib)
    oracle.use_library(lib)
    failures = 0
    try:
        for fn in PIN_FUNCS:
            try:
                fn()
            except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                failures += 1
    finally:
        oracle.use_library(None)
    assert failures > 0, f"no pin caught mutant {name}"
