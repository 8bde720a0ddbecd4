"""The neighbourhood-attention oracle's pins must catch plausible mistakes.

Each mutant is ``oracle/natten_oracle.c`` with one deliberate slip (an
off-by-one window start, a wrong radius, a transposed coordinate decode, a
dropped scale, a wrong value row, a wrong lse), compiled on the CPU into a
temporary library together with the unchanged segment oracle, swapped in, and
run against the pins of ``test_natten_oracle.py``: at least one pin must fail
for every mutant.  Every mutant stays inside the grid, so none can read out
of bounds.  Nothing here touches a GPU.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle.build import NATTEN_SRC, build_oracle
import test_natten_oracle as pins

MUTANTS = [
    ("start_off_by_one", "int64_t s = c - k / 2;", "int64_t s = c - k / 2 + 1;"),
    ("radius_halved", "int64_t s = c - k / 2;", "int64_t s = c - k / 4;"),
    ("x_y_decode_swapped", "const int64_t x = i % J->NW, y = (i / J->NW) % J->NH,",
     "const int64_t x = (i / J->NH) % J->NW, y = i % J->NH,"),
    ("t_window_pinned_to_zero", "const int64_t t0 = window_start(t, J->KT, J->NT);",
     "const int64_t t0 = window_start(0, J->KT, J->NT);"),
    ("scale_dropped", "s_buf[n] = J->scale * dot;", "s_buf[n] = dot;"),
    ("value_of_query_token", "const uint16_t *vj = J->v + elem(J, b, j, h);",
     "const uint16_t *vj = J->v + elem(J, b, i, h);"),
    ("lse_drops_max", "*lse_row = m + log(l);", "*lse_row = log(l);"),
    ("sens_signed", "sens_row[d] += w * fabs(bf16_bits_to_f64(vj[d]));",
     "sens_row[d] += w * bf16_bits_to_f64(vj[d]);"),
    ("sens_unnormalised", "for (int64_t d = 0; d < D; ++d) sens_row[d] /= l;", ""),
]

PIN_FUNCS = [
    lambda: pins.test_matches_sdpa_with_nearest_positions_mask((3, 4, 5), (3, 3, 3)),
    lambda: pins.test_matches_sdpa_with_nearest_positions_mask((4, 5, 6), (3, 5, 3)),
    pins.test_whole_grid_window_is_full_attention,
    pins.test_unit_window_returns_own_value,
    pins.test_zero_query_gives_window_mean_and_constant_volume,
    lambda: pins.test_reflection_along_an_axis_reflects_the_output(0),
    lambda: pins.test_reflection_along_an_axis_reflects_the_output(2),
    pins.test_matches_40_digit_decimal_evaluation,
    pins.test_output_sensitivity_bounds_reduces_and_sums_window_terms,
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="vdx_natten_mut_")
    yield d
    oracle.use_library(None)
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    src = open(NATTEN_SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = os.path.join(workdir, f"lib_{name}.so")
    build_oracle(natten_src=path, out=lib)
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
