"""The oracle's pins must catch plausible mistakes.

Each mutant is the oracle source with one deliberate slip (a flipped sign, a
dropped term, a wrong index, a wrong masking rule).  It is compiled on the CPU
into a temporary library, swapped in, and the pin suite of ``test_oracle.py``
is run against it: at least one pin must fail for every mutant.  Nothing here
touches a GPU.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from oracle.build import SRC, build_oracle
import test_oracle as pins

# (name, original text, replacement) -- each original must occur in the source.
MUTANTS = [
    ("exp_sign", "exp(s_buf[j] - m)", "exp(m - s_buf[j])"),
    ("scale_dropped", "s_buf[j] = J->scale * dot;", "s_buf[j] = dot;"),
    ("key_uses_query_index", "const uint16_t *kj = J->k + tok_index(J, b, j, h);",
     "const uint16_t *kj = J->k + tok_index(J, b, i, h);"),
    ("value_uses_query_index", "const uint16_t *vj = J->v + tok_index(J, b, j, h);",
     "const uint16_t *vj = J->v + tok_index(J, b, i, h);"),
    ("pad_matches_pad", "ok = (c != 0) && (J->seg_kv[b * S + j] == c);",
     "ok = (J->seg_kv[b * S + j] == c);"),
    ("kv_reads_seg_q", "ok = (c != 0) && (J->seg_kv[b * S + j] == c);",
     "ok = (c != 0) && (J->seg_q[b * S + j] == c);"),
    ("lse_drops_max", "*lse_row = m + log(l);", "*lse_row = log(l);"),
    ("no_normalisation", "for (int64_t d = 0; d < D; ++d) out_row[d] /= l;", ""),
    ("dot_drops_last_term",
     "for (int64_t d = 0; d < D; ++d) dot += bf16_to_f64(qi[d]) * bf16_to_f64(kj[d]);",
     "for (int64_t d = 0; d + 1 < D; ++d) dot += bf16_to_f64(qi[d]) * bf16_to_f64(kj[d]);"),
    ("masked_row_lse_zero", "*lse_row = -INFINITY;", "*lse_row = 0.0;"),
    ("head_index_dropped", "return ((b * J->S + s) * J->H + h) * J->D;",
     "return ((b * J->S + s) * J->H) * J->D;"),
    ("bf16_low_bits", "uint32_t w = ((uint32_t)bits) << 16;", "uint32_t w = ((uint32_t)bits) << 15;"),
    ("out_overwritten_not_summed", "out_row[d] += w * bf16_to_f64(vj[d]);",
     "out_row[d] = w * bf16_to_f64(vj[d]);"),
    # the output rounding-sensitivity sums
    ("sens_signed", "sens_row[d] += w * fabs(bf16_to_f64(vj[d]));", "sens_row[d] += w * bf16_to_f64(vj[d]);"),
    ("sens_unnormalised", "for (int64_t d = 0; d < D; ++d) sens_row[d] /= l;", ""),
    ("sens_weight_squared", "sens_row[d] += w * fabs(bf16_to_f64(vj[d]));",
     "sens_row[d] += w * w * fabs(bf16_to_f64(vj[d]));"),
]

PIN_FUNCS = [
    lambda: pins.test_matches_torch_sdpa_f64(64, "packed"),
    lambda: pins.test_matches_torch_sdpa_f64(128, "interleaved"),
    pins.test_unmasked_matches_torch_sdpa_f64,
    pins.test_singleton_segments_return_own_value,
    pins.test_zero_query_gives_segment_mean,
    pins.test_constant_value_returned,
    pins.test_two_token_segment_is_logistic_blend,
    lambda: pins.test_arithmetic_progression_scores_geometric_series(0.05),
    pins.test_fully_masked_rows_zero_and_neg_inf,
    pins.test_query_segment_without_keys_is_masked,
    pins.test_probability_rows_sum_to_one_and_vanish_off_segment,
    pins.test_other_segment_does_not_leak,
    pins.test_lse_bounds,
    pins.test_matches_40_digit_decimal_evaluation,
    lambda: pins.test_output_sensitivity_equals_first_order_deviation("packed"),
    pins.test_output_sensitivity_bounds_and_reduces,
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="vdx_oracle_mut_")
    yield d
    oracle.use_library(None)
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = os.path.join(workdir, f"lib_{name}.so")
    build_oracle(src=path, out=lib)
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
