"""The gradient oracle's pins must catch plausible mistakes.

Each mutant is ``oracle/attn_bwd_oracle.c`` with one slip (the delta term
dropped, a missing scale, a transposed probability or score-gradient index,
the wrong operand in a product, an unnormalised softmax, padding matching
padding), compiled on the CPU with the other oracle sources unchanged,
swapped in and run against the pins of ``test_bwd_oracle.py``: at least one
pin must fail for every mutant.  The slips in the rounding-sensitivity sums
(which set the GPU backward's per-element tolerance) are made the same way in
the dense and the row function, so that the two still agree with each other.
Nothing here touches a GPU.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle.build import BWD_SRC, build_oracle
import test_bwd_oracle as pins

MUTANTS = [
    ("delta_dropped", "dS[i * S + j] = P[i * S + j] * (dS[i * S + j] - delta);",
     "dS[i * S + j] = P[i * S + j] * dS[i * S + j];"),
    ("dq_no_scale", "J->dq[at(J, b, i, h) + d] = J->scale * acc[d];",
     "J->dq[at(J, b, i, h) + d] = acc[d];"),
    ("dk_uses_k", "acc[d] += ds * b2d(qi[d]);",
     "acc[d] += ds * b2d(J->k[at(J, b, i, h) + d]);"),
    # after the in-place transpose P[j * S + i] holds P_ij
    ("dv_transposed_p", "accv[d] += p * b2d(oi[d]);",
     "accv[d] += P[i * S + j] * b2d(oi[d]);"),
    ("dp_uses_q", "dp += b2d(J->dout[at(J, b, i, h) + d]) * b2d(J->v[at(J, b, j, h) + d]);",
     "dp += b2d(J->q[at(J, b, i, h) + d]) * b2d(J->v[at(J, b, j, h) + d]);"),
    ("softmax_unnormalised", "P[i * S + j] = (l > 0.0) ? P[i * S + j] / l : 0.0;",
     "P[i * S + j] = P[i * S + j];"),
    ("pad_matches_pad", "return c != 0 && J->seg_kv[b * J->S + j] == c;",
     "return J->seg_kv[b * J->S + j] == c;"),
    ("dq_transposed_ds", "const double ds = dS[i * S + j];",
     "const double ds = dS[j * S + i];"),
    # rounding-sensitivity sums, each slip in both the dense and the row function
    ("sens_e_doubled", [("E[i] = e;", "E[i] = 2.0 * e;"),
                        ("+ P[j] * e) * fabs", "+ 2.0 * P[j] * e) * fabs")]),
    ("sens_e_dropped", [("const double w = fabs(ds) + P[i * S + j] * E[i];", "const double w = fabs(ds);"),
                        ("const double w = fabs(ds) + p * E[i];", "const double w = fabs(ds);"),
                        ("+ P[j] * e) * fabs", ") * fabs")]),
    ("sens_no_scale", [("if (E) J->tq[at(J, b, i, h) + d] = J->scale * tacc[d];",
                        "if (E) J->tq[at(J, b, i, h) + d] = tacc[d];"),
                       ("J->tk[at(J, b, j, h) + d] = J->scale * tacc[d];", "J->tk[at(J, b, j, h) + d] = tacc[d];"),
                       ("tq[d] = J->scale * t;", "tq[d] = t;")]),
    # E_i from |dout_i . v_j| instead of sum_d |dout_id| |v_jd|
    ("sens_e_abs_of_dot", [("a += fabs(b2d(J->dout[at(J, b, i, h) + d])) * fabs(b2d(J->v[at(J, b, j, h) + d]));\n"
                            "                e += P[i * S + j] * a;",
                            "a += b2d(J->dout[at(J, b, i, h) + d]) * b2d(J->v[at(J, b, j, h) + d]);\n"
                            "                e += P[i * S + j] * fabs(a);"),
                           ("a += fabs(b2d(J->dout[at(J, b, i, h) + d])) * fabs(b2d(J->v[at(J, b, j, h) + d]));\n"
                            "            e += P[j] * a;",
                            "a += b2d(J->dout[at(J, b, i, h) + d]) * b2d(J->v[at(J, b, j, h) + d]);\n"
                            "            e += P[j] * fabs(a);")]),
    # |dS_ij| replaced by P_ij |dP_ij| (delta left out of the magnitude)
    ("sens_ds_without_delta", [("const double w = fabs(ds) + P[i * S + j] * E[i];",
                                "const double w = fabs(ds + P[i * S + j] * dl[i]) + P[i * S + j] * E[i];"),
                               ("const double w = fabs(ds) + p * E[i];",
                                "const double w = fabs(ds + p * dl[i]) + p * E[i];"),
                               ("E[i] = e;", "E[i] = e;\n            dl[i] = delta;"),
                               ("double *acc = (double *)malloc(sizeof(double) * (size_t)(4 * D));",
                                "double *acc = (double *)malloc(sizeof(double) * (size_t)(4 * D));\n"
                                "    static __thread double dl[4096];"),
                               ("t += (fabs(P[j] * (dP[j] - delta)) + P[j] * e)", "t += (P[j] * fabs(dP[j]) + P[j] * e)")]),
    # |k_jd| without the absolute value in tq
    ("sens_k_signed", [("for (int64_t d = 0; d < D; ++d) tacc[d] += w * fabs(b2d(kj[d]));",
                        "for (int64_t d = 0; d < D; ++d) tacc[d] += w * b2d(kj[d]);"),
                       ("+ P[j] * e) * fabs(b2d(J->k[at(J, b, j, h) + d]));", "+ P[j] * e) * b2d(J->k[at(J, b, j, h) + d]);")]),
]

PIN_FUNCS = [
    lambda: pins.test_matches_torch_autograd_f64("packed", 64),
    lambda: pins.test_matches_torch_autograd_f64(None, 128),
    pins.test_matches_central_differences,
    pins.test_singletons_pass_dout_to_dv_only,
    pins.test_constant_value_gives_zero_dq_dk,
    pins.test_zero_query_closed_form,
    pins.test_segment_sums_and_masked_rows,
    pins.test_sensitivity_sums_bound_and_reduce,
    pins.test_dq_rows_sensitivity_matches_dense,
    lambda: pins.test_sensitivity_sums_equal_first_order_deviation("packed_signed"),
    lambda: pins.test_sensitivity_sums_equal_first_order_deviation("packed_nonneg_k"),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="vdx_bwd_mut_")
    yield d
    oracle.use_library(None)
    shutil.rmtree(d, ignore_errors=True)


def _edits(m):
    """(name, old, new) or (name, [(old, new), ...]) -> [(old, new), ...]."""
    return [(m[1], m[2])] if len(m) == 3 else list(m[1])


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, mutant):
    name = mutant[0]
    src = open(BWD_SRC).read()
    for old, new in _edits(mutant):
        assert src.count(old) >= 1, f"mutation site for {name} not found: {old!r}"
        src = src.replace(old, new, 1)
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(workdir, f"lib_{name}.so")
    build_oracle(bwd_src=path, out=lib)
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
