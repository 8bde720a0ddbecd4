"""The gradient oracle's pins must catch plausible mistakes.

Each mutant is ``oracle/attn_bwd_oracle.c`` with one slip (the delta term
dropped, a missing scale, a transposed probability or score-gradient index,
the wrong operand in a product, an unnormalised softmax, padding matching
padding), compiled on the CPU with the other oracle sources unchanged,
swapped in and run against the pins of ``test_bwd_oracle.py``: at least one
pin must fail for every mutant.  Nothing here touches a GPU.
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
]

PIN_FUNCS = [
    lambda: pins.test_matches_torch_autograd_f64("packed", 64),
    lambda: pins.test_matches_torch_autograd_f64(None, 128),
    pins.test_matches_central_differences,
    pins.test_singletons_pass_dout_to_dv_only,
    pins.test_constant_value_gives_zero_dq_dk,
    pins.test_zero_query_closed_form,
    pins.test_segment_sums_and_masked_rows,
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="vdx_bwd_mut_")
    yield d
    oracle.use_library(None)
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    src = open(BWD_SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
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
