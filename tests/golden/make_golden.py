"""Writes tests/golden/oracle_tiny_packed.json from the oracle alone.

The pages print no attention inputs or outputs (vidax paper: no worked
example), so this fixture is a regression anchor for the oracle, not a page
value: it freezes the oracle's fp64 output on a tiny seeded packed-segment
case so that any later change to the oracle's arithmetic shows up.  Only
``oracle/`` and the input generators are called here.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as W  # noqa: E402

CASE = dict(B=1, S=12, H=1, D=64, seed=777, seg_seed=778, scale=0.125)


def main():
    c = CASE
    x = W.make_random(c["B"], c["S"], c["H"], c["D"], seed=c["seed"], sigma_qk=2.0)
    seg = W.random_segments(c["B"], c["S"], c["seg_seed"], "packed")
    out, lse, _ = oracle.attn_fwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                  seg.numpy(), seg.numpy(), c["scale"], n_threads=1)
    doc = {
        "what": "oracle fp64 output on a tiny seeded packed-segment case (regression anchor)",
        "source": "written by tests/golden/make_golden.py from oracle/ only; the pages print no values",
        "case": c,
        "sigma_qk": 2.0,
        "segments": seg.tolist(),
        "out": [float.hex(float(t)) for t in out.reshape(-1)],
        "lse": [float.hex(float(t)) for t in lse.reshape(-1)],
    }
    with open(os.path.join(HERE, "oracle_tiny_packed.json"), "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
