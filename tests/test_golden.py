"""Regression anchor: the oracle reproduces its frozen fp64 output bit for bit
(tests/golden/oracle_tiny_packed.json, written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_tiny_packed.json")


def test_oracle_matches_frozen_fixture():
    doc = json.load(open(GOLD))
    c = doc["case"]
    x = W.make_random(c["B"], c["S"], c["H"], c["D"], seed=c["seed"], sigma_qk=doc["sigma_qk"])
    seg = np.array(doc["segments"], dtype=np.int32)
    assert np.array_equal(seg, W.random_segments(c["B"], c["S"], c["seg_seed"], "packed").numpy())
    out, lse, _ = oracle.attn_fwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                  seg, seg, c["scale"], n_threads=3)
    want_out = np.array([float.fromhex(t) for t in doc["out"]]).reshape(out.shape)
    want_lse = np.array([float.fromhex(t) for t in doc["lse"]]).reshape(lse.shape)
    assert np.array_equal(out, want_out)
    assert np.array_equal(np.isneginf(lse), np.isneginf(want_lse))
    fin = ~np.isneginf(lse)
    assert np.array_equal(lse[fin], want_lse[fin])
