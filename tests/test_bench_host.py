"""Host logic of bench.py, on the CPU: the multi-GPU refusal, the FLOP and
byte counts behind `value` and `roofline`, and the rule that ties the
committed HBM-counter summaries to the kernel sources they were taken on.

The expected FLOP and byte figures were worked out separately from the
workload definitions (valid-pair FLOP = 4 D H x #valid pairs, algorithmic
bytes = read q, k, v and segment IDs, write out and lse); the counts here
come from bench.py's run-length formulas and, independently, from the
per-token segment arrays the tests and the benchmark feed the kernel.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402

# name: (valid-pair TFLOP, dense TFLOP, algorithmic GB), 4 significant digits
EXPECTED = {
    "tiny_ref": (1.074e-3, 1.074e-3, 2.1e-3),
    "dit480p_small": (6.594, 6.594, 0.4038),
    "joint_video_text_pad": (7.766, 7.892, 0.8850),
    "dit720p_large": (117.05, 117.05, 3.109),
    "packed_clips": (11.677, 30.924, 1.011),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_flop_and_byte_counts(name):
    w = W.WORKLOADS[name]
    valid_t, dense_t, gb = EXPECTED[name]
    flop = 4.0 * w.D * w.H * bench.valid_pairs(w)
    assert flop / 1e12 == pytest.approx(valid_t, rel=1e-3)
    assert 4.0 * w.D * w.H * w.B * w.S * w.S / 1e12 == pytest.approx(dense_t, rel=1e-3)
    assert bench.algorithmic_bytes(w) / 1e9 == pytest.approx(gb, rel=2e-2)


@pytest.mark.parametrize("name", [n for n, w in W.WORKLOADS.items() if w.seg_runs is not None])
def test_valid_pairs_match_the_token_arrays(name):
    """Count valid pairs from the per-token ID array (ID 0 matches nothing)."""
    w = W.WORKLOADS[name]
    seg = W.seg_from_runs(w.seg_runs, w.B, w.S).numpy()
    total = 0
    for b in range(w.B):
        ids, counts = np.unique(seg[b], return_counts=True)
        total += int(sum(int(c) * int(c) for i, c in zip(ids, counts) if i != 0))
    assert bench.valid_pairs(w) == total


def test_natten_counts():
    w = W.NATTEN_WORKLOADS["natten_vae_decoder"]
    # every query sees the full 11^3 window (it shifts inward at the borders)
    assert bench.natten_window_volume(w) == 11 ** 3
    assert bench.natten_brick_frames(16, 32, 11, 11) == 4   # 14 x 12 rows beat 11 x 18
    assert bench.natten_brick_frames(1, 32, 11, 11) == 1    # single frame: 1 x 8 bricks
    assert bench.natten_brick_frames(16, 32, 1, 11) == 1    # 1-frame t window
    # 8 heads x 8,952 two-row steps per head (4x2x32 bricks walk up to 14
    # frames x 12 key rows, fewer where windows clip at the borders), each
    # step 2 rows x 8 waves x 32 queries x 16 keys x 2 products x 2 D
    assert bench.natten_executed_flop(w) == pytest.approx(8 * 8952 * 2 * 8 * 32 * 16 * 4 * 128, rel=0)


def test_traffic_served_only_for_matching_sources(tmp_path, monkeypatch):
    import json
    doc = {"kernel_source_sha256": bench.kernel_source_hash(), "traffic_bytes_per_launch": 123}
    (tmp_path / "attn_fwd_dit720p_large_hbm_counters.json").write_text(json.dumps(doc))
    monkeypatch.setattr(bench, "COUNTERS_DIR", str(tmp_path))
    assert bench.load_traffic("dit720p_large") == 123
    doc["kernel_source_sha256"] = "0" * 64
    (tmp_path / "attn_fwd_dit720p_large_hbm_counters.json").write_text(json.dumps(doc))
    assert bench.load_traffic("dit720p_large") is None
    assert bench.load_traffic("packed_clips") is None  # no summary for it
    # the neighbourhood kernel's summary is keyed on its own sources
    doc = {"kernel_source_sha256": bench.kernel_source_hash(bench.NATTEN_KERNEL_SOURCES),
           "traffic_bytes_per_launch": 456}
    (tmp_path / "natten_fwd_vae_decoder_hbm_counters.json").write_text(json.dumps(doc))
    assert bench.load_traffic("natten_vae_decoder", "natten") == 456
    doc["kernel_source_sha256"] = bench.kernel_source_hash()
    (tmp_path / "natten_fwd_vae_decoder_hbm_counters.json").write_text(json.dumps(doc))
    assert bench.load_traffic("natten_vae_decoder", "natten") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_docs():
    import glob
    import json
    return [(os.path.basename(p), json.load(open(p)))
            for p in sorted(glob.glob(os.path.join(bench.COUNTERS_DIR, "*_hbm_counters.json")))]


@pytest.mark.parametrize("name,doc", _counter_docs(), ids=[n for n, _ in _counter_docs()])
def test_counter_summaries_are_consistent(name, doc):
    """Each committed FETCH_SIZE/WRITE_SIZE summary: the copy calibration gives
    its scale factors, the per-launch bytes are the per-dispatch KiB times
    1024 times those factors, the traffic is their sum, the algorithmic bytes
    are bench.py's, and the stored commands run committed files only."""
    cal = doc["copy_calibration"]
    copy_kib = cal["copy_bytes"] / 1024
    assert cal["fetch_factor"] == pytest.approx(copy_kib / cal["fetch_size_kib"], rel=1e-3)
    assert cal["write_factor"] == pytest.approx(copy_kib / cal["write_size_kib"], rel=1e-3)
    # every kernel of a call (backward: prep, sweeps and block order; masked
    # forward: set-up kernels and the persistent kernel; else one kernel)
    fb = sum(k["fetch_bytes"] for k in doc["kernels"].values())
    wb = sum(k["write_bytes"] for k in doc["kernels"].values())
    for k in doc["kernels"].values():  # the KiB figures are stored to 0.1 KiB
        for c in ("fetch", "write"):
            f = cal[c + "_factor"]
            assert k[c + "_bytes"] == pytest.approx(k[c + "_size_kib_per_dispatch"] * 1024 * f,
                                                    rel=1e-6, abs=0.06 * 1024 * f)
    if name.startswith("attn_bwd_"):
        assert doc["traffic_bytes_per_call"] == pytest.approx(fb + wb, rel=1e-9)
        w = W.WORKLOADS[name[len("attn_bwd_"):-len("_hbm_counters.json")]]
        n = w.B * w.S * w.H * w.D
        assert doc["algorithmic_bytes_per_call"] == 2 * 8 * n + 4 * w.B * w.H * w.S
    else:
        assert doc["traffic_bytes_per_launch"] == pytest.approx(fb + wb, rel=1e-9)
        if name.startswith("natten_fwd_"):
            w = W.NATTEN_WORKLOADS["natten_" + name[len("natten_fwd_"):-len("_hbm_counters.json")]]
            n = w.B * w.S * w.H * w.D
            assert doc["algorithmic_bytes_per_launch"] == 4 * 2 * n + 4 * w.B * w.H * w.S
        else:
            w = W.WORKLOADS[name[len("attn_fwd_"):-len("_hbm_counters.json")]]
            assert doc["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(w)
    for c in doc["commands"]:
        assert "rocprofv3 --pmc" in c and "-- python3 /root/repo/bench.py" in c
        assert "_work" not in c


@pytest.mark.parametrize("args", [["--plain", "--rope"], ["--plain", "--pass", "bwd"],
                                  ["--plain", "--workload", "natten_vae_decoder"]])
def test_plain_entry_only_for_the_attention_forward(args):
    """--plain (time vdx_attn_fwd instead of vdx_attn_fwd_ws) is refused with
    the rotary call, the backward and the neighbourhood kernel, before any GPU
    work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--plain applies to the attention forward" in r.stderr
    assert r.stdout == ""
