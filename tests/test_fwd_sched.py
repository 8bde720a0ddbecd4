"""The scheduled masked forward (vdx_attn_fwd_ws: a persistent grid pulling
(block, head) items longest first from per-XCD work counters, with key tiles
classified from per-tile summaries) against the plain one (vdx_attn_fwd: one
workgroup per query block, index order, tiles classified from the IDs): the
same bits for every segment layout and size, whatever the workspace holds on
entry, wherever no item is split along its keys (always when a single round
holds every item; the split items of longer launches are tested in
test_fwd_split.py and, at full size, below).  Against the oracle it is checked by the
parity sweeps, which call attn_fwd and so take this path for every masked
case.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (assert_split_close, check_rows, differing_blocks, n_split_items, persistent_grid,
                         run_oracle, valid_rows)

pytestmark = pytest.mark.gpu

KINDS = ["single", "padded", "packed", "interleaved", "singletons", "allpad", "negative", "extreme"]


def _dev(x, seg_q, seg_kv):
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    return d, seg_q.cuda(), seg_kv.cuda()


def run_both(x, seg_q, seg_kv, scale, workspace=None):
    import spatiotemporal_attention_amd as vdx
    d, sq, sk = _dev(x, seg_q, seg_kv)
    o1, l1 = vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=scale, workspace=workspace)
    o2, l2 = vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=scale, scheduled=False)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def assert_same_bits(a, b):
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 65, 257, 1000, 4097])
@pytest.mark.parametrize("kind", KINDS)
def test_scheduled_equals_plain(need_gpu, S, D, kind):
    B, H = (2, 3) if S <= 1000 else (1, 2)
    seed = 31 * S + D
    x = W.make_random(B, S, H, D, seed=seed)
    seg = W.random_segments(B, S, seed + 5, kind)
    print(f"case sched B={B} S={S} H={H} D={D} kind={kind}", flush=True)
    assert_same_bits(*run_both(x, seg, seg.clone(), 1.0 / math.sqrt(D)))


def test_distinct_query_and_key_segments(need_gpu):
    B, S, H, D = 2, 700, 2, 128
    x = W.make_random(B, S, H, D, seed=91)
    seg_q = W.random_segments(B, S, 92, "interleaved")
    seg_kv = W.random_segments(B, S, 93, "packed")
    print("case sched distinct segs", flush=True)
    assert_same_bits(*run_both(x, seg_q, seg_kv, 0.1))


def test_workspace_contents_do_not_matter(need_gpu):
    """A workspace full of garbage, then the same one again (its counters left
    at the previous call's values), then a smaller call in it: every call
    matches the plain path."""
    import spatiotemporal_attention_amd as vdx
    B, S, H, D = 1, 5000, 3, 128
    ws = torch.full((vdx.attn_fwd_workspace_size(B, S, H),), 0xA5, dtype=torch.uint8, device="cuda")
    for i, (s, kind) in enumerate([(S, "packed"), (S, "packed"), (1300, "interleaved")]):
        x = W.make_random(B, s, H, D, seed=300 + i)
        seg = W.random_segments(B, s, 310 + i, kind)
        print(f"case sched workspace reuse {i} S={s}", flush=True)
        assert_same_bits(*run_both(x, seg, seg.clone(), 0.125, workspace=ws))


@pytest.mark.parametrize("name", ["packed_clips"])
def test_full_size_scheduled_equals_plain(need_gpu, name):
    """At the workload's full size (thousands of items, so every workgroup of
    the persistent grid runs many), in the launch configuration the benchmark
    times.  Packed clips' 3,840 items: 13 rounds of each XCD's own items and
    a pool of 512 shared by all XCDs, whose last 64 are split; every other
    block gives the plain call's bits, the split ones agree within the
    rounding of their parts and match the oracle (joint video+text is in
    test_fwd_split.py)."""
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    print(f"case sched full size {name}", flush=True)
    (o1, l1), (o2, l2) = run_both(x, x["seg_q"], x["seg_kv"], w.scale)
    n_split = n_split_items(w.B * w.H * ((w.S + 255) // 256), persistent_grid())
    diff = differing_blocks(o1, l1, o2, l2)
    assert len(diff) <= n_split, (len(diff), n_split)
    assert_split_close(o1, l1, o2, l2)
    # rows of the split blocks (first, last and two random ones) against the oracle
    g = np.random.default_rng(17)
    rows = []
    for b, h, blk in diff:
        lo, hi = blk * 256, min(w.S, (blk + 1) * 256)
        rows += [(b, h, i) for i in sorted({lo, hi - 1} | set(int(i) for i in g.integers(lo, hi, size=2)))]
    if rows:
        rows = np.array(rows, dtype=np.int64)
        oo, lo_, sens = run_oracle(x, x["seg_q"], x["seg_kv"], w.scale, rows=rows)
        has = valid_rows(x["seg_q"], x["seg_kv"], w.B, w.S)
        print(check_rows(o1.cpu(), l1.cpu(), rows, oo, lo_, has, sens), flush=True)


def test_all_ones_at_480p_size_equals_unmasked(need_gpu):
    """All IDs 1 at the 480p layer's size (1,536 items: 4 rounds of each
    XCD's own items and a pool of 512, the last 64 split): every tile is
    full, every block has the same count; the one-workgroup-per-block call
    gives the unmasked call's bits, and the scheduled one too except on the
    split items' blocks, which agree within the rounding of their parts."""
    import spatiotemporal_attention_amd as vdx
    w = W.WORKLOADS["dit480p_small"]
    x = W.make_inputs(w)
    ones = torch.ones((w.B, w.S), dtype=torch.int32)
    print("case sched all-ones 480p", flush=True)
    (o1, l1), (o2, l2) = run_both(x, ones, ones.clone(), w.scale)
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    o3, l3 = vdx.attn_fwd(d["q"], d["k"], d["v"], scale=w.scale)
    torch.cuda.synchronize()
    assert_same_bits((o2, l2), (o3, l3))
    n_split = n_split_items(w.B * w.H * ((w.S + 255) // 256), persistent_grid())
    diff = differing_blocks(o1, l1, o3, l3)
    assert len(diff) <= n_split, (len(diff), n_split)
    assert_split_close(o1, l1, o3, l3)


def test_graph_replays_reset_the_work_counters(need_gpu):
    """The scheduled call captured in a HIP graph (its counters are zeroed by
    a kernel, not a memset), replayed three times with eager work between the
    replays: every replay equals the eager call, bit for bit."""
    import spatiotemporal_attention_amd as vdx
    B, S, H, D = 1, 6000, 2, 128
    x = W.make_random(B, S, H, D, seed=500)
    seg = W.random_segments(B, S, 501, "packed")
    d, sq, sk = _dev(x, seg, seg.clone())
    ref_o, ref_l = vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, scheduled=False)
    ws = torch.empty(vdx.attn_fwd_workspace_size(B, S, H), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, out=out, lse=lse, workspace=ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("case sched graph capture", flush=True)
    with torch.cuda.graph(g):
        vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, out=out, lse=lse, workspace=ws,
                     stream=torch.cuda.current_stream())
    for i in range(3):
        out.zero_()
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"case sched graph replay {i}", flush=True)
        assert_same_bits((out, lse), (ref_o, ref_l))
        # eager work between replays, reusing the same workspace
        vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, workspace=ws)
        torch.cuda.synchronize()
