"""Split items of vdx_attn_fwd_ws.  In a persistent launch with more items
than workgroups, some items are divided along their active key tiles into
parts that run side by side: without segment IDs each XCD's last items (a
quarter round's worth in a long launch, its ragged last round in a short
one), the XCDs stealing units from each other; with them the last items of
a pool of items shared by all XCDs.  A combine kernel merges the parts'
(O, m, l).

Against vdx_attn_fwd (which never splits): every query block that is not
split gives the same bits; the split ones round their probabilities against
each part's own reference maximum, so they agree to within that rounding
(lse, summed from unrounded probabilities, to about 1e-6).  Against the oracle: rows of the split blocks at
the parity bar, with the blocks and parts chosen so that parts with no key
tile, padding rows and ragged tails all occur.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (assert_split_close, block_mask, check_rows, differing_blocks, n_split_items,
                         persistent_grid, run_oracle, split_unmasked_blocks, valid_rows)

pytestmark = pytest.mark.gpu


def _run(x, seg_q, seg_kv, scale, split):
    import spatiotemporal_attention_amd as vdx
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    sq = None if seg_q is None else seg_q.cuda()
    sk = None if seg_kv is None else seg_kv.cuda()
    B, S, H, _ = x["q"].shape
    ws = torch.empty(vdx.attn_fwd_workspace_size(B, S, H), dtype=torch.uint8, device="cuda") if split else None
    o, l = vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=scale, workspace=ws, scheduled=split)
    torch.cuda.synchronize()
    return o, l


def _rows_of(blocks, S, per_block, seed):
    g = np.random.default_rng(seed)
    rows = []
    for b, h, blk in blocks:
        lo, hi = blk * 256, min(S, (blk + 1) * 256)
        picks = {lo, hi - 1} | set(int(i) for i in g.integers(lo, hi, size=per_block))
        rows += [(b, h, i) for i in sorted(picks)]
    return np.array(rows, dtype=np.int64)


def _check_against_oracle(x, seg_q, seg_kv, scale, o, l, blocks, per_block, seed):
    B, S, H, D = x["q"].shape
    rows = _rows_of(blocks, S, per_block, seed)
    oo, lo, sens = run_oracle(x, seg_q, seg_kv, scale, rows=rows)
    has = valid_rows(seg_q, seg_kv, B, S)
    return check_rows(o.cpu(), l.cpu(), rows, oo, lo, has, sens)


@pytest.mark.parametrize("B,S,H,D", [(1, 8192, 9, 128), (1, 8192, 9, 64), (2, 4000, 10, 128), (1, 32760, 12, 128),
                                     (1, 75600, 40, 128)])
def test_unmasked_split_blocks(need_gpu, B, S, H, D):
    """Unmasked: only the blocks the schedule splits differ from vdx_attn_fwd,
    within rounding; their rows match the oracle."""
    grid = persistent_grid()
    blocks = split_unmasked_blocks(B, S, H, grid)
    if not blocks:
        pytest.skip(f"{B * H * ((S + 255) // 256)} items on a {grid}-workgroup grid split none")
    if S in (75600, 32760):
        w = W.WORKLOADS["dit720p_large" if S == 75600 else "dit480p_small"]
        x, scale = W.make_inputs(w), w.scale
    else:
        x, scale = W.make_random(B, S, H, D, seed=S + H + D), 1.0 / math.sqrt(D)
    print(f"case split unmasked B={B} S={S} H={H} D={D} split blocks={len(blocks)}", flush=True)
    o1, l1 = _run(x, None, None, scale, split=True)
    o2, l2 = _run(x, None, None, scale, split=False)
    diff = differing_blocks(o1, l1, o2, l2)
    assert set(diff) <= set(blocks), sorted(set(diff) - set(blocks))[:8]
    m = block_mask(B, H, S, blocks)
    keep = torch.from_numpy(~m)
    assert torch.equal(o1.view(torch.int16).cpu()[keep], o2.view(torch.int16).cpu()[keep])
    assert_split_close(o1, l1, o2, l2)
    sample = blocks[::max(1, len(blocks) // 16)]
    stats = _check_against_oracle(x, None, None, scale, o1, l1, sample, 4 if S > 20000 else 16, S)
    print(stats, flush=True)


@pytest.mark.parametrize("kind", ["singletons", "packed", "padded", "allpad", "negative"])
def test_masked_split_blocks(need_gpu, kind):
    """Masked (the scheduled persistent kernel): 288 items on a 256-workgroup
    grid leave a pool of 32 items, split 8 ways; with one-token segments a
    block has about 4 active tiles, so most parts get none.
    At most the split items' blocks differ from vdx_attn_fwd; their rows
    match the oracle and padding rows stay +0.0 / -inf."""
    B, S, H, D = 1, 8192, 9, 128
    grid = persistent_grid()
    n_items = B * H * ((S + 255) // 256)
    n_split = n_split_items(n_items, grid)
    if n_split == 0:
        pytest.skip(f"{n_items} items on a {grid}-workgroup grid split none")
    x = W.make_random(B, S, H, D, seed=7000 + len(kind))
    seg = W.random_segments(B, S, 7100 + len(kind), kind)
    print(f"case split masked kind={kind} items={n_items} split={n_split}", flush=True)
    o1, l1 = _run(x, seg, seg.clone(), 0.1, split=True)
    o2, l2 = _run(x, seg, seg.clone(), 0.1, split=False)
    diff = differing_blocks(o1, l1, o2, l2)
    assert len(diff) <= n_split, (len(diff), n_split)
    assert_split_close(o1, l1, o2, l2)
    if diff:
        print(_check_against_oracle(x, seg, seg, 0.1, o1, l1, diff, 16, 11), flush=True)
    has = valid_rows(seg, seg, B, S)
    dead = torch.from_numpy(~has)
    assert torch.all(o1.view(torch.int16).cpu()[dead] == 0)
    assert torch.all(torch.isneginf(l1.cpu().permute(0, 2, 1)[dead]))


def test_joint_video_text_split_tail(need_gpu):
    """The padded joint video+text workload at full size (3,360 items: 11
    rounds of 256 and 32 items left; 11 rounds of each XCD's own items, a
    pool of 544 and its last 64 split 4 ways): at most 64 blocks differ from vdx_attn_fwd, within rounding, and
    their rows (text, video and pad rows among them) match the oracle."""
    w = W.WORKLOADS["joint_video_text_pad"]
    x = W.make_inputs(w)
    n_items = w.B * w.H * ((w.S + 255) // 256)
    n_split = n_split_items(n_items, persistent_grid())
    print(f"case split joint video+text split={n_split}", flush=True)
    o1, l1 = _run(x, x["seg_q"], x["seg_kv"], w.scale, split=True)
    o2, l2 = _run(x, x["seg_q"], x["seg_kv"], w.scale, split=False)
    diff = differing_blocks(o1, l1, o2, l2)
    assert len(diff) <= n_split, (len(diff), n_split)
    assert_split_close(o1, l1, o2, l2)
    if diff:
        print(_check_against_oracle(x, x["seg_q"], x["seg_kv"], w.scale, o1, l1, diff, 4, 13), flush=True)


def test_split_workspace_reuse_and_smaller_call(need_gpu):
    """One workspace, garbage on entry, used by a split unmasked call, a split
    masked call and a smaller unsplit call: each equals a fresh-workspace run
    bit for bit (the part records are written before the combine reads them)."""
    import spatiotemporal_attention_amd as vdx
    B, S, H, D = 1, 8192, 9, 128
    ws = torch.full((vdx.attn_fwd_workspace_size(B, S, H),), 0x7F, dtype=torch.uint8, device="cuda")
    x = W.make_random(B, S, H, D, seed=8100)
    seg = W.random_segments(B, S, 8101, "packed")
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    for i, (sq, s_len) in enumerate([(None, S), (seg, S), (None, 3000)]):
        dd = {n: t[:, :s_len].contiguous() for n, t in d.items()}
        sqd = None if sq is None else sq[:, :s_len].contiguous().cuda()
        print(f"case split workspace reuse {i}", flush=True)
        o1, l1 = vdx.attn_fwd(dd["q"], dd["k"], dd["v"], sqd, None if sqd is None else sqd.clone(), scale=0.1,
                              workspace=ws)
        fresh = torch.empty_like(ws)
        o2, l2 = vdx.attn_fwd(dd["q"], dd["k"], dd["v"], sqd, None if sqd is None else sqd.clone(), scale=0.1,
                              workspace=fresh)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def _rope_run(x, r, seg, scale, split):
    import spatiotemporal_attention_amd as vdx
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    sd = None if seg is None else seg.cuda()
    rr = dict(pos=r.pos.cuda(), cos=[c.cuda() for c in r.cos], sin=[s.cuda() for s in r.sin], dims=r.dims,
              interleaved=r.interleaved)
    B, S, H, _ = x["q"].shape
    ws = torch.empty(vdx.attn_fwd_workspace_size(B, S, H), dtype=torch.uint8, device="cuda") if split else None
    o, l = vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], **rr, seg_q=sd, seg_kv=sd, scale=scale, workspace=ws,
                               scheduled=split)
    torch.cuda.synchronize()
    return o, l


@pytest.mark.parametrize("D,kind", [(128, None), (64, None), (128, "packed"), (64, "padded")])
def test_rope_split_blocks(need_gpu, D, kind):
    """vdx_rope3d_attn_fwd_ws with split items (288 items on a 256-workgroup
    grid: 4 items per XCD split 8 ways unmasked, a pool of 32 items split 8
    ways masked)
    against vdx_rope3d_attn_fwd: at most the split blocks differ, within
    rounding, and their rows match the oracle (rotation, then attention)."""
    import oracle
    B, S, H = 1, 8192, 9
    grid = persistent_grid()
    n_items = B * H * ((S + 255) // 256)
    n_split = n_split_items(n_items, grid, masked=kind is not None)
    if n_split == 0:
        pytest.skip(f"{n_items} items on a {grid}-workgroup grid split none")
    x = W.make_random(B, S, H, D, seed=9000 + D)
    dims = W.ROPE_DIMS[D]
    n = (8, 16, 64)
    tabs = [W.rope3d_tables(n[a], dims[a]) for a in range(3)]
    r = W.Rope3D(pos=W.random_positions(B, S, n, 9001 + D, 0.05), cos=tuple(t[0] for t in tabs),
                 sin=tuple(t[1] for t in tabs), dims=tuple(dims), interleaved=True)
    seg = None if kind is None else W.random_segments(B, S, 9002 + D, kind)
    scale = 1.0 / math.sqrt(D)
    print(f"case split rope D={D} kind={kind} split={n_split}", flush=True)
    o1, l1 = _rope_run(x, r, seg, scale, split=True)
    o2, l2 = _rope_run(x, r, seg, scale, split=False)
    diff = differing_blocks(o1, l1, o2, l2)
    assert len(diff) <= n_split, (len(diff), n_split)
    if kind is None:
        assert set(diff) <= set(split_unmasked_blocks(B, S, H, grid))
    assert_split_close(o1, l1, o2, l2)
    if diff:
        rows = _rows_of(diff, S, 8, 17)
        pos, cos, sin = r.numpy()
        s = None if seg is None else seg.numpy()
        sens = np.zeros((len(rows), D))
        out_o, lse_o = oracle.rope3d_attn_fwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                              pos, cos, sin, r.dims, r.interleaved, s,
                                              None if s is None else s.copy(), float(np.float32(scale)),
                                              rows=rows, sens=sens)
        print(check_rows(o1.cpu(), l1.cpu(), rows, out_o, lse_o, valid_rows(seg, seg, B, S), sens), flush=True)


def test_split_graph_replays(need_gpu):
    """A split call (unmasked and masked) captured in a HIP graph and
    replayed three times, with eager calls on the same workspace in between:
    every replay equals the eager call, bit for bit."""
    import spatiotemporal_attention_amd as vdx
    B, S, H, D = 1, 8192, 9, 128
    if n_split_items(B * H * ((S + 255) // 256), persistent_grid()) == 0:
        pytest.skip("no split items on this grid")
    x = W.make_random(B, S, H, D, seed=9100)
    seg = W.random_segments(B, S, 9101, "packed").cuda()
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    for sq in (None, seg):
        sk = None if sq is None else sq.clone()
        ws = torch.empty(vdx.attn_fwd_workspace_size(B, S, H), dtype=torch.uint8, device="cuda")
        ref_o, ref_l = vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, workspace=ws)
        out = torch.empty_like(d["q"])
        lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, out=out, lse=lse, workspace=ws, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        print(f"case split graph capture masked={sq is not None}", flush=True)
        with torch.cuda.graph(g):
            vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, out=out, lse=lse, workspace=ws,
                         stream=torch.cuda.current_stream())
        for i in range(3):
            out.zero_()
            lse.fill_(7.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
            assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))
            vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=0.1, workspace=ws)
            torch.cuda.synchronize()


def test_rope_split_at_720p_equals_composed_split(need_gpu):
    """At the 720p layer's size, in the launch configuration the benchmark
    times with --rope: vdx_rope3d_attn_fwd_ws (work stealing and split items) equals
    vdx_attn_fwd_ws on separately rotated q and k, bit for bit (the same split
    schedule on the same rotated bits)."""
    import spatiotemporal_attention_amd as vdx
    w = W.WORKLOADS["dit720p_large"]
    x = W.make_inputs(w)
    r = W.workload_rope3d(w)
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    rr = dict(pos=r.pos.cuda(), cos=[c.cuda() for c in r.cos], sin=[s.cuda() for s in r.sin], dims=r.dims,
              interleaved=r.interleaved)
    ws = torch.empty(vdx.attn_fwd_workspace_size(w.B, w.S, w.H), dtype=torch.uint8, device="cuda")
    print("case split rope 720p: fused vs composed", flush=True)
    o1, l1 = vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], **rr, scale=w.scale, workspace=ws)
    qr = vdx.rope3d_apply(d["q"], **rr)
    kr = vdx.rope3d_apply(d["k"], **rr)
    o2, l2 = vdx.attn_fwd(qr, kr, d["v"], scale=w.scale, workspace=torch.empty_like(ws))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def _random_split_cases(n=10, seed=2024):
    """Seeded shapes whose item count makes the masked call split items on a
    256-workgroup grid, with random segment kinds."""
    g = np.random.default_rng(seed)
    kinds = [None, "single", "padded", "packed", "interleaved", "singletons", "negative", "extreme"]
    cases = []
    while len(cases) < n:
        B = int(g.integers(1, 4))
        D = int(g.choice([64, 128]))
        S = int(g.integers(700, 6000))
        n_qblk = (S + 255) // 256
        H = int(g.integers(1, 40))
        n_items = B * H * n_qblk
        if n_items > 2000 or n_split_items(n_items, 256) == 0:
            continue
        cases.append((B, S, H, D, kinds[int(g.integers(0, len(kinds)))], int(g.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("B,S,H,D,kind,seed", _random_split_cases())
def test_random_split_shapes(need_gpu, B, S, H, D, kind, seed):
    """Random shapes and segment layouts with split items: the split
    call against vdx_attn_fwd (unsplit blocks bit for bit when unmasked, at
    most the split items' blocks differing when masked, split blocks within
    rounding) and rows of the differing blocks against the oracle."""
    grid = persistent_grid()
    n_items = B * H * ((S + 255) // 256)
    n_split = n_split_items(n_items, grid, masked=kind is not None)
    if n_split == 0:
        pytest.skip(f"{n_items} items on a {grid}-workgroup grid split none")
    x = W.make_random(B, S, H, D, seed=seed % 100000)
    seg = None if kind is None else W.random_segments(B, S, seed % 99991, kind)
    scale = 1.0 / math.sqrt(D)
    print(f"case split random B={B} S={S} H={H} D={D} kind={kind} split={n_split}", flush=True)
    o1, l1 = _run(x, seg, None if seg is None else seg.clone(), scale, split=True)
    o2, l2 = _run(x, seg, None if seg is None else seg.clone(), scale, split=False)
    diff = differing_blocks(o1, l1, o2, l2)
    assert len(diff) <= n_split, (len(diff), n_split)
    if seg is None:
        assert set(diff) <= set(split_unmasked_blocks(B, S, H, grid))
    assert_split_close(o1, l1, o2, l2)
    if diff:
        print(_check_against_oracle(x, seg, seg, scale, o1, l1, diff[:12], 6, seed % 1000), flush=True)
