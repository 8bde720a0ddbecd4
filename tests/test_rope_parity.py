"""GPU parity of the 3D rotary position embedding (vdx_rope3d_apply and the
fused vdx_rope3d_attn_fwd, through the C ABI) against the oracle on the same
seeded inputs.

  * vdx_rope3d_apply equals the oracle's rotation bit for bit on every
    element (both compute each feature in fp64 with one rounding of exact
    products, then round once to bf16), for both pairings, several head-dim
    splits, tokens outside the tables, and in place;
  * vdx_rope3d_attn_fwd equals vdx_attn_fwd on separately rotated q and k bit
    for bit (the queries are rotated in the kernel's prologue, the keys by the
    pre-pass), at small sizes and at the full 720p-layer and packed-clips
    sizes, and with zero angles equals vdx_attn_fwd on the raw inputs;
  * element by element against the oracle (rotation, then attention) on
    shape / segment sweeps, and on sampled rows at full size, to the bar of
    the forward (tests/gpu_helpers.py).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (assert_split_close, check_full, check_rows, differing_blocks, n_split_items,
                         persistent_grid, sample_rows, valid_rows)

pytestmark = pytest.mark.gpu


def dev_rope(r: W.Rope3D):
    return dict(pos=r.pos.cuda(), cos=[c.cuda() for c in r.cos], sin=[s.cuda() for s in r.sin],
                dims=r.dims, interleaved=r.interleaved)


def random_rope(B, S, D, seed, dims=None, interleaved=True, n=(5, 7, 9), outside=0.1):
    dims = W.ROPE_DIMS[D] if dims is None else dims
    tabs = [W.rope3d_tables(n[a], dims[a]) for a in range(3)]
    return W.Rope3D(pos=W.random_positions(B, S, n, seed, outside), cos=tuple(t[0] for t in tabs),
                    sin=tuple(t[1] for t in tabs), dims=tuple(dims), interleaved=interleaved)


def oracle_rotate(x, r: W.Rope3D):
    pos, cos, sin = r.numpy()
    return oracle.rope3d(W.bf16_bits(x), pos, cos, sin, r.dims, r.interleaved)[0]


def bits_of(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# --- the rotation alone -----------------------------------------------------------------------
@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("D,dims", [(128, (44, 42, 42)), (128, (0, 64, 64)), (128, (32, 32, 30)),
                                    (64, (20, 22, 22)), (64, (2, 0, 60)), (64, (0, 0, 0))])
def test_apply_bit_exact(need_gpu, interleaved, D, dims):
    B, S, H = 2, 97, 3
    x = W.randn_bf16((B, S, H, D), 100 + D + sum(dims))
    r = random_rope(B, S, D, 101 + sum(dims), dims, interleaved)
    print(f"case rope apply D={D} dims={dims} interleaved={interleaved}", flush=True)
    import spatiotemporal_attention_amd as vdx
    d = dev_rope(r)
    y = vdx.rope3d_apply(x.cuda(), **d)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(y), oracle_rotate(x, r))


def test_apply_in_place_and_large_values(need_gpu):
    """In place (y = x), and N(0, 3^2) values with the workload's tables."""
    import spatiotemporal_attention_amd as vdx
    w = W.WORKLOADS["packed_clips"]
    B, S, H, D = 1, 4096 + 300, 2, 128
    x = W.randn_bf16((B, S, H, D), 105, sigma=3.0)
    r = W.make_rope3d(B, S, D, W.ROPE_GRIDS[w.name][:1] + [(4096, (1, 10, 30))], interleaved=False)
    print("case rope apply in place", flush=True)
    xd = x.cuda()
    d = dev_rope(r)
    y = vdx.rope3d_apply(xd, **d, out=xd)
    torch.cuda.synchronize()
    assert y.data_ptr() == xd.data_ptr()
    assert np.array_equal(bits_of(xd), oracle_rotate(x, r))


def test_zero_angles_are_identity_and_plain_attention(need_gpu):
    import spatiotemporal_attention_amd as vdx
    B, S, H, D = 1, 700, 2, 128
    x = W.make_random(B, S, H, D, seed=107)
    n, dims = (3, 4, 5), W.ROPE_DIMS[D]
    pos = W.random_positions(B, S, n, 108).cuda()
    cos = [torch.ones(n[a], dims[a] // 2, device="cuda") for a in range(3)]
    sin = [torch.zeros(n[a], dims[a] // 2, device="cuda") for a in range(3)]
    seg = W.random_segments(B, S, 109, "packed").cuda()
    d = {k_: x[k_].cuda() for k_ in ("q", "k", "v")}
    print("case rope zero angles", flush=True)
    y = vdx.rope3d_apply(d["k"], pos, cos, sin, dims)
    o1, l1 = vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], pos, cos, sin, dims, seg_q=seg, seg_kv=seg)
    o2, l2 = vdx.attn_fwd(d["q"], d["k"], d["v"], seg, seg)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), d["k"].view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


# --- fused attention ----------------------------------------------------------------------------
def fused_and_composed(x, r, seg, scale):
    import spatiotemporal_attention_amd as vdx
    d = {k_: x[k_].cuda() for k_ in ("q", "k", "v")}
    sd = None if seg is None else seg.cuda()
    rr = dev_rope(r)
    o1, l1 = vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], **rr, seg_q=sd, seg_kv=sd, scale=scale)
    qr = vdx.rope3d_apply(d["q"], **rr)
    kr = vdx.rope3d_apply(d["k"], **rr)
    o2, l2 = vdx.attn_fwd(qr, kr, d["v"], sd, sd, scale=scale)
    torch.cuda.synchronize()
    return (o1.cpu(), l1.cpu()), (o2.cpu(), l2.cpu())


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 65, 257, 1000])
@pytest.mark.parametrize("kind", [None, "packed", "padded", "negative"], ids=str)
def test_fused_sweep(need_gpu, interleaved, D, S, kind):
    B, H = (2, 2) if S <= 257 else (1, 2)
    x = W.make_random(B, S, H, D, seed=200 * S + D)
    r = random_rope(B, S, D, 201 * S + D, interleaved=interleaved)
    seg = None if kind is None else W.random_segments(B, S, 202 * S + D, kind)
    scale = 1.0 / math.sqrt(D)
    print(f"case rope fused B={B} S={S} H={H} D={D} kind={kind} interleaved={interleaved}", flush=True)
    (o1, l1), (o2, l2) = fused_and_composed(x, r, seg, scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    pos, cos, sin = r.numpy()
    s = None if seg is None else seg.numpy()
    sens = np.zeros((B, S, H, D))
    out_o, lse_o = oracle.rope3d_attn_fwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                          pos, cos, sin, r.dims, r.interleaved, s,
                                          None if s is None else s.copy(), float(np.float32(scale)),
                                          sens=sens)
    check_full(o1, l1, out_o, lse_o, valid_rows(seg, seg, B, S), sens)


def test_fused_k_rot_in_place(need_gpu):
    import spatiotemporal_attention_amd as vdx
    B, S, H, D = 1, 1500, 2, 128
    x = W.make_random(B, S, H, D, seed=211)
    r = random_rope(B, S, D, 212)
    d = {k_: x[k_].cuda() for k_ in ("q", "k", "v")}
    rr = dev_rope(r)
    print("case rope fused k_rot = k", flush=True)
    o1, l1 = vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], **rr)
    k2 = d["k"].clone()
    o2, l2 = vdx.rope3d_attn_fwd(d["q"], k2, d["v"], **rr, k_rot=k2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert np.array_equal(bits_of(k2), oracle_rotate(x["k"], r))


@pytest.mark.parametrize("name", ["dit720p_large", "packed_clips", "joint_video_text_pad"])
def test_full_size_fused_equals_composed_and_sampled_rows(need_gpu, name):
    """At the workload's full size, in the launch configuration the benchmark
    times: fused == composed bit for bit; sampled rows of a few heads against
    the oracle (rotation, then attention)."""
    w = W.WORKLOADS[name]
    print(f"case {name}: rope fused full size", flush=True)
    x = W.make_inputs(w)
    r = W.workload_rope3d(w)
    seg = x["seg_q"]
    (o1, l1), (o2, l2) = fused_and_composed(x, r, seg, w.scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    heads = [0, w.H // 2, w.H - 1]
    sub = {k_: x[k_][:, :, heads].contiguous() for k_ in ("q", "k", "v")}
    rows = sample_rows(w.S, len(heads), w.B, w.seg_runs, n_random=32, seed=3)
    print(f"case {name}: oracle on {len(rows)} rows", flush=True)
    pos, cos, sin = r.numpy()
    s = None if seg is None else seg.numpy()
    sens = np.zeros((len(rows), w.D))
    out_o, lse_o = oracle.rope3d_attn_fwd(W.bf16_bits(sub["q"]), W.bf16_bits(sub["k"]), W.bf16_bits(sub["v"]),
                                          pos, cos, sin, r.dims, r.interleaved, s,
                                          None if s is None else s.copy(), float(np.float32(w.scale)),
                                          rows=rows, sens=sens)
    og = o1[:, :, heads].contiguous()
    lg = l1[:, heads].contiguous()
    st = check_rows(og, lg, rows, out_o, lse_o, valid_rows(seg, seg, w.B, w.S), sens)
    print(name, st, flush=True)


# --- the scheduled masked path (vdx_rope3d_attn_fwd_ws) ------------------------------------------
def fused_both_schedules(x, r, seg, scale):
    """The scheduled call against the one-workgroup-per-block call: the same
    bits on every block the schedule does not split (none when the launch
    has no more items than workgroups); at most the split items' blocks
    differ, within the rounding of their parts."""
    import spatiotemporal_attention_amd as vdx
    d = {k_: x[k_].cuda() for k_ in ("q", "k", "v")}
    sd = seg.cuda()
    rr = dev_rope(r)
    o1, l1 = vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], **rr, seg_q=sd, seg_kv=sd, scale=scale)
    o2, l2 = vdx.rope3d_attn_fwd(d["q"], d["k"], d["v"], **rr, seg_q=sd, seg_kv=sd, scale=scale, scheduled=False)
    torch.cuda.synchronize()
    B, S, H, _ = x["q"].shape
    n_split = n_split_items(B * H * ((S + 255) // 256), persistent_grid())
    if n_split == 0:
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    else:
        diff = differing_blocks(o1, l1, o2, l2)
        assert len(diff) <= n_split, (len(diff), n_split)
        assert_split_close(o1, l1, o2, l2)


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["packed", "padded", "negative", "interleaved"])
def test_fused_scheduled_equals_plain(need_gpu, kind, D, interleaved):
    """vdx_rope3d_attn_fwd_ws (persistent, longest-first) and vdx_rope3d_attn_fwd
    (one workgroup per block) give the same bits."""
    B, S, H = 2, 2100, 2
    x = W.make_random(B, S, H, D, seed=400 + D)
    r = random_rope(B, S, D, 401 + D, interleaved=interleaved)
    seg = W.random_segments(B, S, 402 + D, kind)
    print(f"case rope scheduled B={B} S={S} H={H} D={D} kind={kind} interleaved={interleaved}", flush=True)
    fused_both_schedules(x, r, seg, 1.0 / math.sqrt(D))


def test_full_size_packed_clips_scheduled_equals_plain(need_gpu):
    """Packed clips at full size (3,840 items, a pool of 512 whose last 64 are
    split): the rotary scheduled call against the one-workgroup-per-block
    call, split-aware."""
    w = W.WORKLOADS["packed_clips"]
    print("case packed_clips: rope scheduled vs plain, full size", flush=True)
    x = W.make_inputs(w)
    fused_both_schedules(x, W.workload_rope3d(w), x["seg_q"], w.scale)
