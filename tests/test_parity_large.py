"""GPU parity at the full workload shapes (480p small-DiT layer, joint
video+text with padding, 720p large-DiT layer, packed clips), in the launch
configuration the benchmark times.

The oracle evaluates sampled rows one by one (row 0, 1, S-1, tile edges,
segment boundaries, pad rows and seeded random rows for every head); closed
forms check every row at full size: with Q = 0 each valid row is the mean of
V over its segment with lse = ln(segment size), pad rows are zero / -inf;
with every token its own segment out = V bit for bit and lse = scale q.k;
with V constant over the tokens every valid row returns that constant.
Masked calls also run at the largest sequence the on-chip tile list allows.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import OUT_ATOL, LSE_ATOL, check_rows, run_oracle, sample_rows, valid_rows

pytestmark = pytest.mark.gpu

LARGE = ["dit480p_small", "joint_video_text_pad", "dit720p_large", "packed_clips"]


def _run(d, w, seg=True):
    import spatiotemporal_attention_amd as vdx
    out, lse = vdx.attn_fwd(d["q"], d["k"], d["v"], d.get("seg_q") if seg else None,
                            d.get("seg_kv") if seg else None, scale=w.scale)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name", LARGE)
def test_sampled_rows_vs_oracle(need_gpu, name):
    w = W.WORKLOADS[name]
    print(f"case {name}: generating inputs", flush=True)
    x = W.make_inputs(w)
    d = {n: (None if t is None else t.cuda()) for n, t in x.items()}
    print(f"case {name}: gpu run B={w.B} S={w.S} H={w.H} D={w.D}", flush=True)
    out, lse = _run(d, w)
    out_c, lse_c = out.cpu(), lse.cpu()
    del d, out, lse
    heads = list(range(w.H)) if w.H <= 16 else list(range(0, w.H, 3))
    rows = sample_rows(w.S, w.H, w.B, w.seg_runs, n_random=48, seed=1, heads=heads)
    print(f"case {name}: oracle on {len(rows)} rows", flush=True)
    out_o, lse_o, sens_o = run_oracle(x, x["seg_q"], x["seg_kv"], w.scale, rows=rows)
    has = valid_rows(x["seg_q"], x["seg_kv"], w.B, w.S)
    st = check_rows(out_c, lse_c, rows, out_o, lse_o, has, sens_o)
    print(name, st, flush=True)


@pytest.mark.parametrize("name", LARGE)
def test_zero_query_closed_form_every_row(need_gpu, name):
    w = W.WORKLOADS[name]
    print(f"case {name}: Q=0 closed form", flush=True)
    x = W.make_inputs(w)
    x["q"].zero_()
    d = {n: (None if t is None else t.cuda()) for n, t in x.items()}
    out, lse = _run(d, w)
    del d
    runs = w.seg_runs if w.seg_runs is not None else [(0, w.S, 1)]
    # Group the runs by segment ID: runs sharing an ID form one segment.
    by_id = {}
    for a, e, sid in runs:
        by_id.setdefault(sid, []).append((a, e))
    v = x["v"]
    for b in range(w.B):
        for sid, spans in by_id.items():
            n_tok = sum(e - a for a, e in spans)
            for h in range(w.H):
                if sid == 0:
                    for a, e in spans:
                        assert np.all(out[b, a:e, h].view(torch.int16).cpu().numpy() == 0)
                        assert np.all(np.isneginf(lse[b, h, a:e].cpu().numpy()))
                    continue
                mean = sum(v[b, a:e, h].double().sum(0) for a, e in spans).numpy() / n_tok
                for a, e in spans:
                    o = out[b, a:e, h].float().cpu().numpy()
                    l = lse[b, h, a:e].cpu().numpy()
                    err = np.abs(o - mean[None]).max()
                    assert err <= OUT_ATOL, (b, a, e, h, err)
                    # bf16 rounding of the mean itself is the dominant error here
                    assert err <= np.abs(mean).max() * 2.0 ** -8 + 1e-6, (b, a, e, h, err)
                    assert np.abs(l - math.log(n_tok)).max() <= LSE_ATOL
    del out, lse


# The largest sequence a masked call accepts: the on-chip active-tile list
# holds 30,720 key tiles of 64 (S = 1,966,080).  Key tile t carries ID 1 on its
# first token and the tile-unique ID 2 + t on the others; the last 5 tokens are
# padding on both sides.  Query block 0 (tokens 0..255) has ID 1, so every key
# tile is active (and partial) for it and its list is full; any other query
# has the tile-unique ID of its own tile and attends the 63 other keys there.
# The ragged case ends in a partly filled last tile, still 30,720 tiles.
@pytest.mark.parametrize("S,D", [(1_966_080, 128), (1_966_063, 64)])
def test_masked_maximum_sequence(need_gpu, S, D):
    import spatiotemporal_attention_amd as vdx
    B, H = 1, 1
    assert (S + 63) // 64 == 30_720
    tok = torch.arange(S, dtype=torch.int64)
    seg_kv = torch.where(tok % 64 == 0, 1, 2 + tok // 64).to(torch.int32)
    seg_q = torch.where(tok < 256, 1, 2 + tok // 64).to(torch.int32)
    seg_kv[S - 5:] = 0
    seg_q[S - 5:] = 0
    seg_q, seg_kv = seg_q[None].contiguous(), seg_kv[None].contiguous()
    print(f"case masked max S={S} D={D}: generating inputs", flush=True)
    x = W.make_random(B, S, H, D, seed=S % 100_000)
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    print(f"case masked max S={S} D={D}: gpu run", flush=True)
    out, lse = vdx.attn_fwd(d["q"], d["k"], d["v"], seg_q.cuda(), seg_kv.cuda(),
                            scale=1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    out_c, lse_c = out.cpu(), lse.cpu()
    del d, out, lse
    rows = sample_rows(S, H, B, None, n_random=48, seed=3)
    extra = [(0, 0, i) for i in (2, 63, 64, 100, 200, 254, 255, 256, 257)]
    rows = np.unique(np.concatenate([rows, np.array(extra, dtype=np.int64)]), axis=0)
    print(f"case masked max S={S} D={D}: oracle on {len(rows)} rows", flush=True)
    out_o, lse_o, sens_o = run_oracle(x, seg_q, seg_kv, 1.0 / math.sqrt(D), rows=rows)
    has = valid_rows(seg_q, seg_kv, B, S)
    assert has[0, :256].all() and not has[0, S - 5:].any()
    st = check_rows(out_c, lse_c, rows, out_o, lse_o, has, sens_o)
    print(st, flush=True)
    # Every padded row is +0.0 / -inf, every other output is finite.
    assert np.all(out_c[0, S - 5:].view(torch.int16).numpy() == 0)
    assert np.all(np.isneginf(lse_c[0, 0, S - 5:].numpy()))
    assert torch.isfinite(out_c[0, :S - 5].float()).all()
    assert torch.isfinite(lse_c[0, 0, :S - 5]).all()


@pytest.mark.parametrize("name", LARGE)
def test_distinct_ids_return_value_every_row(need_gpu, name):
    """Every token its own segment (IDs 1..S): a row's only valid key is
    itself, so P = 2^0 = 1 exactly and out = v bit for bit, lse = scale q.k."""
    import spatiotemporal_attention_amd as vdx
    w = W.WORKLOADS[name]
    print(f"case {name}: distinct IDs", flush=True)
    x = W.make_inputs(w)
    seg = torch.arange(1, w.S + 1, dtype=torch.int32).repeat(w.B, 1).contiguous()
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    out, lse = vdx.attn_fwd(d["q"], d["k"], d["v"], seg.cuda(), seg.cuda(), scale=w.scale)
    torch.cuda.synchronize()
    del d
    assert torch.equal(out.cpu().view(torch.int16), x["v"].view(torch.int16))
    scale = float(np.float32(w.scale))
    for b in range(w.B):
        s_ii = (x["q"][b].double() * x["k"][b].double()).sum(-1).numpy() * scale  # [S, H]
        err = np.abs(lse[b].cpu().numpy().T.astype(np.float64) - s_ii).max()
        assert err <= LSE_ATOL, (b, err)


@pytest.mark.parametrize("name", LARGE)
def test_constant_value_every_row(need_gpu, name):
    """V[b, j, h, :] = c_h for every token: each valid row's output is c_h
    (its probabilities sum to 1).  The GPU weights c by the bf16-rounded
    probabilities but divides by their unrounded fp32 sum, a ratio within
    u = 2^-8 of 1 (each term rounds by at most u relative), and rounds the
    output once more by u: |out - c| <= 2u |c|, plus 1e-4 |c| for the fp32
    sums.  Padding rows stay +0.0."""
    import spatiotemporal_attention_amd as vdx
    w = W.WORKLOADS[name]
    print(f"case {name}: constant V", flush=True)
    x = W.make_inputs(w)
    c = W.randn_bf16((w.H, w.D), 4242)
    x["v"] = c[None, None].expand(w.B, w.S, w.H, w.D).contiguous()
    d = {n: (None if t is None else t.cuda()) for n, t in x.items()}
    out, _ = _run(d, w)
    del d
    o = out.float().cpu().numpy()
    has = valid_rows(x["seg_q"], x["seg_kv"], w.B, w.S)
    cc = c.double().numpy()[None]
    err = np.abs(o[has] - cc)
    assert np.all(err <= (2 * 2.0 ** -8 + 1e-4) * np.abs(cc) + 1e-6), float(err.max())
    if (~has).any():
        assert np.all(out.cpu().view(torch.int16).numpy()[~has] == 0)


# Bit canaries at the 480p layer's size (B=1, S=32,760, H=12): 1,536 query
# blocks, so the unmasked call's persistent grid of 256 workgroups runs six
# items per workgroup (reusing its LDS and registers after each), while the
# masked call through vdx_attn_fwd runs one workgroup per item and a one-head
# call 128 items on 128 workgroups.  Every route must give the same bits (the
# scheduled masked route splits some items; test_fwd_sched.py covers it).
def test_full_size_bit_canaries(need_gpu):
    import spatiotemporal_attention_amd as vdx
    w = W.WORKLOADS["dit480p_small"]
    print(f"case {w.name}: bit canaries (repeat, all-ones IDs, head split)", flush=True)
    x = W.make_inputs(w)
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    a_out, a_lse = vdx.attn_fwd(d["q"], d["k"], d["v"], scale=w.scale)
    b_out, b_lse = vdx.attn_fwd(d["q"], d["k"], d["v"], scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16)), "repeat run"
    assert torch.equal(a_lse.view(torch.int32), b_lse.view(torch.int32)), "repeat run"
    del b_out, b_lse
    ones = torch.ones(w.B, w.S, dtype=torch.int32, device="cuda")
    c_out, c_lse = vdx.attn_fwd(d["q"], d["k"], d["v"], ones, ones.clone(), scale=w.scale, scheduled=False)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.int16), c_out.view(torch.int16)), "NULL vs all-ones IDs"
    assert torch.equal(a_lse.view(torch.int32), c_lse.view(torch.int32)), "NULL vs all-ones IDs"
    del c_out, c_lse
    for h in (0, 5, w.H - 1):
        dh = {n: d[n][:, :, h:h + 1].contiguous() for n in ("q", "k", "v")}
        o1, l1 = vdx.attn_fwd(dh["q"], dh["k"], dh["v"], scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), a_out[:, :, h:h + 1].contiguous().view(torch.int16)), h
        assert torch.equal(l1.view(torch.int32), a_lse[:, h:h + 1].contiguous().view(torch.int32)), h
