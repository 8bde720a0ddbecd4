"""GPU parity of the attention gradient (vdx_attn_bwd through the C ABI)
against the fp64 oracle on the same seeded bf16 inputs.

The GPU backward takes the GPU forward's out and lse, as in training; the
oracle recomputes everything from q, k, v in fp64, so the comparison covers
the forward's rounding too.  Small and moderate sequences are compared
element by element over shapes spanning several 64-row tiles and 128-row
workgroups with ragged tails, every segment layout of the forward sweep, and
D = 64 / 128.  The 720p DiT shape (B=1, S=75,600, H=40, D=128) is compared on
sampled dq rows and, on every row, against the closed forms of q = 0 and
k = 0; the packed-clips shape (S=61,440, H=16) on a whole clip computed by
the oracle as its own sequence (clips are independent) and on sampled dq rows;
the padded joint video+text shape (B=2, S=17,920, H=24) on sampled dq rows
of both batch rows and, with k = 0, every dk and dv row against the closed
form over its valid tokens.

Tolerances for a gradient g (bf16) against the oracle o (fp64):
  |g - o| <= 2 * BF16_U * t + BF16_U * |o| + G_ATOL    element by element
  ||g - o|| <= G_REL_L2 * ||o|| + G_ATOL * sqrt(n)     per tensor
t is the oracle's rounding-sensitivity sum of the element: the sum of the
absolute values of the terms it adds up, tq = scale sum_j (|dS_ij| + P_ij E_i)
|k_j|, tk = scale sum_i (|dS_ij| + P_ij E_i) |q_i|, tv = sum_i P_ij |dout_i|,
with E_i = sum_j P_ij |dout_i| . |v_j|.  The GPU rounds each dS (dq, dk) or P
(dv) term once to bf16 (relative error <= BF16_U = 2^-8: at most BF16_U * t),
and delta comes from the bf16 forward output, whose terms carry one bf16
rounding each plus the final one (|delta error| <= 2 BF16_U E_i, at most
BF16_U * t once more); BF16_U * |o| is the final rounding of the gradient.
Everything else (fp32 accumulation and exp2, the fp32 lse) is below 1e-6
relative.  G_ATOL = 1e-5 absorbs fp32 cancellation where the exact gradient
is 0 (one-token segments).  The element bound is worst case; the relative L2
gate is the statistical one: independent roundings give about
sqrt(3) * 2^-8/sqrt(3) = 0.004 (G_REL_L2 = 1e-2, as for the forward output).

Where the oracle cannot give t (the q = 0 / k = 0 closed forms at full size,
whose O(S^2 D) sums are out of reach), every gradient row is a sum over all S
keys or queries of random-sign terms, so its RMS over the head dim is the
error scale: |g - o| <= G_MAX_RMS * rms_row(o) + BF16_U * |o| + G_ATOL with
G_MAX_RMS = 0.05 (~6 sigma of a 2^-8/sqrt(3) relative error is 0.014).
Rows without a valid key must give dq exactly 0, and keys no query attends
dk = dv = 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import BF16_U, valid_rows

pytestmark = pytest.mark.gpu

G_MAX_RMS = 5e-2
G_REL_L2 = 1e-2
G_ATOL = 1e-5


def run_gpu_bwd(x, dout, seg_q=None, seg_kv=None, scale=None):
    import spatiotemporal_attention_amd as vdx
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    sq = None if seg_q is None else seg_q.cuda()
    sk = None if seg_kv is None else seg_kv.cuda()
    out, lse = vdx.attn_fwd(d["q"], d["k"], d["v"], sq, sk, scale=scale)
    dq, dk, dv = vdx.attn_bwd(d["q"], d["k"], d["v"], out, lse, dout.cuda(), sq, sk, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def run_oracle_bwd(x, dout, seg_q=None, seg_kv=None, scale=None):
    """(dq, dk, dv, tq, tk, tv) in fp64."""
    D = x["q"].shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    return oracle.attn_bwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                           W.bf16_bits(dout), None if seg_q is None else seg_q.numpy(),
                           None if seg_kv is None else seg_kv.numpy(), float(np.float32(scale)),
                           sensitivity=True)


def check_grad(name, g, o, zero=None, t=None):
    """g: bf16 tensor, o: fp64 array of the same [.., D] shape, t: its
    rounding-sensitivity sums (None: the row-RMS rule); zero: bool mask over
    the leading dims where g must be exactly 0."""
    gg = g.float().numpy().astype(np.float64)
    stats = {"name": name, "max_abs": 0.0, "rel_l2": 0.0, "max_tol_frac": 0.0}
    keep = np.ones(gg.shape[:-1], dtype=bool) if zero is None else ~zero
    if keep.any():
        a, b = gg[keep], o[keep]
        err = np.abs(a - b)
        if t is not None:
            tol = 2 * BF16_U * t[keep] + BF16_U * np.abs(b) + G_ATOL
        else:
            rms_row = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
            tol = G_MAX_RMS * rms_row + BF16_U * np.abs(b) + G_ATOL
        stats["max_abs"] = float(err.max())
        stats["max_tol_frac"] = float((err / tol).max())
        nrm = float(np.linalg.norm(b))
        stats["rel_l2"] = float(np.linalg.norm(a - b) / max(nrm, 1e-300))
        assert stats["max_tol_frac"] <= 1.0, stats
        assert np.linalg.norm(a - b) <= G_REL_L2 * nrm + G_ATOL * math.sqrt(a.size), stats
    if zero is not None and zero.any():
        assert np.all(gg[zero] == 0.0), f"{name}: rows without a valid pair must be 0"
    return stats


def masks(seg_q, seg_kv, B, S, H):
    """[B, S, H] bool: query rows without a valid key, keys without a valid query."""
    if seg_q is None:
        return None, None
    q_dead = ~valid_rows(seg_q, seg_kv, B, S)
    k_dead = ~valid_rows(seg_kv, seg_q, B, S)
    rep = lambda m: np.repeat(m[:, :, None], H, axis=2)
    return rep(q_dead), rep(k_dead)


def compare_all(x, dout, seg_q, seg_kv, scale):
    B, S, H, D = x["q"].shape
    g = run_gpu_bwd(x, dout, seg_q, seg_kv, scale)
    o = run_oracle_bwd(x, dout, seg_q, seg_kv, scale)
    qd, kd = masks(seg_q, seg_kv, B, S, H)
    return [check_grad(n, gi, oi, z, ti) for n, gi, oi, z, ti in
            zip(("dq", "dk", "dv"), g, o[:3], (qd, kd, kd), o[3:])]


SEQS = [1, 2, 63, 64, 65, 127, 128, 129, 255, 257, 1000]
KINDS = [None, "single", "padded", "packed", "interleaved", "singletons", "allpad", "negative",
         "extreme"]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", SEQS)
@pytest.mark.parametrize("kind", KINDS, ids=[str(k) for k in KINDS])
def test_shape_and_segment_sweep(need_gpu, S, D, kind):
    B, H = (2, 2) if S <= 257 else (1, 2)
    x = W.make_random(B, S, H, D, seed=300 * S + D)
    dout = W.randn_bf16((B, S, H, D), 300 * S + D + 7)
    seg = None if kind is None else W.random_segments(B, S, 300 * S + 11, kind)
    print(f"case bwd sweep B={B} S={S} H={H} D={D} kind={kind}", flush=True)
    print(compare_all(x, dout, seg, None if seg is None else seg.clone(), 1.0 / math.sqrt(D)))


@pytest.mark.parametrize("kind", [None, "packed", "interleaved"], ids=str)
def test_long_ragged_sequence(need_gpu, kind):
    B, S, H, D = 1, 2049, 1, 128
    x = W.make_random(B, S, H, D, seed=2049, sigma_qk=2.0)
    dout = W.randn_bf16((B, S, H, D), 2050)
    seg = None if kind is None else W.random_segments(B, S, 2051, kind)
    print(f"case bwd long S={S} kind={kind}", flush=True)
    print(compare_all(x, dout, seg, None if seg is None else seg.clone(), 1.0 / math.sqrt(D)))


def test_distinct_query_and_key_segments(need_gpu):
    """seg_q and seg_kv differ: query IDs missing from seg_kv give dead rows,
    key IDs missing from seg_q give dead keys."""
    B, S, H, D = 2, 300, 2, 64
    x = W.make_random(B, S, H, D, seed=377)
    dout = W.randn_bf16((B, S, H, D), 378)
    seg_q = W.random_segments(B, S, 5, "interleaved")
    seg_kv = W.random_segments(B, S, 6, "interleaved")
    seg_kv[seg_kv == 3] = 2   # ID 3 only among the queries
    seg_q[seg_q == 1] = 2     # ID 1 only among the keys
    print("case bwd distinct segs", flush=True)
    compare_all(x, dout, seg_q, seg_kv, 0.125)


def test_peaky_scores(need_gpu):
    B, S, H, D = 1, 1000, 2, 128
    x = W.make_random(B, S, H, D, seed=559, sigma_qk=3.0)
    dout = W.randn_bf16((B, S, H, D), 560)
    print("case bwd peaky", flush=True)
    print(compare_all(x, dout, None, None, 1.0 / math.sqrt(D)))


def test_repeat_and_head_split_bit_identical(need_gpu):
    B, S, H, D = 2, 700, 3, 128
    x = W.make_random(B, S, H, D, seed=991)
    dout = W.randn_bf16((B, S, H, D), 992)
    seg = W.random_segments(B, S, 993, "packed")
    a = run_gpu_bwd(x, dout, seg, seg.clone(), 0.1)
    b = run_gpu_bwd(x, dout, seg, seg.clone(), 0.1)
    for u, w in zip(a, b):
        assert torch.equal(u.view(torch.int16), w.view(torch.int16))
    xs = {n: t[1:2, :, 2:3].contiguous() for n, t in x.items()}
    c = run_gpu_bwd(xs, dout[1:2, :, 2:3].contiguous(), seg[1:2].contiguous(), seg[1:2].clone(), 0.1)
    for u, w in zip(c, a):
        assert torch.equal(u.view(torch.int16), w[1:2, :, 2:3].contiguous().view(torch.int16))


# ---- full-size shapes -----------------------------------------------------------------

def _dq_rows_check(x, dout, seg, scale, dq_g, heads, n_rows, seed):
    B, S, H, D = x["q"].shape
    rng = np.random.default_rng(seed)
    idx = sorted({0, 1, 127, 128, S - 1} | set(int(i) for i in rng.choice(S, n_rows, replace=False)))
    rows = np.array([(0, h, i) for h in heads for i in idx], dtype=np.int64)
    s = None if seg is None else seg.numpy()
    o, t = oracle.attn_bwd_dq_rows(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                   W.bf16_bits(dout), s, None if s is None else s.copy(),
                                   float(np.float32(scale)), rows, sensitivity=True)
    g = dq_g[rows[:, 0], rows[:, 2], rows[:, 1]]
    dead = None
    if seg is not None:
        dead = ~valid_rows(seg, seg, B, S)[rows[:, 0], rows[:, 2]]
    return check_grad("dq rows", g, o, dead, t)


def test_dit720p_sampled_dq_rows(need_gpu):
    w = W.WORKLOADS["dit720p_large"]
    x = W.make_inputs(w)
    dout = W.randn_bf16((w.B, w.S, w.H, w.D), 4003)
    print(f"case {w.name}: bwd sampled dq rows", flush=True)
    dq, _, _ = run_gpu_bwd(x, dout, None, None, w.scale)
    print(_dq_rows_check(x, dout, None, w.scale, dq, heads=(0, 17, 39), n_rows=24, seed=1))


def _closed_form_head(x, dout, scale, which, h):
    """q = 0 (which='q') or k = 0 (which='k'): P uniform over all S keys.
    Returns the fp64 closed form of the non-zero gradient of head h (dq for
    q = 0, dk for k = 0; the other of dq, dk is exactly 0) and dv (every key:
    the mean of dout over the queries).
      q = 0: dq_i = scale * M dout_i with M = sum_j k_j (v_j - vbar)^T / S
      k = 0: dk_j = scale * N (v_j - vbar) with N = sum_i q_i dout_i^T / S"""
    S = x["q"].shape[1]
    v = x["v"][0, :, h].double().numpy()
    do = dout[0, :, h].double().numpy()
    vc = v - v.mean(0)
    if which == "q":
        k = x["k"][0, :, h].double().numpy()
        g = scale * do @ (k.T @ vc / S).T
    else:
        q = x["q"][0, :, h].double().numpy()
        g = scale * vc @ (q.T @ do / S).T
    dv = np.broadcast_to(do.mean(0), do.shape)
    return g, dv


@pytest.mark.parametrize("which", ["q", "k"])
def test_dit720p_uniform_closed_forms_every_row(need_gpu, which):
    w = W.WORKLOADS["dit720p_large"]
    x = W.make_inputs(w)
    x[which] = torch.zeros_like(x[which])
    dout = W.randn_bf16((w.B, w.S, w.H, w.D), 4004)
    print(f"case {w.name}: bwd {which}=0 closed form", flush=True)
    dq, dk, dv = run_gpu_bwd(x, dout, None, None, w.scale)
    nonzero, zero = (dq, dk) if which == "q" else (dk, dq)
    assert torch.count_nonzero(zero.float()) == 0, f"{'dk' if which == 'q' else 'dq'} must be exactly 0"
    scale = float(np.float32(w.scale))
    for h in range(w.H):
        g, gv = _closed_form_head(x, dout, scale, which, h)
        check_grad("dq" if which == "q" else "dk", nonzero[0, :, h], g)
        check_grad("dv", dv[0, :, h], gv)
        if h % 8 == 7:
            print(f"  heads 0..{h} ok", flush=True)


def test_packed_clips_whole_clip_and_sampled_rows(need_gpu):
    w = W.WORKLOADS["packed_clips"]
    x = W.make_inputs(w)
    dout = W.randn_bf16((w.B, w.S, w.H, w.D), 5003)
    seg = x["seg_q"]
    print(f"case {w.name}: bwd whole clip 1 + sampled dq rows", flush=True)
    dq, dk, dv = run_gpu_bwd(x, dout, seg, x["seg_kv"], w.scale)
    # Clip 1 (tokens 0..4095) as its own unmasked sequence, head 5.
    a, b_ = w.seg_runs[0][:2]
    h = 5
    xs = {n: x[n][:, a:b_, h:h + 1].contiguous() for n in ("q", "k", "v")}
    o = run_oracle_bwd(xs, dout[:, a:b_, h:h + 1].contiguous(), None, None, w.scale)
    for n, gi, oi, ti in zip(("dq", "dk", "dv"), (dq, dk, dv), o[:3], o[3:]):
        print(check_grad(n + " clip1", gi[:, a:b_, h:h + 1], oi, None, ti))
    # Pad tokens: no valid pair on either side.
    pad = seg[0] == 0
    for n, gi in zip(("dq", "dk", "dv"), (dq, dk, dv)):
        assert torch.count_nonzero(gi[0, pad].float()) == 0, n
    print(_dq_rows_check(x, dout, seg, w.scale, dq, heads=(0, 15), n_rows=24, seed=2))


def test_joint_video_text_padding_full_size(need_gpu):
    """Joint video+text layer with padding (B=2, S=17,920, H=24, one segment
    of 17,776 tokens and 144 pad tokens in each batch row).  Random inputs:
    dq on sampled rows of both batch rows (pad rows among them) against the
    row oracle, and pad tokens exactly 0 in dq, dk and dv.  Then k = 0, so P
    is uniform over the valid keys: dq must be exactly 0, and every row of dk
    and dv is compared with the closed form over the valid tokens
    (dk_j = scale (sum_i q_i dout_i^T / n)(v_j - vbar), dv_j = mean_i dout_i,
    sums and means over the n valid tokens)."""
    w = W.WORKLOADS["joint_video_text_pad"]
    x = W.make_inputs(w)
    seg = x["seg_q"]
    dout = W.randn_bf16((w.B, w.S, w.H, w.D), 3007)
    print(f"case {w.name}: bwd sampled dq rows, both batch rows", flush=True)
    dq, dk, dv = run_gpu_bwd(x, dout, seg, x["seg_kv"], w.scale)
    rng = np.random.default_rng(3)
    idx = sorted({0, 127, 128, 17549, 17550, 17775, 17776, w.S - 1}
                 | set(int(i) for i in rng.choice(w.S, 16, replace=False)))
    rows = np.array([(b, h, i) for b in range(w.B) for h in (0, 23) for i in idx], dtype=np.int64)
    o, t = oracle.attn_bwd_dq_rows(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                   W.bf16_bits(dout), seg.numpy(), x["seg_kv"].numpy(),
                                   float(np.float32(w.scale)), rows, sensitivity=True)
    dead = ~valid_rows(seg, seg, w.B, w.S)[rows[:, 0], rows[:, 2]]
    assert dead.sum() == 2 * 2 * 2  # rows 17776 and S-1 of both heads and batch rows
    print(check_grad("dq rows", dq[rows[:, 0], rows[:, 2], rows[:, 1]], o, dead, t), flush=True)
    pad = seg[0] == 0
    for n, gi in zip(("dq", "dk", "dv"), (dq, dk, dv)):
        assert torch.count_nonzero(gi[:, pad].float()) == 0, n
        assert torch.isfinite(gi.float()).all(), n

    print(f"case {w.name}: bwd k=0 closed form over the valid tokens", flush=True)
    x["k"] = torch.zeros_like(x["k"])
    dq, dk, dv = run_gpu_bwd(x, dout, seg, x["seg_kv"], w.scale)
    assert torch.count_nonzero(dq.float()) == 0, "dq must be exactly 0"
    scale = float(np.float32(w.scale))
    ok = ~pad
    n = int(ok.sum())
    for b in range(w.B):
        for h in range(w.H):
            q = x["q"][b, ok, h].double().numpy()
            v = x["v"][b, ok, h].double().numpy()
            do = dout[b, ok, h].double().numpy()
            gk = scale * (v - v.mean(0)) @ (q.T @ do / n).T
            gv = np.broadcast_to(do.mean(0), do.shape)
            check_grad("dk", dk[b, ok, h], gk)
            check_grad("dv", dv[b, ok, h], gv)
        print(f"  batch row {b}: {w.H} heads ok", flush=True)
    for n_, gi in zip(("dk", "dv"), (dk, dv)):
        assert torch.count_nonzero(gi[:, pad].float()) == 0, n_


def test_masked_maximum_sequence(need_gpu):
    """The largest sequence a masked backward accepts: 14,000 tiles of 64 in
    its on-chip lists (S = 896,000).  Key tile t carries ID 1 on its first
    token and the tile-unique ID 2 + t on the others; query block 0 (tokens
    0..255) has ID 1 and every other query the tile-unique ID of its tile; the
    last 5 tokens are padding.  So the dQ sweep of query block 0 lists every
    key tile and the dK/dV sweep of the last key block lists every query tile.
    dq is compared on sampled rows (all of block 0 among them) with the row
    oracle; dq, dk and dv of the local segments of the last tiles with the
    oracle run on each tile as its own sequence (segments are independent; a
    tile's first key, ID 1, belongs to block 0's segment and is left out)."""
    B, S, H, D = 1, 896_000, 1, 128
    assert S // 64 == 14_000
    tok = torch.arange(S, dtype=torch.int64)
    seg_kv = torch.where(tok % 64 == 0, 1, 2 + tok // 64).to(torch.int32)
    seg_q = torch.where(tok < 256, 1, 2 + tok // 64).to(torch.int32)
    seg_kv[S - 5:] = 0
    seg_q[S - 5:] = 0
    seg_q, seg_kv = seg_q[None].contiguous(), seg_kv[None].contiguous()
    scale = 1.0 / math.sqrt(D)
    print(f"case bwd masked max S={S}: generating inputs", flush=True)
    x = W.make_random(B, S, H, D, seed=8960)
    dout = W.randn_bf16((B, S, H, D), 8967)
    print(f"case bwd masked max S={S}: gpu run", flush=True)
    dq, dk, dv = run_gpu_bwd(x, dout, seg_q, seg_kv, scale)
    # dq rows: block 0 (every key tile), tile edges, the end, seeded random rows.
    rng = np.random.default_rng(17)
    idx = sorted(set(range(256)) | {256, 257, 319, 320, S - 65, S - 64, S - 6, S - 5, S - 1}
                 | set(int(i) for i in rng.choice(S, 40, replace=False)))
    rows = np.array([(0, 0, i) for i in idx], dtype=np.int64)
    print(f"case bwd masked max S={S}: dq row oracle on {len(rows)} rows", flush=True)
    o, t = oracle.attn_bwd_dq_rows(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                   W.bf16_bits(dout), seg_q.numpy(), seg_kv.numpy(),
                                   float(np.float32(scale)), rows, sensitivity=True)
    dead = ~valid_rows(seg_q, seg_kv, B, S)[rows[:, 0], rows[:, 2]]
    print(check_grad("dq rows", dq[rows[:, 0], rows[:, 2], rows[:, 1]], o, dead, t), flush=True)
    # Local segments of the last 4 tiles, each as its own 64-token sequence.
    for k in range(S // 64 - 4, S // 64):
        a, e = 64 * k, 64 * k + 64
        xs = {n: x[n][:, a:e].contiguous() for n in ("q", "k", "v")}
        sq, sk = seg_q[:, a:e].clone(), seg_kv[:, a:e].clone()
        o = run_oracle_bwd(xs, dout[:, a:e].contiguous(), sq, sk, scale)
        qd, kd = masks(sq, sk, 1, 64, 1)
        check_grad(f"dq tile {k}", dq[:, a:e], o[0], qd, o[3])
        # keys a+1 .. a+63: key a (ID 1) also serves block 0, outside this sub-problem
        for n, gi, oi, ti in (("dk", dk, o[1], o[4]), ("dv", dv, o[2], o[5])):
            check_grad(f"{n} tile {k}", gi[:, a + 1:e], oi[:, 1:], kd[:, 1:], ti[:, 1:])
    pad = slice(S - 5, S)
    for n, gi in zip(("dq", "dk", "dv"), (dq, dk, dv)):
        assert torch.count_nonzero(gi[0, pad].float()) == 0, n
        assert torch.isfinite(gi.float()).all(), n
