"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same bf16 bits, and compare to the tolerances
of the parity bar.

Tolerances (fixed for bf16 output of fp32-accumulated attention):
  OUT_ATOL = 1e-2   max |out_gpu - out_oracle| over compared elements, plus
                    BF16_U * |out_oracle| (BF16_U = 2^-8, the unit roundoff of
                    bf16): rounding the exact value once to bf16 already moves
                    it by up to that much, which exceeds 1e-2 alone once
                    |out| > 2.56 (tiny segments, peaky rows);
  LSE_ATOL = 1e-3   max |lse_gpu - lse_oracle| over rows with a valid key;
  REL_L2   = 1e-2   ||out_gpu - out_oracle|| / ||out_oracle|| per case, an extra
                    gate because the absolute bound is loose at long S (output
                    magnitudes shrink like sqrt(e/S)); bf16 rounding of the output
                    and of the probabilities each contribute about 2^-9 relative.
Fully masked rows must be +0.0 bit for bit with lse == -inf.
"""
import math

import numpy as np
import torch

import oracle
import workloads as W

OUT_ATOL = 1e-2
BF16_U = 2.0 ** -8
LSE_ATOL = 1e-3
REL_L2 = 1e-2


def to_dev(x, seg_q=None, seg_kv=None):
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    d["seg_q"] = None if seg_q is None else seg_q.cuda()
    d["seg_kv"] = None if seg_kv is None else seg_kv.cuda()
    return d


def run_gpu(x, seg_q=None, seg_kv=None, scale=None):
    import spatiotemporal_attention_amd as vdx
    d = to_dev(x, seg_q, seg_kv)
    out, lse = vdx.attn_fwd(d["q"], d["k"], d["v"], d["seg_q"], d["seg_kv"], scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_oracle(x, seg_q=None, seg_kv=None, scale=None, rows=None):
    D = x["q"].shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return oracle.attn_fwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                           None if seg_q is None else seg_q.numpy(),
                           None if seg_kv is None else seg_kv.numpy(), float(np.float32(scale)),
                           rows=rows)[:2]


def valid_rows(seg_q, seg_kv, B, S):
    """bool [B, S]: query i of batch b has at least one valid key."""
    if seg_q is None:
        return np.ones((B, S), dtype=bool)
    out = np.zeros((B, S), dtype=bool)
    for b in range(B):
        kv_ids = set(np.unique(seg_kv[b].numpy()).tolist())
        sq = seg_q[b].numpy()
        out[b] = np.array([(s != 0 and s in kv_ids) for s in sq], dtype=bool)
    return out


def check_full(out_g, lse_g, out_o, lse_o, has):
    """Compare full outputs ([B,S,H,D] / [B,H,S]); returns a stats dict."""
    og = out_g.float().numpy().astype(np.float64)
    lg = lse_g.numpy().astype(np.float64)
    B, S, H, D = og.shape
    stats = {"max_abs": 0.0, "max_lse": 0.0, "rel_l2": 0.0}
    if has.any():
        diff = np.abs(og[has] - out_o[has])
        stats["max_abs"] = float(diff.max())
        stats["max_tol_frac"] = float((diff / (OUT_ATOL + BF16_U * np.abs(out_o[has]))).max())
        ref_n = float(np.linalg.norm(out_o[has]))
        stats["rel_l2"] = float(np.linalg.norm(og[has] - out_o[has]) / max(ref_n, 1e-300))
        lh = np.transpose(lg, (0, 2, 1))[has]
        lo = np.transpose(lse_o, (0, 2, 1))[has]
        stats["max_lse"] = float(np.abs(lh - lo).max())
        assert stats["max_tol_frac"] <= 1.0, stats
        assert stats["max_lse"] <= LSE_ATOL, stats
        assert stats["rel_l2"] <= REL_L2, stats
    if (~has).any():
        bits = out_g.view(torch.int16).numpy()[~has]
        assert np.all(bits == 0), "fully masked rows must be +0.0"
        assert np.all(np.isneginf(np.transpose(lg, (0, 2, 1))[~has])), "masked rows need lse=-inf"
    return stats


def sample_rows(S, H, B, seg_runs=None, n_random=64, tile=64, seed=0, heads=None):
    """(b, h, i) triples: rows 0, 1, S-1; tile edges +-1 of the first and last
    4 tiles (64- and 256-row tiles); segment boundaries +-1; n_random rows."""
    g = np.random.default_rng(seed)
    cand = {0, 1, S - 1}
    for t in (64, 256):
        nt = (S + t - 1) // t
        for k in list(range(min(4, nt))) + list(range(max(0, nt - 4), nt)):
            for off in (-1, 0, 1, t - 1, t):
                cand.add(k * t + off)
    if seg_runs:
        for a, b_, _ in seg_runs:
            for off in (-1, 0, 1):
                cand.add(a + off)
                cand.add(b_ - 1 + off)
    cand = sorted(i for i in cand if 0 <= i < S)
    rows = []
    hs = range(H) if heads is None else heads
    for b in range(B):
        for h in hs:
            rnd = g.choice(S, size=min(n_random, S), replace=False)
            for i in sorted(set(cand) | set(int(r) for r in rnd)):
                rows.append((b, h, i))
    return np.array(rows, dtype=np.int64)


def check_rows(out_g, lse_g, rows, out_o, lse_o, has):
    og = out_g[rows[:, 0], rows[:, 2], rows[:, 1]].float().numpy().astype(np.float64)
    lg = lse_g[rows[:, 0], rows[:, 1], rows[:, 2]].numpy().astype(np.float64)
    hv = has[rows[:, 0], rows[:, 2]]
    stats = {"rows": int(len(rows)), "max_abs": 0.0, "max_lse": 0.0, "rel_l2": 0.0}
    if hv.any():
        diff = np.abs(og[hv] - out_o[hv])
        stats["max_abs"] = float(diff.max())
        stats["max_tol_frac"] = float((diff / (OUT_ATOL + BF16_U * np.abs(out_o[hv]))).max())
        stats["max_lse"] = float(np.abs(lg[hv] - lse_o[hv]).max())
        stats["rel_l2"] = float(np.linalg.norm(og[hv] - out_o[hv]) / np.linalg.norm(out_o[hv]))
        assert stats["max_tol_frac"] <= 1.0, stats
        assert stats["max_lse"] <= LSE_ATOL, stats
        assert stats["rel_l2"] <= REL_L2, stats
    if (~hv).any():
        bits = out_g[rows[:, 0], rows[:, 2], rows[:, 1]].view(torch.int16).numpy()[~hv]
        assert np.all(bits == 0)
        assert np.all(np.isneginf(lg[~hv]))
    return stats
