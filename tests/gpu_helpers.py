"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same bf16 bits, and compare to the tolerances
of the parity bar.

Tolerances (bf16 output of fp32-accumulated attention):
  OUT_ATOL = 1e-2   |out_gpu - out_oracle| on every compared element (the
                    acceptance bound of the product, max |err| <= 1e-2),
                    except where the first-order rounding bound of the
                    arithmetic itself is larger (out_tol): the P V product
                    takes each probability rounded once to bf16 (relative
                    error up to BF16_U = 2^-8) and the output is rounded once
                    to bf16, so an element may be off by
                    BF16_U * sens + half a bf16 ULP of |out| + BF16_U * sens,
                    with sens = sum_j P_ij |v_jd| from the oracle.  That only
                    exceeds 1e-2 on peaky rows with a large |out|; each case
                    also reports its plain max |err| and how many elements
                    are above 1e-2;
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


def half_ulp_bf16(x):
    """Half a bf16 ULP of |x| (elementwise): bf16 keeps 8 significant bits,
    so a value in [2^e, 2^(e+1)) has ULP 2^(e-7); below 2^-126 the spacing
    is 2^-133."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 8).astype(np.int64))


def out_tol(ref, sens):
    """Per-element bound on |out_gpu - out_oracle|: OUT_ATOL, or where larger
    the first-order rounding bound BF16_U * sens (each probability rounded
    once to bf16) plus half a bf16 ULP of the value before the final
    rounding, plus 1e-5 for the fp32 score and sum arithmetic."""
    ref = np.asarray(ref, dtype=np.float64)
    sens = np.asarray(sens, dtype=np.float64)
    pre = np.abs(ref) + BF16_U * sens
    return np.maximum(OUT_ATOL, BF16_U * sens + half_ulp_bf16(pre) + 1e-5)


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
    """(out, lse, sens) of the oracle: fp64 [B,S,H,D] / [B,H,S] / [B,S,H,D], or
    [n, D] / [n] / [n, D] for listed (b, h, i) rows."""
    B, S, H, D = x["q"].shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    sens = np.zeros((B, S, H, D) if rows is None else (len(rows), D), dtype=np.float64)
    out, lse, _ = oracle.attn_fwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                  None if seg_q is None else seg_q.numpy(),
                                  None if seg_kv is None else seg_kv.numpy(), float(np.float32(scale)),
                                  rows=rows, sens=sens)
    return out, lse, sens


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


def _out_stats(stats, diff, ref, sens):
    tol = out_tol(ref, sens)
    stats["max_abs"] = float(diff.max())
    stats["max_tol_frac"] = float((diff / tol).max())
    stats["n_over_1e-2"] = int((diff > OUT_ATOL).sum())
    over = diff > OUT_ATOL
    if over.any():
        # how much of the rounding bound the elements above 1e-2 use
        stats["max_over_frac_of_rounding_bound"] = float(
            ((diff[over] - half_ulp_bf16(ref[over])) / (BF16_U * sens[over] + 1e-300)).max())


def check_full(out_g, lse_g, out_o, lse_o, has, sens):
    """Compare full outputs ([B,S,H,D] / [B,H,S]); sens: the oracle's
    rounding-sensitivity sums; returns a stats dict."""
    og = out_g.float().numpy().astype(np.float64)
    lg = lse_g.numpy().astype(np.float64)
    B, S, H, D = og.shape
    stats = {"max_abs": 0.0, "max_lse": 0.0, "rel_l2": 0.0}
    if has.any():
        diff = np.abs(og[has] - out_o[has])
        _out_stats(stats, diff, out_o[has], sens[has])
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


def check_rows(out_g, lse_g, rows, out_o, lse_o, has, sens):
    og = out_g[rows[:, 0], rows[:, 2], rows[:, 1]].float().numpy().astype(np.float64)
    lg = lse_g[rows[:, 0], rows[:, 1], rows[:, 2]].numpy().astype(np.float64)
    hv = has[rows[:, 0], rows[:, 2]]
    stats = {"rows": int(len(rows)), "max_abs": 0.0, "max_lse": 0.0, "rel_l2": 0.0}
    if hv.any():
        diff = np.abs(og[hv] - out_o[hv])
        _out_stats(stats, diff, out_o[hv], sens[hv])
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


# --- the split last round of vdx_attn_fwd_ws -----------------------------------------
# The schedule only (which query blocks are split into parts), restated from
# The library's documented rules.  A persistent grid has G workgroups (the CU
# count rounded down to a multiple of 8, W = G / 8 per XCD); with n > G items
# XCD x holds n_x = per + (x < rem) of them (per = n // 8, rem = n % 8).
# Unmasked (work stealing): XCD x's items are a contiguous run starting at
# item x per + min(x, rem) (item = (b H + h) n_qblk + block), and when
# n_x > W its last R are split into P = min(8, W // R) >= 2 parts, R = W // 4
# when n_x // W >= 4, else R = n_x % W.  Masked (shared pool): each XCD runs
# K rounds of its own items (K = per // W - 2 when per // W >= 4, else
# per // W); the rest forms a pool of n - K G items whose last R (G // 4 for
# the long launches, else all of them) are split into
# P = min(8, 256 // R, G // R) >= 2 parts.
def persistent_grid():
    return torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8


def tail_plan(x, n_items, W):
    """(n_x, R, P) of XCD x, unmasked."""
    n_x = n_items // 8 + (1 if x < n_items % 8 else 0)
    if n_x > W:
        R = W // 4 if n_x // W >= 4 else n_x % W
        P = min(8, W // R) if R else 1
        if P >= 2:
            return n_x, R, P
    return n_x, 0, 1


def pool_plan(n_items, G):
    """(per, rem, K, n_pool, R, P) of the masked pool."""
    W = G // 8
    per, rem = n_items // 8, n_items % 8
    rounds = per // W
    long_launch = rounds >= 4
    K = rounds - 2 if long_launch else rounds
    n_pool = n_items - K * G
    R = min(n_pool, G // 4) if long_launch else n_pool % G
    P = min(8, 256 // R, G // R) if R > 0 else 1
    if P < 2:
        R, P = 0, 1
    return per, rem, K, n_pool, R, P


def n_split_items(n_items, grid, masked=True):
    if grid > 256 or n_items <= grid:
        return 0
    if masked:
        return pool_plan(n_items, grid)[4]
    return sum(tail_plan(x, n_items, grid // 8)[1] for x in range(8))


def split_unmasked_blocks(B, S, H, grid):
    """(b, h, block) of every 256-query block the unmasked vdx_attn_fwd_ws
    splits: XCD x owns a contiguous run of items, its local item j being
    item x per + min(x, rem) + j, and splits its last R."""
    n_qblk = (S + 255) // 256
    n = B * H * n_qblk
    if n <= grid or grid > 256:
        return []
    per, rem = n // 8, n % 8
    out = []
    for x in range(8):
        n_x, R, _ = tail_plan(x, n, grid // 8)
        for j in range(n_x - R, n_x):
            lid = x * per + min(x, rem) + j
            bh = lid // n_qblk
            out.append((bh // H, bh % H, lid % n_qblk))
    return out


def block_mask(B, H, S, blocks):
    """bool [B, S, H]: rows of the listed (b, h, block) query blocks."""
    m = np.zeros((B, S, H), dtype=bool)
    for b, h, blk in blocks:
        m[b, blk * 256:min(S, (blk + 1) * 256), h] = True
    return m


def differing_blocks(o1, l1, o2, l2):
    """(b, h, block) of the 256-query blocks where two results differ in any bit."""
    B, S, H, _ = o1.shape
    ob = (o1.view(torch.int16) != o2.view(torch.int16)).any(dim=3).cpu().numpy()  # [B, S, H]
    lb = (l1.view(torch.int32) != l2.view(torch.int32)).cpu().numpy().transpose(0, 2, 1)
    rows = ob | lb
    out = set()
    for b, i, h in zip(*np.nonzero(rows)):
        out.add((int(b), int(h), int(i) // 256))
    return sorted(out)


def assert_split_close(o1, l1, o2, l2):
    """A split block against the same block computed whole.  The parts round
    their probabilities to bf16 against their own reference maxima, so the
    two results carry different rounding errors, each within the oracle
    bound (which the callers check on rows of the split blocks): they may
    then lie on opposite sides of the exact value, so every element must be
    within twice max(OUT_ATOL, one bf16 ULP of the larger magnitude) of the
    other (the ULP term matters from |o| >= 2, as with the peaky N(0, 3^2)
    scores of packed clips), and the relative L2 distance within REL_L2.
    The sums l are taken from the unrounded probabilities in fp32, so lse
    agrees to 1e-5 (+1e-6 relative); empty rows (+0.0, -inf) are the same."""
    a = o1.float().cpu().numpy().astype(np.float64)
    b = o2.float().cpu().numpy().astype(np.float64)
    tol = 2.0 * np.maximum(OUT_ATOL, 2.0 * half_ulp_bf16(np.maximum(np.abs(a), np.abs(b))))
    assert np.all(np.abs(a - b) <= tol), float(np.abs(a - b).max())
    nb = np.linalg.norm(b)
    if nb > 0:
        assert np.linalg.norm(a - b) / nb <= REL_L2
    la = l1.cpu().numpy().astype(np.float64)
    lb = l2.cpu().numpy().astype(np.float64)
    fa, fb = np.isfinite(la), np.isfinite(lb)
    assert np.array_equal(fa, fb)
    assert np.array_equal(la[~fa], lb[~fb])
    assert np.all(np.abs(la[fa] - lb[fa]) <= 1e-5 + 1e-6 * np.abs(la[fa]))
    dead = torch.from_numpy(~fa.transpose(0, 2, 1).copy())  # [B, S, H]
    assert torch.all(o1.view(torch.int16).cpu()[dead] == 0)
