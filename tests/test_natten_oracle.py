"""Pins for the 3D neighbourhood-attention oracle (``oracle/natten_oracle.c``),
run without a GPU.

The pages name the operation (a windowed-attention primitive for the
neighbourhood-attention VAE decoder, window 11 x 11 x 11) but print no values,
so the oracle is pinned by mathematics:

  * library routine -- torch's CPU float64 scaled_dot_product_attention with
    a boolean mask built here from an independent characterisation of the
    window: along each axis, the window of coordinate c is the set of the
    k_eff grid positions nearest to c (unique for odd k), found by sorting
    distances, not by the oracle's clamp formula; and the whole-grid window,
    which must equal unmasked attention;
  * closed forms -- a 1 x 1 x 1 window returns the own value with lse = s_ii;
    Q = 0 returns the window mean of V with lse = ln(window volume), the same
    volume for every query (the window shifts inward at the border);
  * invariants -- reflecting the grid along any axis reflects the output;
    other heads and batches do not leak; row subsets and thread counts
    change nothing;
  * exact arithmetic -- a 40-digit Decimal evaluation on a tiny grid.
Window sizes must be odd; the oracle rejects even sizes.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def bits(t):
    return W.bf16_bits(t)


def run(x, grid, window, scale=0.125, **kw):
    return oracle.natten3d_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), grid, window, scale, **kw)


def nearest_window(c, k, n):
    """The min(k, n) positions of [0, n) nearest to c (k odd: no ties at the cut)."""
    order = sorted(range(n), key=lambda p: (abs(p - c), p))
    return set(order[:min(k, n)])


def window_mask(grid, window):
    """bool [S, S]: key j is in query i's window, built from nearest_window."""
    NT, NH, NW = grid
    KT, KH, KW = window
    coords = [(t, y, x) for t in range(NT) for y in range(NH) for x in range(NW)]
    wt = [nearest_window(c, KT, NT) for c in range(NT)]
    wh = [nearest_window(c, KH, NH) for c in range(NH)]
    ww = [nearest_window(c, KW, NW) for c in range(NW)]
    S = len(coords)
    m = np.zeros((S, S), dtype=bool)
    for i, (t, y, x) in enumerate(coords):
        for j, (t2, y2, x2) in enumerate(coords):
            m[i, j] = (t2 in wt[t]) and (y2 in wh[y]) and (x2 in ww[x])
    return m


def sdpa_masked(x, mask, scale):
    q = x["q"].double().permute(0, 2, 1, 3)
    k = x["k"].double().permute(0, 2, 1, 3)
    v = x["v"].double().permute(0, 2, 1, 3)
    m = torch.from_numpy(mask)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    lse = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


# --- library routine ------------------------------------------------------------
@pytest.mark.parametrize("grid,window", [
    ((3, 4, 5), (3, 3, 3)),
    ((4, 5, 6), (3, 5, 3)),
    ((2, 3, 9), (5, 1, 7)),     # window longer than the t axis: whole axis
    ((5, 2, 4), (1, 3, 3)),
    ((3, 6, 7), (3, 3, 5)),
])
def test_matches_sdpa_with_nearest_positions_mask(grid, window):
    S = grid[0] * grid[1] * grid[2]
    x = W.make_random(2, S, 2, 64, seed=401 + S)
    out, lse = run(x, grid, window, 0.2)
    ro, rl = sdpa_masked(x, window_mask(grid, window), 0.2)
    assert np.abs(out - ro).max() < 1e-12
    assert np.abs(lse - rl).max() < 1e-12


def test_whole_grid_window_is_full_attention():
    grid = (3, 3, 4)
    S = 36
    x = W.make_random(1, S, 3, 128, seed=411)
    out, lse = run(x, grid, (7, 5, 9), 0.09)
    ro, rl = sdpa_masked(x, np.ones((S, S), dtype=bool), 0.09)
    assert np.abs(out - ro).max() < 1e-12
    assert np.abs(lse - rl).max() < 1e-12


# --- closed forms -------------------------------------------------------------
def test_unit_window_returns_own_value():
    grid = (2, 3, 4)
    x = W.make_random(1, 24, 2, 64, seed=421)
    out, lse = run(x, grid, (1, 1, 1), 0.3)
    v = x["v"].double().numpy()
    assert np.array_equal(out, v)
    q = x["q"].double().numpy()
    k = x["k"].double().numpy()
    s = 0.3 * np.einsum("bshd,bshd->bhs", q, k)
    assert np.abs(lse - s).max() < 1e-12


def test_zero_query_gives_window_mean_and_constant_volume():
    grid, window = (4, 5, 7), (3, 3, 5)
    S = 140
    x = W.make_random(1, S, 2, 64, seed=431)
    x["q"] = torch.zeros_like(x["q"])
    out, lse = run(x, grid, window, 0.5)
    m = window_mask(grid, window)
    vol = 3 * 3 * 5
    assert np.all(m.sum(1) == vol)
    v = x["v"].double().numpy()[0]
    for i in range(S):
        J = np.nonzero(m[i])[0]
        want = v[J].mean(0)
        assert np.abs(out[0, i] - want).max() < 1e-12
    assert np.abs(lse - np.log(vol)).max() < 1e-12


# --- invariants ---------------------------------------------------------------
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_reflection_along_an_axis_reflects_the_output(axis):
    grid, window = (3, 5, 6), (3, 3, 5)
    S = 90
    x = W.make_random(1, S, 1, 64, seed=441 + axis)
    out, lse = run(x, grid, window, 0.25)

    def flip(t):
        shp = t.shape  # [B, S, H, D]
        g = t.reshape(shp[0], *grid, *shp[2:])
        return torch.flip(g, dims=[1 + axis]).reshape(shp)

    xf = {n: flip(x[n]) for n in ("q", "k", "v")}
    out_f, lse_f = run(xf, grid, window, 0.25)
    back = flip(torch.from_numpy(out_f)).numpy()
    assert np.abs(back - out).max() < 1e-12
    lse_b = flip(torch.from_numpy(lse_f).permute(0, 2, 1)[..., None])[..., 0].permute(0, 2, 1).numpy()
    assert np.abs(lse_b - lse).max() < 1e-12


def test_batches_and_heads_do_not_leak():
    grid, window = (2, 4, 5), (3, 3, 3)
    x = W.make_random(2, 40, 3, 64, seed=451)
    out, lse = run(x, grid, window, 0.2)
    y = {n: t.clone() for n, t in x.items()}
    for n in ("q", "k", "v"):
        y[n][1] = torch.randn_like(y[n][1].float()).bfloat16()
        y[n][0, :, 2] = torch.randn_like(y[n][0, :, 2].float()).bfloat16()
    out2, lse2 = run(y, grid, window, 0.2)
    assert np.array_equal(out[0, :, :2], out2[0, :, :2])
    assert np.array_equal(lse[0, :2], lse2[0, :2])


def test_row_subset_and_thread_count_match_full_evaluation():
    grid, window = (3, 4, 6), (3, 3, 3)
    x = W.make_random(2, 72, 2, 64, seed=461)
    out, lse = run(x, grid, window, 0.2, n_threads=1)
    out7, lse7 = run(x, grid, window, 0.2, n_threads=7)
    assert np.array_equal(out, out7) and np.array_equal(lse, lse7)
    rows = np.array([[0, 0, 0], [1, 1, 71], [0, 1, 35], [1, 0, 17]], dtype=np.int64)
    o, l = run(x, grid, window, 0.2, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(o[r], out[b, i, h]) and l[r] == lse[b, h, i]


def test_even_window_is_rejected():
    x = W.make_random(1, 24, 1, 64, seed=471)
    with pytest.raises(RuntimeError):
        run(x, (2, 3, 4), (3, 2, 3))


# --- exact arithmetic -----------------------------------------------------------
def test_matches_40_digit_decimal_evaluation():
    getcontext().prec = 40
    grid, window = (2, 2, 3), (1, 3, 3)
    S, D = 12, 4
    x = W.make_random(1, S, 1, D, seed=481, sigma_qk=2.0)
    scale = 0.375
    out, lse = run(x, grid, window, scale)
    m = window_mask(grid, window)
    q = x["q"].float().numpy()[0, :, 0]
    k = x["k"].float().numpy()[0, :, 0]
    v = x["v"].float().numpy()[0, :, 0]
    for i in range(S):
        J = list(np.nonzero(m[i])[0])
        s = {}
        for j in J:
            dot = sum(Fraction(float(q[i, d])) * Fraction(float(k[j, d])) for d in range(D))
            exact = Fraction(scale) * dot
            s[j] = Decimal(exact.numerator) / Decimal(exact.denominator)
        e = {j: s[j].exp() for j in J}
        tot = sum(e.values())
        assert abs(lse[0, 0, i] - float(tot.ln())) < 1e-14 * max(1.0, abs(float(tot.ln())))
        for d in range(D):
            want = float(sum(e[j] * Decimal(float(v[j, d])) for j in J) / tot)
            assert abs(out[0, i, 0, d] - want) < 1e-14


def test_output_sensitivity_bounds_reduces_and_sums_window_terms():
    """sum over the window of P_ij |v_jd|: >= |out|, == out bit for bit when
    v >= 0, and equal to the sum computed here from the probabilities of the
    whole-grid-masked reference on a small grid."""
    grid, window = (3, 4, 5), (3, 3, 3)
    B, H, D = 1, 2, 8
    S = grid[0] * grid[1] * grid[2]
    x = W.make_random(B, S, H, D, seed=181)
    b3 = [W.bf16_bits(x[n]) for n in ("q", "k", "v")]
    sens = np.zeros((B, S, H, D))
    out, _ = oracle.natten3d_fwd(*b3, grid, window, 0.2, sens=sens)
    assert np.all(sens >= np.abs(out) - 1e-15)
    sens2 = np.zeros_like(sens)
    out2, _ = oracle.natten3d_fwd(b3[0], b3[1], W.bf16_bits(x["v"].abs()), grid, window, 0.2, sens=sens2)
    assert np.array_equal(sens2, out2)
    # the same sums from an independent window mask and softmax in numpy
    mask = window_mask(grid, window)
    for h in range(H):
        q, k, v = (x[n][0, :, h].double().numpy() for n in ("q", "k", "v"))
        sc = 0.2 * q @ k.T
        sc[~mask] = -np.inf
        p = np.exp(sc - sc.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        assert np.abs(p @ np.abs(v) - sens[0, :, h]).max() < 1e-12
