"""Pins for the 3D rotary-embedding oracle (``oracle/rope_oracle.c``), run
without a GPU.

The rotation is pinned against what the mathematics fixes, not against a
restatement of its formula:
  * rounding -- the final bf16 rounding equals a brute-force nearest search
    over all finite bf16 values in exact rational arithmetic (ties to even),
    including ties and the subnormal range;
  * special cases -- zero angles return the input bits; a quarter turn maps a
    pair (x0, x1) to (-x1, x0) and a half turn negates it, bit for bit;
  * a library routine -- each pair, read as the complex number x0 + i x1 (or
    its split-halves counterpart), times cos + i sin in numpy complex128,
    gives the unrounded values exactly;
  * invariants -- a pair's norm scales by cos^2 + sin^2; q . k of rotated
    vectors depends only on the position difference per axis (exactly with
    quarter-turn tables, to the tables' fp32 rounding with the frequency
    schedule); moving one axis's position changes only that axis's section;
    the split-halves pairing is the interleaved one conjugated by a feature
    permutation; tokens outside the tables and features past the sections
    are untouched;
  * the attention composition -- zero angles reproduce plain attention, and
    a common shift of every token's position leaves quarter-turn attention
    unchanged.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def bits(t):
    return W.bf16_bits(t)


def bf16_to_f64(b):
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tables_const(n, dims, c, s):
    return (tuple(np.full((n[a], dims[a] // 2), c, dtype=np.float32) for a in range(3)),
            tuple(np.full((n[a], dims[a] // 2), s, dtype=np.float32) for a in range(3)))


def tables_schedule(n, dims):
    cs = [W.rope3d_tables(n[a], dims[a]) for a in range(3)]
    return tuple(c[0].numpy() for c in cs), tuple(c[1].numpy() for c in cs)


def quarter_tables(n, dims):
    """angle(pos, p) = (pos + p) * pi/2: cos and sin in {-1, 0, 1}, exact."""
    cos, sin = [], []
    for a in range(3):
        k = (np.arange(n[a])[:, None] + np.arange(dims[a] // 2)[None, :]) % 4
        cos.append(np.array([1, 0, -1, 0], dtype=np.float32)[k])
        sin.append(np.array([0, 1, 0, -1], dtype=np.float32)[k])
    return tuple(cos), tuple(sin)


def pairs(D, dims, interleaved):
    """(i0, i1, axis, p) of every rotated pair."""
    out, off = [], 0
    for a in range(3):
        h = dims[a] // 2
        for p in range(h):
            out.append((off + 2 * p, off + 2 * p + 1, a, p) if interleaved else (off + p, off + p + h, a, p))
        off += dims[a]
    return out


# --- rounding -------------------------------------------------------------------------------
_ALL_BF16 = None


def _finite_bf16_sorted():
    global _ALL_BF16
    if _ALL_BF16 is None:
        b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        v = bf16_to_f64(b)
        ok = np.isfinite(v) & ~((v == 0) & (b == 0x8000))  # one zero
        _ALL_BF16 = (v[ok][np.argsort(v[ok])], b[ok][np.argsort(v[ok])])
    return _ALL_BF16


def brute_round(x):
    vals, bs = _finite_bf16_sorted()
    i = int(np.searchsorted(vals, x))
    cand = [j for j in (i - 1, i) if 0 <= j < len(vals)]
    fx = Fraction(x)
    best = min(cand, key=lambda j: (abs(Fraction(float(vals[j])) - fx), int(bs[j]) & 1))
    r = bs[best]
    if r == 0 and math.copysign(1.0, x) < 0:
        return np.uint16(0x8000)
    return r


def test_round_bf16_matches_brute_force():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(300) * np.exp2(rng.integers(-140, 120, 300)))
    # exact midpoints between neighbouring bf16 values (ties), both parities
    for base in (1.0, 1.0 + 2 ** -7, 3.5, -2.0 ** -126, 2.0 ** -130, 1.0 + 3 * 2 ** -7):
        ulp = 2.0 ** (math.floor(math.log2(abs(base))) - 7) if abs(base) >= 2 ** -126 else 2.0 ** -133
        vals += [base + ulp / 2, base - ulp / 2, base + ulp / 2 * (1 + 2 ** -30)]
    vals += [0.0, -0.0, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -133 * 1.5]
    got = oracle.round_bf16(np.array(vals))
    for x, g in zip(vals, got):
        assert g == brute_round(x), (x, hex(int(g)), hex(int(brute_round(x))))


# --- special cases --------------------------------------------------------------------------
@pytest.mark.parametrize("interleaved", [True, False])
def test_zero_angle_returns_input_bits(interleaved):
    B, S, H, D = 2, 17, 3, 64
    x = W.randn_bf16((B, S, H, D), 11)
    n, dims = (3, 4, 5), (20, 22, 22)
    pos = W.random_positions(B, S, n, 12).numpy()
    cos, sin = tables_const(n, dims, 1.0, 0.0)
    y, yd = oracle.rope3d(bits(x), pos, cos, sin, dims, interleaved)
    assert np.array_equal(y, bits(x))
    assert np.array_equal(yd, x.double().numpy())


@pytest.mark.parametrize("interleaved", [True, False])
def test_quarter_and_half_turns(interleaved):
    B, S, H, D = 1, 9, 2, 128
    x = W.randn_bf16((B, S, H, D), 21)
    n, dims = (2, 3, 4), (44, 42, 42)
    pos = W.random_positions(B, S, n, 22, outside=0.0).numpy()
    xb = bits(x)
    neg = lambda u: u ^ np.uint16(0x8000)
    # (cos, sin) -> the pair (x0, x1) it must produce, by sign flips and swaps
    turns = {(0.0, 1.0): lambda a, b: (neg(b), a), (-1.0, 0.0): lambda a, b: (neg(a), neg(b)),
             (0.0, -1.0): lambda a, b: (b, neg(a))}
    for (c, s), f in turns.items():
        cos, sin = tables_const(n, dims, c, s)
        y, _ = oracle.rope3d(xb, pos, cos, sin, dims, interleaved)
        want = xb.copy()
        for i0, i1, _, _ in pairs(D, dims, interleaved):
            want[..., i0], want[..., i1] = f(xb[..., i0], xb[..., i1])
        assert np.array_equal(y, want), (c, s)


# --- library routine ------------------------------------------------------------------------
@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("D,dims", [(64, (20, 22, 22)), (128, (44, 42, 42)), (128, (0, 64, 32)),
                                    (64, (2, 0, 60))])
def test_complex_multiplication(interleaved, D, dims):
    B, S, H = 2, 13, 2
    x = W.randn_bf16((B, S, H, D), 31 + D)
    n = (5, 6, 7)
    pos = W.random_positions(B, S, n, 32).numpy()
    cos, sin = tables_schedule(n, dims)
    _, yd = oracle.rope3d(bits(x), pos, cos, sin, dims, interleaved)
    xf = x.double().numpy()
    want = xf.copy()
    inside = np.all((pos >= 0) & (pos < np.array(n)), axis=-1)
    for i0, i1, a, p in pairs(D, dims, interleaved):
        z = xf[..., i0] + 1j * xf[..., i1]
        pa = np.clip(pos[..., a], 0, n[a] - 1)
        e = cos[a][pa, p].astype(np.float64) + 1j * sin[a][pa, p].astype(np.float64)
        r = z * e[:, :, None]
        m = inside[:, :, None]
        want[..., i0] = np.where(m, r.real, xf[..., i0])
        want[..., i1] = np.where(m, r.imag, xf[..., i1])
    assert np.array_equal(yd, want)


# --- invariants -----------------------------------------------------------------------------
def test_pair_norm_scales_by_table_norm():
    B, S, H, D = 1, 31, 2, 128
    dims = (44, 42, 42)
    x = W.randn_bf16((B, S, H, D), 41)
    n = (21, 45, 80)
    pos = W.random_positions(B, S, n, 42, outside=0.0).numpy()
    cos, sin = tables_schedule(n, dims)
    _, yd = oracle.rope3d(bits(x), pos, cos, sin, dims, True)
    xf = x.double().numpy()
    for i0, i1, a, p in pairs(D, dims, True):
        c = cos[a][pos[..., a], p].astype(np.float64)[:, :, None]
        s = sin[a][pos[..., a], p].astype(np.float64)[:, :, None]
        lhs = yd[..., i0] ** 2 + yd[..., i1] ** 2
        rhs = (xf[..., i0] ** 2 + xf[..., i1] ** 2) * (c * c + s * s)
        assert np.all(np.abs(lhs - rhs) <= 1e-14 * rhs + 1e-300)


@pytest.mark.parametrize("interleaved", [True, False])
def test_dot_product_depends_on_position_difference(interleaved):
    B, S, H, D = 1, 2, 1, 128
    dims = (44, 42, 42)
    q = W.randn_bf16((B, 1, H, D), 51)
    k = W.randn_bf16((B, 1, H, D), 52)
    n = (24, 24, 24)
    rng = np.random.default_rng(53)
    for tabs, tol in ((quarter_tables(n, dims), 0.0), (tables_schedule(n, dims), 2e-6)):
        cos, sin = tabs
        ref = None
        for shift in range(4):
            m = rng.integers(0, 8, 3)
            delta = np.array([3, 1, 5])
            pq = np.array([[m + shift * 4]], dtype=np.int32)
            pk = np.array([[m + shift * 4 + delta]], dtype=np.int32)
            _, yq = oracle.rope3d(bits(q), pq, cos, sin, dims, interleaved)
            _, yk = oracle.rope3d(bits(k), pk, cos, sin, dims, interleaved)
            dot = float(np.dot(yq.ravel(), yk.ravel()))
            scale = float(np.linalg.norm(yq) * np.linalg.norm(yk))
            if ref is None:
                ref = dot
            assert abs(dot - ref) <= tol * scale + 1e-12 * scale, (shift, dot, ref)


def test_each_axis_moves_only_its_section():
    B, S, H, D = 1, 1, 2, 128
    dims = (44, 42, 42)
    x = W.randn_bf16((B, S, H, D), 61)
    n = (8, 8, 8)
    cos, sin = tables_schedule(n, dims)
    base = np.array([[[2, 3, 4]]], dtype=np.int32)
    y0, _ = oracle.rope3d(bits(x), base, cos, sin, dims, False)
    edges = [0, 44, 86, 128]
    for a in range(3):
        p2 = base.copy()
        p2[..., a] += 3
        y1, _ = oracle.rope3d(bits(x), p2, cos, sin, dims, False)
        changed = np.nonzero(np.any(y1 != y0, axis=(0, 1, 2)))[0]
        assert len(changed) > 0
        assert changed.min() >= edges[a] and changed.max() < edges[a + 1], (a, changed)


def test_split_halves_is_a_permuted_interleaving():
    B, S, H, D = 2, 11, 2, 64
    dims = (20, 22, 22)
    x = W.randn_bf16((B, S, H, D), 71)
    n = (5, 5, 5)
    pos = W.random_positions(B, S, n, 72).numpy()
    cos, sin = tables_schedule(n, dims)
    # perm[j] = the split-halves feature that sits at interleaved slot j
    perm = np.arange(D)
    for (h0, h1, _, _), (j0, j1, _, _) in zip(pairs(D, dims, False), pairs(D, dims, True)):
        perm[j0], perm[j1] = h0, h1
    xb = bits(x)
    yh, _ = oracle.rope3d(xb, pos, cos, sin, dims, False)
    yi, _ = oracle.rope3d(np.ascontiguousarray(xb[..., perm]), pos, cos, sin, dims, True)
    assert np.array_equal(yh[..., perm], yi)


def test_outside_tables_and_tail_features_untouched():
    B, S, H, D = 1, 40, 2, 128
    dims = (30, 30, 30)  # features 90..127 are never rotated
    x = W.randn_bf16((B, S, H, D), 81)
    n = (3, 4, 5)
    pos = W.random_positions(B, S, n, 82, outside=0.5).numpy()
    cos, sin = tables_schedule(n, dims)
    y, _ = oracle.rope3d(bits(x), pos, cos, sin, dims, True)
    xb = bits(x)
    inside = np.all((pos >= 0) & (pos < np.array(n)), axis=-1)
    assert (~inside).sum() > 5 and inside.sum() > 5
    assert np.array_equal(y[~inside], xb[~inside])
    assert np.array_equal(y[..., 90:], xb[..., 90:])
    assert not np.array_equal(y[inside][..., :90], xb[inside][..., :90])


# --- composition with attention -------------------------------------------------------------
def test_zero_angles_reproduce_plain_attention():
    B, S, H, D = 1, 70, 2, 64
    x = W.make_random(B, S, H, D, seed=91)
    seg = W.random_segments(B, S, 92, "packed").numpy()
    dims = W.ROPE_DIMS[D]
    n = (2, 3, 4)
    cos, sin = tables_const(n, dims, 1.0, 0.0)
    pos = W.random_positions(B, S, n, 93).numpy()
    o1, l1 = oracle.rope3d_attn_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), pos, cos, sin, dims, True,
                                    seg, seg.copy(), 0.125)
    o2, l2, _ = oracle.attn_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), seg, seg.copy(), 0.125)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("interleaved", [True, False])
def test_common_position_shift_leaves_attention_unchanged(interleaved):
    """Quarter-turn tables rotate exactly, so every q . k keeps its terms up
    to order: a shift of all positions changes the output by summation order
    only."""
    B, S, H, D = 1, 48, 2, 128
    x = W.make_random(B, S, H, D, seed=95)
    dims = W.ROPE_DIMS[D]
    n = (12, 12, 12)
    cos, sin = quarter_tables(n, dims)
    pos = W.random_positions(B, S, (6, 6, 6), 96, outside=0.0).numpy()
    o1, l1 = oracle.rope3d_attn_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), pos, cos, sin, dims,
                                    interleaved, None, None, 0.1)
    o2, l2 = oracle.rope3d_attn_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), pos + np.int32(3), cos, sin,
                                    dims, interleaved, None, None, 0.1)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12
    # and the rotation did change the result (it is not the identity)
    o3, _, _ = oracle.attn_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), None, None, 0.1)
    assert np.abs(o1 - o3).max() > 1e-3
