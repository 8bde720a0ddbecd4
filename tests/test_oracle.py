"""Pins for the CPU oracle (``oracle/``), run without a GPU.

The pages print no attention inputs or outputs, so the oracle is pinned by
mathematics rather than by page values:

  * library routine -- torch's CPU float64 scaled_dot_product_attention with
    a boolean mask, and torch.logsumexp, on random segment layouts
    (catches a transposed operand, a wrong index, a dropped or wrong scale);
  * closed forms -- one-token segments return their own V and lse = s_ii;
    Q = 0 returns the segment mean of V with lse = ln|J|; constant V returns
    that constant; a two-token segment is a logistic blend; scores in
    arithmetic progression give geometric-series sums for lse and a weighted
    index mean for out (catches the sign of the exponent, key vs query
    indexing and the normaliser);
  * invariants -- rows of P sum to 1 and vanish off the segment; permuting
    keys inside a segment changes nothing; permuting queries permutes rows;
    joint permutation permutes rows; other segments, batches and heads do not
    leak into a row; (2q, scale/2) equals (q, scale) bit for bit;
    max s <= lse <= max s + ln|J|;
  * exact arithmetic -- a 40-digit Decimal evaluation of the definition on
    tiny inputs.
Masking conventions (ID 0 = padding, fully masked rows -> +0.0 and -inf) are
the readings recorded in the design notes.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def bits(t):
    return W.bf16_bits(t)


def run(x, seg_q=None, seg_kv=None, scale=0.125, **kw):
    sq = None if seg_q is None else seg_q.numpy()
    sk = None if seg_kv is None else seg_kv.numpy()
    return oracle.attn_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), sq, sk, scale, **kw)


def lse_close(a, b, tol):
    """|a - b| <= tol elementwise, with -inf matching -inf exactly."""
    a = np.asarray(a)
    b = np.asarray(b)
    ninf = np.isneginf(a)
    if not np.array_equal(ninf, np.isneginf(b)):
        return False
    return bool(np.all(np.abs(a[~ninf] - b[~ninf]) <= tol))


def sdpa_ref(x, seg, scale):
    """torch CPU float64 SDPA with a boolean mask; rows with no valid key are
    reported as NaN by torch, so callers compare only rows with J non-empty."""
    q = x["q"].double().permute(0, 2, 1, 3)
    k = x["k"].double().permute(0, 2, 1, 3)
    v = x["v"].double().permute(0, 2, 1, 3)
    B, H, S, D = q.shape
    if seg is None:
        mask = torch.ones(B, 1, S, S, dtype=torch.bool)
    else:
        mask = (seg[:, :, None] == seg[:, None, :]) & (seg[:, :, None] != 0)
        mask = mask[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    scores = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)  # [B, H, S]
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy(), mask[:, 0].numpy()


# --- library routine ----------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["single", "padded", "packed", "interleaved", "singletons", "negative",
                                  "extreme"])
def test_matches_torch_sdpa_f64(D, kind):
    B, S, H = 2, 97, 2
    x = W.make_random(B, S, H, D, seed=11 + D)
    seg = W.random_segments(B, S, seed=5, kind=kind)
    scale = 1.0 / math.sqrt(D)
    out, lse, _ = run(x, seg, seg.clone(), scale)
    ref_out, ref_lse, mask = sdpa_ref(x, seg, scale)
    has = mask.any(-1)  # [B, S]
    for b in range(B):
        for i in range(S):
            if has[b, i]:
                assert np.abs(out[b, i] - ref_out[b, i]).max() < 1e-12
                assert np.abs(lse[b, :, i] - ref_lse[b, :, i]).max() < 1e-12
            else:
                assert np.all(out[b, i] == 0.0)
                assert np.all(np.isneginf(lse[b, :, i]))


def test_unmasked_matches_torch_sdpa_f64():
    x = W.make_random(1, 300, 3, 64, seed=3)
    out, lse, _ = run(x, None, None, 0.125)
    ref_out, ref_lse, _ = sdpa_ref(x, None, 0.125)
    assert np.abs(out - ref_out).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12


# --- closed forms -------------------------------------------------------------
def test_singleton_segments_return_own_value():
    B, S, H, D = 1, 40, 2, 64
    x = W.make_random(B, S, H, D, seed=21)
    seg = W.random_segments(B, S, 0, "singletons")
    out, lse, _ = run(x, seg, seg.clone(), 0.3)
    v = x["v"].double().numpy()
    q = x["q"].double().numpy()
    k = x["k"].double().numpy()
    assert np.array_equal(out, v)  # weight exactly 1 -> exact V
    s_ii = 0.3 * np.einsum("bshd,bshd->bhs", q, k)
    assert np.abs(lse - s_ii).max() < 1e-12


def test_zero_query_gives_segment_mean():
    B, S, H, D = 1, 50, 2, 128
    x = W.make_random(B, S, H, D, seed=31)
    x["q"].zero_()
    seg = torch.tensor([[1] * 20 + [2] * 25 + [0] * 5], dtype=torch.int32)
    out, lse, _ = run(x, seg, seg.clone(), 0.2)
    v = x["v"].double().numpy()
    for lo, hi in ((0, 20), (20, 45)):
        mean = v[0, lo:hi].mean(axis=0)  # [H, D]
        assert np.abs(out[0, lo:hi] - mean[None]).max() < 1e-12
        assert np.abs(lse[0, :, lo:hi] - math.log(hi - lo)).max() < 1e-12
    assert np.all(out[0, 45:] == 0.0) and np.all(np.isneginf(lse[0, :, 45:]))


def test_constant_value_returned():
    B, S, H, D = 2, 33, 1, 64
    x = W.make_random(B, S, H, D, seed=41, sigma_qk=3.0)
    x["v"].fill_(-1.75)
    seg = W.random_segments(B, S, 7, "interleaved")
    out, lse, _ = run(x, seg, seg.clone(), 0.125)
    has = ((seg[:, :, None] == seg[:, None, :]) & (seg[:, :, None] != 0)).any(-1).numpy()
    for b in range(B):
        for i in range(S):
            want = -1.75 if has[b, i] else 0.0
            assert np.abs(out[b, i] - want).max() < 1e-14


def test_two_token_segment_is_logistic_blend():
    B, S, H, D = 1, 6, 1, 64
    x = W.make_random(B, S, H, D, seed=51)
    seg = torch.tensor([[4, 9, 4, 9, 7, 7]], dtype=torch.int32)
    scale = 0.25
    out, lse, _ = run(x, seg, seg.clone(), scale)
    q = x["q"].double().numpy()[0, :, 0]
    k = x["k"].double().numpy()[0, :, 0]
    v = x["v"].double().numpy()[0, :, 0]
    for a, b in ((0, 2), (1, 3), (4, 5)):
        for i in (a, b):
            s1 = scale * float(q[i] @ k[a])
            s2 = scale * float(q[i] @ k[b])
            w1 = 1.0 / (1.0 + math.exp(s2 - s1))
            want = w1 * v[a] + (1.0 - w1) * v[b]
            assert np.abs(out[0, i, 0] - want).max() < 1e-13
            want_lse = max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2)))
            assert abs(lse[0, 0, i] - want_lse) < 1e-13


@pytest.mark.parametrize("delta", [0.05, -0.3, 1.7])
def test_arithmetic_progression_scores_geometric_series(delta):
    """s_j = delta * j for j < n: lse and out follow geometric-series sums."""
    n, D = 200, 64
    q = torch.zeros(1, n, 1, D)
    k = torch.zeros(1, n, 1, D)
    v = torch.zeros(1, n, 1, D)
    q[..., 0] = 1.0
    k[0, :, 0, 0] = torch.arange(n, dtype=torch.float32)  # integers < 256: exact in bf16
    v[0, :, 0, 0] = torch.arange(n, dtype=torch.float32)
    v[0, :, 0, 1] = 1.0
    x = {"q": q.bfloat16(), "k": k.bfloat16(), "v": v.bfloat16()}
    out, lse, _ = run(x, None, None, delta)
    r = math.exp(delta)
    geo = math.expm1(n * delta) / math.expm1(delta)  # sum_j r^j
    arith = r * (1 - n * r ** (n - 1) + (n - 1) * r ** n) / (1 - r) ** 2  # sum_j j r^j
    assert np.abs(lse - math.log(geo)).max() < 1e-11 * max(1.0, abs(math.log(geo)))
    assert np.abs(out[0, :, 0, 0] - arith / geo).max() < 1e-9
    assert np.abs(out[0, :, 0, 1] - 1.0).max() < 1e-14
    assert np.all(out[0, :, 0, 2:] == 0.0)


def test_fully_masked_rows_zero_and_neg_inf():
    B, S, H, D = 2, 16, 2, 64
    x = W.make_random(B, S, H, D, seed=61)
    seg = torch.zeros(B, S, dtype=torch.int32)
    seg[1, :8] = 3  # batch 0 is all padding; batch 1 has 8 pad rows
    out, lse, _ = run(x, seg, seg.clone(), 0.1)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[1, 8:] == 0.0) and np.all(np.isneginf(lse[1, :, 8:]))
    assert np.all(np.isfinite(lse[1, :, :8]))
    assert not np.signbit(out[0]).any()  # +0.0, not -0.0


def test_query_segment_without_keys_is_masked():
    """seg_q and seg_kv differ: a query ID absent from seg_kv has no valid key."""
    B, S, H, D = 1, 12, 1, 64
    x = W.make_random(B, S, H, D, seed=62)
    seg_q = torch.tensor([[1] * 6 + [5] * 6], dtype=torch.int32)
    seg_kv = torch.tensor([[1] * 12], dtype=torch.int32)
    out, lse, _ = run(x, seg_q, seg_kv, 0.2)
    assert np.all(out[0, 6:] == 0.0) and np.all(np.isneginf(lse[0, :, 6:]))
    ref, ref_lse, _ = run(x, None, None, 0.2)
    assert np.abs(out[0, :6] - ref[0, :6]).max() < 1e-14


def test_large_scale_selects_argmax_key():
    B, S, H, D = 1, 64, 1, 64
    x = W.make_random(B, S, H, D, seed=71)
    scale = 400.0
    out, lse, _ = run(x, None, None, scale)
    q = x["q"].double().numpy()[0, :, 0]
    k = x["k"].double().numpy()[0, :, 0]
    v = x["v"].double().numpy()[0, :, 0]
    s = scale * q @ k.T
    for i in range(S):
        order = np.sort(s[i])
        if order[-1] - order[-2] > 60:  # runner-up weight < e^-60
            j = int(np.argmax(s[i]))
            assert np.abs(out[0, i, 0] - v[j]).max() < 1e-20
            assert abs(lse[0, 0, i] - s[i, j]) < 1e-12 * abs(s[i, j])


# --- invariants ---------------------------------------------------------------
def test_probability_rows_sum_to_one_and_vanish_off_segment():
    B, S, H, D = 1, 48, 2, 64
    x = W.make_random(B, S, H, D, seed=81, sigma_qk=3.0)
    seg = W.random_segments(B, S, 9, "interleaved")
    _, _, p = run(x, seg, seg.clone(), 0.125, want_probs=True)
    p = p.reshape(B, H, S, S)
    allowed = ((seg[:, :, None] == seg[:, None, :]) & (seg[:, :, None] != 0)).numpy()
    has = allowed.any(-1)
    assert np.all(p >= 0.0)
    assert np.all(p[:, :, ~allowed[0]] == 0.0)
    sums = p.sum(-1)
    assert np.abs(sums[:, :, has[0]] - 1.0).max() < 1e-14
    assert np.all(sums[:, :, ~has[0]] == 0.0)


def test_key_permutation_within_segment_is_invariant():
    B, S, H, D = 1, 60, 2, 128
    x = W.make_random(B, S, H, D, seed=91)
    seg = torch.tensor([[1] * 25 + [2] * 35], dtype=torch.int32)
    out, lse, _ = run(x, seg, seg.clone(), 0.09)
    g = torch.Generator().manual_seed(3)
    perm = torch.cat([torch.randperm(25, generator=g), 25 + torch.randperm(35, generator=g)])
    # Permute keys and values only (queries stay put): every row must be unchanged.
    y = {"q": x["q"], "k": x["k"][:, perm].contiguous(), "v": x["v"][:, perm].contiguous()}
    out2, lse2, _ = run(y, seg, seg[:, perm].contiguous(), 0.09)
    assert np.abs(out - out2).max() < 1e-13
    assert lse_close(lse, lse2, 1e-13)


def test_query_permutation_permutes_rows_exactly():
    B, S, H, D = 1, 45, 1, 64
    x = W.make_random(B, S, H, D, seed=101)
    seg = W.random_segments(B, S, 4, "packed")
    out, lse, _ = run(x, seg, seg.clone(), 0.125)
    perm = torch.randperm(S, generator=torch.Generator().manual_seed(8))
    y = {"q": x["q"][:, perm].contiguous(), "k": x["k"], "v": x["v"]}
    out2, lse2, _ = run(y, seg[:, perm].contiguous(), seg.clone(), 0.125)
    assert np.array_equal(out2, out[:, perm.numpy()])
    assert np.array_equal(lse2, lse[:, :, perm.numpy()])


def test_joint_permutation_over_sequence():
    B, S, H, D = 1, 70, 2, 64
    x = W.make_random(B, S, H, D, seed=111)
    seg = W.random_segments(B, S, 12, "packed")
    out, lse, _ = run(x, seg, seg.clone(), 0.125)
    perm = torch.randperm(S, generator=torch.Generator().manual_seed(9))
    y = {n: x[n][:, perm].contiguous() for n in ("q", "k", "v")}
    sp = seg[:, perm].contiguous()
    out2, lse2, _ = run(y, sp, sp.clone(), 0.125)
    assert np.abs(out2 - out[:, perm.numpy()]).max() < 1e-13
    assert lse_close(lse2, lse[:, :, perm.numpy()], 1e-13)


def test_other_segment_does_not_leak():
    B, S, H, D = 1, 64, 2, 64
    x = W.make_random(B, S, H, D, seed=121)
    seg = torch.tensor([[1, 2] * 32], dtype=torch.int32)  # interleaved segments
    out, lse, _ = run(x, seg, seg.clone(), 0.125)
    y = W.make_random(B, S, H, D, seed=999)
    z = {n: x[n].clone() for n in ("q", "k", "v")}
    sel = seg[0] == 2
    for n in ("q", "k", "v"):
        z[n][:, sel] = y[n][:, sel]
    out2, lse2, _ = run(z, seg, seg.clone(), 0.125)
    s1 = (seg[0] == 1).numpy()
    assert np.array_equal(out[:, s1], out2[:, s1])
    assert np.array_equal(lse[:, :, s1], lse2[:, :, s1])


def test_batch_and_head_split_are_exact():
    B, S, H, D = 2, 37, 3, 64
    x = W.make_random(B, S, H, D, seed=131)
    seg = W.random_segments(B, S, 13, "padded")
    out, lse, _ = run(x, seg, seg.clone(), 0.125)
    for b in range(B):
        for h in range(H):
            y = {n: x[n][b:b + 1, :, h:h + 1].contiguous() for n in ("q", "k", "v")}
            sb = seg[b:b + 1].contiguous()
            o1, l1, _ = run(y, sb, sb.clone(), 0.125)
            assert np.array_equal(o1[0, :, 0], out[b, :, h])
            assert np.array_equal(l1[0, 0], lse[b, h])


def test_scale_and_query_doubling_are_equivalent():
    x = W.make_random(1, 50, 2, 64, seed=141)
    out, lse, _ = run(x, None, None, 0.2)
    y = dict(x)
    y["q"] = (x["q"].float() * 2).bfloat16()  # exact in bf16
    out2, lse2, _ = run(y, None, None, 0.1)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_lse_bounds():
    B, S, H, D = 1, 80, 2, 64
    x = W.make_random(B, S, H, D, seed=151, sigma_qk=3.0)
    seg = W.random_segments(B, S, 14, "packed")
    out, lse, p = run(x, seg, seg.clone(), 0.125, want_probs=True)
    q = x["q"].double().numpy()
    k = x["k"].double().numpy()
    allowed = ((seg[:, :, None] == seg[:, None, :]) & (seg[:, :, None] != 0)).numpy()[0]
    for h in range(H):
        s = 0.125 * q[0, :, h] @ k[0, :, h].T
        for i in range(S):
            if not allowed[i].any():
                continue
            smax = s[i][allowed[i]].max()
            n = allowed[i].sum()
            assert smax - 1e-12 <= lse[0, h, i] <= smax + math.log(n) + 1e-12


def test_null_segments_equal_all_ones():
    x = W.make_random(2, 41, 2, 64, seed=161)
    ones = torch.ones(2, 41, dtype=torch.int32)
    a = run(x, None, None, 0.125)
    b = run(x, ones, ones.clone(), 0.125)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_row_subset_matches_full_evaluation():
    B, S, H, D = 2, 30, 2, 64
    x = W.make_random(B, S, H, D, seed=171)
    seg = W.random_segments(B, S, 15, "packed")
    out, lse, _ = run(x, seg, seg.clone(), 0.125)
    rows = np.array([[0, 0, 0], [1, 1, 29], [0, 1, 17], [1, 0, 3]], dtype=np.int64)
    o2, l2, _ = run(x, seg, seg.clone(), 0.125, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(o2[r], out[b, i, h])
        assert l2[r] == lse[b, h, i] or (np.isneginf(l2[r]) and np.isneginf(lse[b, h, i]))


def test_thread_count_does_not_change_results():
    x = W.make_random(1, 64, 4, 64, seed=181)
    a = run(x, None, None, 0.125, n_threads=1)
    b = run(x, None, None, 0.125, n_threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --- exact arithmetic -----------------------------------------------------------
def test_matches_40_digit_decimal_evaluation():
    getcontext().prec = 40
    B, S, H, D = 1, 7, 1, 5
    x = W.make_random(B, S, H, D, seed=191, sigma_qk=2.0)
    seg = torch.tensor([[3, 3, 0, 3, 8, 8, 3]], dtype=torch.int32)
    scale = 0.375
    out, lse, _ = run(x, seg, seg.clone(), scale)
    q = x["q"].float().numpy()[0, :, 0]
    k = x["k"].float().numpy()[0, :, 0]
    v = x["v"].float().numpy()[0, :, 0]
    sg = seg[0].tolist()
    for i in range(S):
        J = [j for j in range(S) if sg[i] != 0 and sg[j] == sg[i]]
        if not J:
            assert np.all(out[0, i, 0] == 0) and np.isneginf(lse[0, 0, i])
            continue
        s = {}
        for j in J:
            dot = sum(Fraction(float(q[i, d])) * Fraction(float(k[j, d])) for d in range(D))
            exact = Fraction(scale) * dot
            s[j] = Decimal(exact.numerator) / Decimal(exact.denominator)
        e = {j: s[j].exp() for j in J}
        tot = sum(e.values())
        want_lse = float(tot.ln())
        assert abs(lse[0, 0, i] - want_lse) < 1e-14 * max(1.0, abs(want_lse))
        for d in range(D):
            want = float(sum(e[j] * Decimal(float(v[j, d])) for j in J) / tot)
            assert abs(out[0, i, 0, d] - want) < 1e-14


# --- the output rounding-sensitivity sums ------------------------------------------------
# sens_id = sum_j P_ij |v_jd| sets the per-element parity tolerance where the
# first-order rounding bound of a bf16-probability kernel exceeds the fixed
# one.  Pinned against a separately written model in which every probability
# carries its own relative perturbation (the normaliser kept exact, as a
# kernel that sums the unrounded weights does): the sum over keys of the
# magnitudes of the one-hot derivatives of out_id must equal sens_id.

def _perturbed_out(x, seg, scale, b, h, eps):
    """out[b, :, h, :] with P_ij -> P_ij (1 + eps[i, j]), numpy fp64."""
    q, k, v = (x[n][b, :, h].double().numpy() for n in ("q", "k", "v"))
    S = q.shape[0]
    out = np.zeros_like(q)
    for i in range(S):
        js = [j for j in range(S) if seg is None or (seg[b, i] != 0 and seg[b, j] == seg[b, i])]
        if not js:
            continue
        s = np.array([scale * float(np.dot(q[i], k[j])) for j in js])
        w = np.exp(s - s.max())
        p = w / w.sum()
        for t, j in enumerate(js):
            out[i] += p[t] * (1.0 + eps[i, j]) * v[j]
    return out


@pytest.mark.parametrize("kind", [None, "packed", "interleaved"])
def test_output_sensitivity_equals_first_order_deviation(kind):
    B, S, H, D = 1, 11, 2, 6
    x = W.make_random(B, S, H, D, seed=171, sigma_qk=2.0)
    seg = None if kind is None else W.random_segments(B, S, 172, kind)
    sens = np.zeros((B, S, H, D))
    s = None if seg is None else seg.numpy()
    out, _, _ = oracle.attn_fwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), s, None if s is None else s.copy(),
                                0.3, sens=sens)
    for h in range(H):
        base = _perturbed_out(x, s, 0.3, 0, h, np.zeros((S, S)))
        assert np.abs(base - out[0, :, h]).max() < 1e-12
        tot = np.zeros((S, D))
        for i in range(S):
            for j in range(S):
                e = np.zeros((S, S))
                e[i, j] = 1.0
                tot += np.abs(_perturbed_out(x, s, 0.3, 0, h, e) - base)
        assert np.all(np.abs(sens[0, :, h] - tot) <= 1e-12 * np.maximum(tot, 1.0)), np.abs(sens[0, :, h] - tot).max()


def test_output_sensitivity_bounds_and_reduces():
    """sens >= |out|; with v >= 0 every term is non-negative and sens == out
    bit for bit; rows without a valid key give 0; the row-subset evaluation
    gives the same values."""
    B, S, H, D = 2, 40, 2, 64
    x = W.make_random(B, S, H, D, seed=173)
    seg = W.random_segments(B, S, 174, "packed").numpy()
    sens = np.zeros((B, S, H, D))
    b3 = [bits(x[n]) for n in ("q", "k", "v")]
    out, lse, _ = oracle.attn_fwd(*b3, seg, seg.copy(), 0.125, sens=sens)
    assert np.all(sens >= np.abs(out) - 1e-15)
    dead = np.isneginf(np.transpose(lse, (0, 2, 1)))
    assert np.all(sens[dead] == 0.0)
    vpos = bits(x["v"].abs())
    sens2 = np.zeros_like(sens)
    out2, _, _ = oracle.attn_fwd(b3[0], b3[1], vpos, seg, seg.copy(), 0.125, sens=sens2)
    assert np.array_equal(sens2, out2)
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(0, S, 3)], dtype=np.int64)
    sr = np.zeros((len(rows), D))
    oracle.attn_fwd(*b3, seg, seg.copy(), 0.125, rows=rows, sens=sr)
    assert np.array_equal(sr, sens[rows[:, 0], rows[:, 2], rows[:, 1]])
