"""Pins for the gradient oracle (``oracle/attn_bwd_oracle.c``), run without a GPU.

  * library routine -- torch CPU float64 autograd through
    scaled_dot_product_attention with the segment mask (rows without a valid
    key get dout = 0 and an all-true mask row on the torch side, which cannot
    represent them; the oracle gets the real dout and must ignore it there);
  * numerical differentiation -- central differences of sum(dout * out) of a
    dense numpy fp64 forward written here, on a few entries of q, k and v;
  * closed forms -- one-token segments: dq = dk = 0, dv = dout; constant v:
    dq = dk = 0; q = 0: dk = 0 and dq_i = scale/n * sum_j (dout_i . (v_j -
    mean v)) k_j over the segment;
  * invariants -- within a segment the dk sum to zero and the dv sum to the
    sum of dout over its query rows; fully masked rows get dq = 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def bits(t):
    return W.bf16_bits(t)


def run(x, dout, seg=None, scale=0.125):
    s = None if seg is None else seg.numpy()
    return oracle.attn_bwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), bits(dout), s,
                           None if s is None else s.copy(), scale)


def torch_grads(x, dout, seg, scale):
    q = x["q"].double().permute(0, 2, 1, 3).clone().requires_grad_()
    k = x["k"].double().permute(0, 2, 1, 3).clone().requires_grad_()
    v = x["v"].double().permute(0, 2, 1, 3).clone().requires_grad_()
    B, H, S, D = q.shape
    do = dout.double().permute(0, 2, 1, 3).clone()
    if seg is None:
        mask = torch.ones(B, 1, S, S, dtype=torch.bool)
    else:
        m = (seg[:, :, None] == seg[:, None, :]) & (seg[:, :, None] != 0)
        dead = ~m.any(-1)                       # rows without a valid key
        m = m | dead[:, :, None]
        do = do.masked_fill(dead[:, None, :, None], 0.0)
        mask = m[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    (out * do).sum().backward()
    f = lambda t: t.grad.permute(0, 2, 1, 3).numpy()
    return f(q), f(k), f(v)


@pytest.mark.parametrize("kind", [None, "single", "padded", "packed", "interleaved", "allpad", "negative",
                                  "extreme"])
@pytest.mark.parametrize("D", [64, 128])
def test_matches_torch_autograd_f64(kind, D):
    B, S, H = 2, 48, 2
    x = W.make_random(B, S, H, D, seed=700 + D)
    dout = W.randn_bf16((B, S, H, D), 709 + D)
    seg = None if kind is None else W.random_segments(B, S, 711, kind)
    dq, dk, dv = run(x, dout, seg, 0.2)
    tq, tk, tv = torch_grads(x, dout, seg, 0.2)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - b).max() < 1e-12


def dense_forward(q, k, v, mask, scale):
    """numpy fp64 forward for one head: q,k,v [S, D], mask [S, S] bool."""
    s = scale * q @ k.T
    s = np.where(mask, s, -np.inf)
    m = s.max(1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(mask, np.exp(s - m), 0.0)
    l = w.sum(1, keepdims=True)
    return np.where(l > 0, (w @ v) / np.where(l > 0, l, 1.0), 0.0)


def test_matches_central_differences():
    S, D, scale = 10, 8, 0.4
    x = W.make_random(1, S, 1, D, seed=721, sigma_qk=1.5)
    dout = W.randn_bf16((1, S, 1, D), 722)
    seg = torch.tensor([[1, 1, 2, 1, 2, 2, 0, 1, 3, 2]], dtype=torch.int32)
    dq, dk, dv = run(x, dout, seg, scale)
    q0, k0, v0 = (x[n][0, :, 0].double().numpy() for n in ("q", "k", "v"))
    do = dout[0, :, 0].double().numpy()
    sg = seg[0].numpy()
    mask = (sg[:, None] == sg[None, :]) & (sg[:, None] != 0)

    def f(q, k, v):
        return float((dense_forward(q, k, v, mask, scale) * do).sum())

    eps = 1e-6
    rng = np.random.default_rng(3)
    for name, base, grad in (("q", q0, dq), ("k", k0, dk), ("v", v0, dv)):
        for _ in range(12):
            i, d = int(rng.integers(S)), int(rng.integers(D))
            args = {"q": q0, "k": k0, "v": v0}
            plus, minus = base.copy(), base.copy()
            plus[i, d] += eps
            minus[i, d] -= eps
            fp = f(**{**args, name: plus})
            fm = f(**{**args, name: minus})
            num = (fp - fm) / (2 * eps)
            assert abs(num - grad[0, i, 0, d]) < 1e-7, (name, i, d, num, grad[0, i, 0, d])


def test_singletons_pass_dout_to_dv_only():
    B, S, H, D = 1, 20, 2, 64
    x = W.make_random(B, S, H, D, seed=731)
    dout = W.randn_bf16((B, S, H, D), 732)
    seg = torch.arange(1, S + 1, dtype=torch.int32)[None]
    dq, dk, dv = run(x, dout, seg, 0.3)
    assert np.all(dq == 0) and np.all(dk == 0)
    assert np.array_equal(dv, dout.double().numpy())


def test_constant_value_gives_zero_dq_dk():
    B, S, H, D = 1, 30, 1, 64
    x = W.make_random(B, S, H, D, seed=741)
    x["v"] = torch.full_like(x["v"], 0.75)
    dout = W.randn_bf16((B, S, H, D), 742)
    dq, dk, dv = run(x, dout, None, 0.2)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_zero_query_closed_form():
    B, S, H, D = 1, 24, 1, 16
    x = W.make_random(B, S, H, D, seed=751)
    x["q"] = torch.zeros_like(x["q"])
    dout = W.randn_bf16((B, S, H, D), 752)
    seg = torch.tensor([[1] * 10 + [2] * 14], dtype=torch.int32)
    scale = 0.3
    dq, dk, dv = run(x, dout, seg, scale)
    assert np.all(dk == 0)
    k = x["k"][0, :, 0].double().numpy()
    v = x["v"][0, :, 0].double().numpy()
    do = dout[0, :, 0].double().numpy()
    for a, b in ((0, 10), (10, 24)):
        n = b - a
        vc = v[a:b] - v[a:b].mean(0)
        C = k[a:b].T @ vc          # sum_j k_j (v_j - mean v)^T, [D, D]
        for i in range(a, b):
            want = scale / n * (C @ do[i])
            assert np.abs(dq[0, i, 0] - want).max() < 1e-12
            assert np.abs(dv[0, i, 0] - do[a:b].mean(0) * 1.0).max() < 1e-12


def test_segment_sums_and_masked_rows():
    B, S, H, D = 1, 40, 2, 64
    x = W.make_random(B, S, H, D, seed=761)
    dout = W.randn_bf16((B, S, H, D), 762)
    seg = W.random_segments(B, S, 763, "interleaved")
    dq, dk, dv = run(x, dout, seg, 0.25)
    sg = seg[0].numpy()
    do = dout.double().numpy()
    for c in set(sg.tolist()) - {0}:
        idx = np.nonzero(sg == c)[0]
        assert np.abs(dk[0, idx].sum(0)).max() < 1e-12
        assert np.abs(dv[0, idx].sum(0) - do[0, idx].sum(0)).max() < 1e-12
    pad = np.nonzero(sg == 0)[0]
    assert np.all(dq[0, pad] == 0) and np.all(dk[0, pad] == 0) and np.all(dv[0, pad] == 0)


@pytest.mark.parametrize("kind", [None, "padded", "interleaved"])
def test_dq_rows_matches_torch_autograd_f64(kind):
    """The row-restricted dq (any S, used on sampled rows of long sequences)
    against torch CPU float64 autograd, on every row of a small case."""
    B, S, H, D = 2, 40, 2, 64
    x = W.make_random(B, S, H, D, seed=731)
    dout = W.randn_bf16((B, S, H, D), 733)
    seg = None if kind is None else W.random_segments(B, S, 735, kind)
    tq, _, _ = torch_grads(x, dout, seg, 0.3)
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(S)], dtype=np.int64)
    s = None if seg is None else seg.numpy()
    got = oracle.attn_bwd_dq_rows(bits(x["q"]), bits(x["k"]), bits(x["v"]), bits(dout), s,
                                  None if s is None else s.copy(), 0.3, rows)
    want = tq[rows[:, 0], rows[:, 2], rows[:, 1]]
    assert np.abs(got - want).max() < 1e-12


def test_dq_rows_beyond_the_dense_limit_q_zero_closed_form():
    """S above the dense routine's limit: with q = 0, dq_i = scale/S *
    sum_j (dout_i . (v_j - mean v)) k_j (uniform probabilities)."""
    B, S, H, D = 1, 16500, 1, 64
    x = W.make_random(B, S, H, D, seed=741)
    x["q"] = torch.zeros_like(x["q"])
    dout = W.randn_bf16((B, S, H, D), 743)
    rows = np.array([(0, 0, i) for i in (0, 1, 8191, S - 1)], dtype=np.int64)
    got = oracle.attn_bwd_dq_rows(bits(x["q"]), bits(x["k"]), bits(x["v"]), bits(dout), None, None,
                                  0.125, rows)
    k = x["k"][0, :, 0].double().numpy()
    v = x["v"][0, :, 0].double().numpy()
    M = k.T @ (v - v.mean(0)) / S          # D x D: sum_j k_j (v_j - vbar)^T / S
    do = dout[0, rows[:, 2], 0].double().numpy()
    want = 0.125 * do @ M.T
    assert np.abs(got - want).max() < 1e-11


def test_sensitivity_sums_bound_and_reduce():
    """The rounding-sensitivity sums (tq, tk, tv) leave the gradients
    untouched, bound them (|sum of terms| <= sum of |terms|), and reduce to
    the gradient itself where every term is non-negative (dout >= 0 gives
    tv = dv)."""
    B, S, H, D = 1, 37, 2, 64
    x = W.make_random(B, S, H, D, seed=761)
    dout = W.randn_bf16((B, S, H, D), 763)
    seg = W.random_segments(B, S, 765, "packed").numpy()
    b = [bits(x["q"]), bits(x["k"]), bits(x["v"])]
    g0 = oracle.attn_bwd(*b, bits(dout), seg, seg.copy(), 0.2)
    g1 = oracle.attn_bwd(*b, bits(dout), seg, seg.copy(), 0.2, sensitivity=True)
    for a, c in zip(g0, g1[:3]):
        assert np.array_equal(a, c)
    for g, t in zip(g1[:3], g1[3:]):
        assert np.all(t >= np.abs(g) - 1e-12)
    pos = dout.abs()
    _, _, dv, _, _, tv = oracle.attn_bwd(*b, bits(pos), seg, seg.copy(), 0.2, sensitivity=True)
    assert np.allclose(tv, dv, rtol=1e-13, atol=0)


def test_dq_rows_sensitivity_matches_dense():
    B, S, H, D = 1, 45, 2, 64
    x = W.make_random(B, S, H, D, seed=771)
    dout = W.randn_bf16((B, S, H, D), 773)
    seg = W.random_segments(B, S, 775, "interleaved").numpy()
    b = [bits(x["q"]), bits(x["k"]), bits(x["v"]), bits(dout)]
    dq, _, _, tq, _, _ = oracle.attn_bwd(*b, seg, seg.copy(), 0.2, sensitivity=True)
    rows = np.array([(0, h, i) for h in range(H) for i in range(S)], dtype=np.int64)
    r, t = oracle.attn_bwd_dq_rows(*b, seg, seg.copy(), 0.2, rows, sensitivity=True)
    assert np.allclose(r, dq[0, rows[:, 2], rows[:, 1]], rtol=0, atol=1e-13)
    assert np.allclose(t, tq[0, rows[:, 2], rows[:, 1]], rtol=1e-12, atol=1e-14)


# ---- the sensitivity sums, characterised from above ----------------------------------
# A separately written fp64 model of the gradient in which every term that a
# finite-precision implementation rounds carries its own relative
# perturbation: term j of dq_id (scale dS_ij k_jd), term i of dk_jd
# (scale dS_ij q_id) and of dv_jd (P_ij dout_id), and term (j, d') of out_id'
# (P_ij v_jd') where out feeds delta_i = dout_i . out_i.  Every output is
# linear in each single perturbation, so one-hot evaluations give its
# partial derivatives exactly, and the sign-aligned first-order deviation for
# perturbations of size u is u times the sum of their magnitudes.  tk and tv
# must equal that sum; so must tq where every k_jd has one sign (its P E term
# takes |k_jd| inside the sum over j, a bound on |sum_j P_ij k_jd| E_i),
# and tq must bound it otherwise.

def _perturbed_grads(q, k, v, do, valid, scale, eq, ek, ev, eo):
    """dq, dk, dv [S, D] of one (b, h) with relative term perturbations:
    eq[i, j, d] on term j of dq[i, d]; ek[j, i, d] on term i of dk[j, d];
    ev[j, i, d] on term i of dv[j, d]; eo[i, j, d] on term (j, d) of out[i, d]
    as it enters delta_i."""
    S = q.shape[0]
    P = np.zeros((S, S))
    for i in range(S):
        js = np.nonzero(valid[i])[0]
        if len(js) == 0:
            continue
        s = np.array([scale * float(np.dot(q[i], k[j])) for j in js])
        w = np.exp(s - s.max())
        P[i, js] = w / w.sum()
    dP = do @ v.T
    out_terms = P[:, :, None] * v[None, :, :] * (1.0 + eo)
    delta = np.array([float(np.sum(do[i][None, :] * out_terms[i])) for i in range(S)])
    dS = P * (dP - delta[:, None])
    dq = (scale * dS[:, :, None] * k[None, :, :] * (1.0 + eq)).sum(axis=1)
    dk = (scale * dS.T[:, :, None] * q[None, :, :] * (1.0 + ek)).sum(axis=1)
    dv = (P.T[:, :, None] * do[None, :, :] * (1.0 + ev)).sum(axis=1)
    return dq, dk, dv


def _first_order_sums(q, k, v, do, valid, scale):
    """Per element of dq, dk, dv: sum over every term perturbation of
    |d output / d perturbation|, from one-hot evaluations of the model."""
    S, D = q.shape
    zero = np.zeros((S, S, D))
    base = _perturbed_grads(q, k, v, do, valid, scale, zero, zero, zero, zero)
    sums = [np.zeros((S, D)) for _ in range(3)]
    for slot in range(4):
        for idx in np.ndindex(S, S, D):
            e = [zero, zero, zero, zero]
            one = np.zeros((S, S, D))
            one[idx] = 1.0
            e[slot] = one
            got = _perturbed_grads(q, k, v, do, valid, scale, *e)
            for n in range(3):
                sums[n] += np.abs(got[n] - base[n])
    return sums


@pytest.mark.parametrize("case", ["unmasked_signed", "packed_signed", "packed_nonneg_k"])
def test_sensitivity_sums_equal_first_order_deviation(case):
    B, S, H, D = 1, 7, 2, 5
    scale = 0.375
    x = W.make_random(B, S, H, D, seed=781)
    dout = W.randn_bf16((B, S, H, D), 783)
    if case == "packed_nonneg_k":
        x["k"] = x["k"].abs()
    seg = None
    if case != "unmasked_signed":
        seg = torch.tensor([[2, 2, 2, 0, -5, -5, 2]], dtype=torch.int32)
    s = None if seg is None else seg.numpy()
    dq, dk, dv, tq, tk, tv = oracle.attn_bwd(bits(x["q"]), bits(x["k"]), bits(x["v"]), bits(dout), s,
                                             None if s is None else s.copy(), scale, sensitivity=True)
    for h in range(H):
        f = lambda t: t[0, :, h].double().numpy()
        q, k, v, do = f(x["q"]), f(x["k"]), f(x["v"]), f(dout)
        if seg is None:
            valid = np.ones((S, S), dtype=bool)
        else:
            sg = seg[0].numpy()
            valid = (sg[:, None] == sg[None, :]) & (sg[:, None] != 0)
        zero = np.zeros((S, S, D))
        g = _perturbed_grads(q, k, v, do, valid, scale, zero, zero, zero, zero)
        for a, b in zip(g, (dq, dk, dv)):
            assert np.abs(a - b[0, :, h]).max() < 1e-12
        sq, sk, sv = _first_order_sums(q, k, v, do, valid, scale)
        close = lambda a, b: np.all(np.abs(a - b) <= 1e-9 * np.abs(b) + 1e-13)
        assert close(tk[0, :, h], sk), (h, np.abs(tk[0, :, h] - sk).max())
        assert close(tv[0, :, h], sv), (h, np.abs(tv[0, :, h] - sv).max())
        if case == "packed_nonneg_k":
            assert close(tq[0, :, h], sq), (h, np.abs(tq[0, :, h] - sq).max())
        else:
            assert np.all(tq[0, :, h] >= sq * (1 - 1e-12) - 1e-13)
            assert np.any(tq[0, :, h] > sq * (1 + 1e-6))  # signed k: a strict bound somewhere
