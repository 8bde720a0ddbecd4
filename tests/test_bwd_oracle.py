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


@pytest.mark.parametrize("kind", [None, "single", "padded", "packed", "interleaved", "allpad"])
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
