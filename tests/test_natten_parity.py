"""GPU parity of 3D neighbourhood attention (vdx_natten3d_fwd through the C
ABI) against the fp64 oracle on the same seeded bf16 inputs.

Small grids are compared element by element: x extents below, at and above
the 32-query brick and the 48-key row (ragged tails), y extents that are not
multiples of the 8-row brick, single-frame grids, windows from 1 to 13 and
windows wider than their axis (whole axis).  The VAE-decoder-sized grid is
compared on sampled rows (grid corners, edges and random interior rows) and,
on every row, against the Q = 0 closed form: the mean of V over the window,
with lse = ln(window volume).  Tolerances are those of the segment-masked
path (tests/gpu_helpers.py).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LSE_ATOL, REL_L2, check_full, check_rows, out_tol

pytestmark = pytest.mark.gpu


def run_gpu(x, grid, window, scale):
    import spatiotemporal_attention_amd as vdx
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    out, lse = vdx.natten3d_fwd(d["q"], d["k"], d["v"], grid, window, scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_oracle(x, grid, window, scale, rows=None):
    """(out, lse, sens): sens is the rounding sensitivity sum over the window
    of P_ij |v_jd| per output element."""
    B, S, H, D = x["q"].shape
    sens = np.zeros((B, S, H, D) if rows is None else (len(rows), D), dtype=np.float64)
    out, lse = oracle.natten3d_fwd(W.bf16_bits(x["q"]), W.bf16_bits(x["k"]), W.bf16_bits(x["v"]),
                                   grid, window, float(np.float32(scale)), rows=rows, sens=sens)
    return out, lse, sens


CASES = [
    # (grid, window, H, D)
    ((1, 1, 1), (1, 1, 1), 1, 64),
    ((1, 3, 5), (3, 3, 3), 2, 64),
    ((2, 8, 32), (3, 3, 3), 2, 128),
    ((3, 9, 33), (3, 5, 7), 1, 128),
    ((2, 7, 63), (1, 7, 13), 2, 64),
    ((2, 8, 64), (3, 3, 11), 1, 128),
    ((1, 12, 65), (1, 11, 11), 1, 128),
    ((3, 5, 100), (3, 3, 13), 1, 64),
    ((4, 6, 40), (5, 9, 9), 1, 128),
    ((2, 17, 24), (3, 31, 5), 1, 64),     # y window wider than the axis
    ((5, 4, 12), (9, 3, 21), 1, 128),     # x window wider than the axis (whole axis)
    ((6, 10, 70), (11, 11, 11), 1, 128),
    # x extents at, below and above the 48-key row the kernel stages per key row
    ((2, 9, 48), (3, 3, 13), 1, 128),
    ((1, 8, 47), (1, 5, 11), 2, 64),
    ((2, 10, 81), (3, 7, 13), 1, 128),
]


@pytest.mark.parametrize("grid,window,H,D", CASES, ids=[f"{g}-{w}-H{h}-D{d}" for g, w, h, d in CASES])
def test_grid_and_window_sweep(need_gpu, grid, window, H, D):
    S = grid[0] * grid[1] * grid[2]
    seed = 9000 + S + sum(window)
    x = W.make_random(2, S, H, D, seed=seed)
    scale = 1.0 / math.sqrt(D)
    print(f"case natten grid={grid} window={window} H={H} D={D}", flush=True)
    out_g, lse_g = run_gpu(x, grid, window, scale)
    out_o, lse_o, sens_o = run_oracle(x, grid, window, scale)
    check_full(out_g, lse_g, out_o, lse_o, np.ones((2, S), dtype=bool), sens_o)


def test_tiny_workload_full(need_gpu):
    w = W.NATTEN_WORKLOADS["natten_tiny"]
    x = W.make_natten_inputs(w)
    print(f"case {w.name}", flush=True)
    out_g, lse_g = run_gpu(x, w.grid, w.window, w.scale)
    out_o, lse_o, sens_o = run_oracle(x, w.grid, w.window, w.scale)
    check_full(out_g, lse_g, out_o, lse_o, np.ones((w.B, w.S), dtype=bool), sens_o)


def test_peaky_scores(need_gpu):
    grid, window = (3, 9, 40), (3, 5, 11)
    S = 1080
    x = W.make_random(1, S, 2, 128, seed=9901, sigma_qk=3.0)
    print("case natten peaky", flush=True)
    out_g, lse_g = run_gpu(x, grid, window, 1.0 / math.sqrt(128))
    out_o, lse_o, sens_o = run_oracle(x, grid, window, 1.0 / math.sqrt(128))
    check_full(out_g, lse_g, out_o, lse_o, np.ones((1, S), dtype=bool), sens_o)


def test_repeat_and_head_split_bit_identical(need_gpu):
    grid, window = (3, 9, 40), (3, 5, 11)
    x = W.make_random(2, 1080, 3, 64, seed=9911)
    a = run_gpu(x, grid, window, 0.125)
    b = run_gpu(x, grid, window, 0.125)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])
    xs = {n: t[1:2, :, 1:2].contiguous() for n, t in x.items()}
    c = run_gpu(xs, grid, window, 0.125)
    assert torch.equal(c[0].view(torch.int16), a[0][1:2, :, 1:2].contiguous().view(torch.int16))
    assert torch.equal(c[1], a[1][1:2, 1:2])


def _box_mean(v, grid, window):
    """Mean of v [S, D] over every query's window, via 3D prefix sums (fp64)."""
    NT, NH, NW = grid
    KT, KH, KW = window
    D = v.shape[-1]
    g = v.reshape(NT, NH, NW, D)
    P = np.zeros((NT + 1, NH + 1, NW + 1, D))
    P[1:, 1:, 1:] = g.cumsum(0).cumsum(1).cumsum(2)

    def starts(n, k):
        ke = min(k, n)
        c = np.arange(n)
        return np.clip(c - k // 2, 0, n - ke), ke

    st, kt = starts(NT, KT)
    sy, kh = starts(NH, KH)
    sx, kw = starts(NW, KW)
    t0 = st[:, None, None]; y0 = sy[None, :, None]; x0 = sx[None, None, :]
    t1, y1, x1 = t0 + kt, y0 + kh, x0 + kw
    box = (P[t1, y1, x1] - P[t0, y1, x1] - P[t1, y0, x1] - P[t1, y1, x0]
           + P[t0, y0, x1] + P[t0, y1, x0] + P[t1, y0, x0] - P[t0, y0, x0])
    return box.reshape(NT * NH * NW, D) / (kt * kh * kw), kt * kh * kw


def test_vae_decoder_sampled_rows(need_gpu):
    w = W.NATTEN_WORKLOADS["natten_vae_decoder"]
    x = W.make_natten_inputs(w)
    print(f"case {w.name}: sampled rows", flush=True)
    out_g, lse_g = run_gpu(x, w.grid, w.window, w.scale)
    NT, NH, NW = w.grid
    rng = np.random.default_rng(5)
    corners = [(t, y, xx) for t in (0, 1, NT // 2, NT - 1) for y in (0, 5, 7, 8, NH - 1)
               for xx in (0, 5, 31, 32, 33, NW - 6, NW - 1)]
    idx = sorted({(t * NH + y) * NW + xx for t, y, xx in corners} |
                 set(int(i) for i in rng.choice(w.S, 256, replace=False)))
    rows = np.array([(0, h, i) for h in range(w.H) for i in idx], dtype=np.int64)
    out_o, lse_o, sens_o = run_oracle(x, w.grid, w.window, w.scale, rows=rows)
    st = check_rows(out_g, lse_g, rows, out_o, lse_o, np.ones((w.B, w.S), dtype=bool), sens_o)
    print(st, flush=True)


def test_vae_decoder_zero_query_closed_form_every_row(need_gpu):
    w = W.NATTEN_WORKLOADS["natten_vae_decoder"]
    x = W.make_natten_inputs(w)
    x["q"] = torch.zeros_like(x["q"])
    print(f"case {w.name}: Q=0 closed form", flush=True)
    out_g, lse_g = run_gpu(x, w.grid, w.window, w.scale)
    v = x["v"].double().numpy()
    for h in range(w.H):
        mean, vol = _box_mean(v[0, :, h], w.grid, w.window)
        sens, _ = _box_mean(np.abs(v[0, :, h]), w.grid, w.window)  # uniform weights: mean |v|
        o = out_g[0, :, h].float().numpy()
        err = np.abs(o - mean)
        assert (err / out_tol(mean, sens)).max() <= 1.0, (h, err.max())
        assert np.linalg.norm(o - mean) / np.linalg.norm(mean) <= REL_L2
        assert np.abs(lse_g[0, h].numpy() - math.log(vol)).max() <= LSE_ATOL
