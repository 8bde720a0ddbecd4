"""Geometry of the neighbourhood-attention kernel, on the CPU.

A restatement of the kernel's index rules (natten_fwd_kernel.hip): the
per-call brick shape (BT frames x 8/BT rows x 32 columns), the walk over the
key rows of a brick's window union two rows per step, the 48-key rows staged
from the brick's first window start rounded down to 4, each wave's 32-key
block within a row, the clamp of keys past the grid row, the LDS slot
layout, and the work-item decode (XCD renumbering, then bricks counted from
the middle outward).
For many grids and windows it checks what the kernel relies on: every
query's window lies inside its wave's 32-key block and inside the walked
rows, every copied key and every LDS access is in bounds, the two copying
waves of a row pair fetch rows 2a and 2a + 1 (or repeat row 2a), and the
decode visits every brick once.  No GPU is involved.
"""
import itertools

import pytest

ROW_KEYS = 48        # keys of one staged key row
BRICK_ROWS = 8       # (t, y) query rows of a brick
BRICK_X = 32         # query columns of a brick


def win_start(c, k, n):
    keff = min(k, n)
    return min(max(c - k // 2, 0), n - keff)


def swap23(x):
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1)


def brick_frames(NT, NH, KT, KH):
    kt, kh = min(KT, NT), min(KH, NH)
    best, best_rows, best_q = 1, 0, 1
    for bt in (1, 2, 4):
        by = BRICK_ROWS // bt
        rows = min(bt + kt - 1, NT) * min(by + kh - 1, NH)
        q = min(bt, NT) * min(by, NH)
        if bt == 1 or rows * best_q <= best_rows * q:
            best, best_rows, best_q = bt, rows, q
    return best


def center_out(k, n):
    if n % 2 == 0:
        return n // 2 + k // 2 if k & 1 else n // 2 - 1 - k // 2
    return n // 2 - (k + 1) // 2 if k & 1 else n // 2 + k // 2


def check_grid(grid, window, D, BT=None):
    NT, NH, NW = grid
    KT, KH, KW = window
    kt, kh, kw = min(KT, NT), min(KH, NH), min(KW, NW)
    assert kw <= 13, "the kernel rejects wider x windows"
    BT = brick_frames(NT, NH, KT, KH) if BT is None else BT
    BY = BRICK_ROWS // BT
    pairs = BY // 2
    row_bytes = 2 * D
    rows_per_load = 1024 // row_bytes
    loads = 2 * ROW_KEYS * row_bytes // 1024 // 4
    assert loads * 2 * rows_per_load == ROW_KEYS
    for bt, by, bx in itertools.product(range(-(-NT // BT)), range(-(-NH // BY)), range(-(-NW // BRICK_X))):
        t0, y0, x0 = bt * BT, by * BY, bx * BRICK_X
        ts = win_start(t0, KT, NT)
        nt = win_start(min(t0 + BT - 1, NT - 1), KT, NT) + kt - ts
        ylo = win_start(y0, KH, NH)
        ny = win_start(min(y0 + BY - 1, NH - 1), KH, NH) + kh - ylo
        n_rows = nt * ny
        n_steps = (n_rows + 1) // 2
        x0k = win_start(x0, KW, NW) & ~3
        for r in range(n_rows):
            assert 0 <= ts + r // ny < NT and 0 <= ylo + r % ny < NH
        for wave in range(8):
            xw = min(x0 + 16 * (wave & 1), NW - 1)
            boff = min((win_start(xw, KW, NW) & ~3) - x0k, ROW_KEYS - 32)
            assert 0 <= boff <= ROW_KEYS - 32 and boff % 4 == 0
            for lane in range(64):
                lr = lane & 31
                # K operand row and transposed V rows inside the two-row slot
                for j in range(2):
                    assert j * ROW_KEYS + boff + swap23(lr) < 2 * ROW_KEYS
                key = boff + 8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)
                for kst in range(4):
                    assert key + (kst >> 1) * ROW_KEYS + (kst & 1) * 16 + 4 < 2 * ROW_KEYS
                tq = t0 + (wave >> 1) // pairs
                yq = y0 + 2 * ((wave >> 1) % pairs) + (lr >> 4)
                xq = x0 + 16 * (wave & 1) + (lr & 15)
                if not (tq < NT and yq < NH and xq < NW):
                    continue
                xs, ys, tsq = win_start(xq, KW, NW), win_start(yq, KH, NH), win_start(tq, KT, NT)
                assert x0k + boff <= xs and xs + kw <= x0k + boff + 32
                assert ylo <= ys and ys + kh <= ylo + ny
                assert ts <= tsq and tsq + kt <= ts + nt
            # the rows this wave copies for each step (waves 0-1 of a copying
            # group fetch the step's first row, waves 2-3 its second)
            second = ((wave & 3) >> 1) != 0
            for a in range(n_steps):
                r = 2 * a + (1 if second and 2 * a + 1 < n_rows else 0)
                base = ((ts + r // ny) * NH + (ylo + r % ny)) * NW + x0k
                for jj in range(loads):
                    i = (wave & 3) * loads + jj
                    for lane in range(0, 64, 7):
                        rin = (rows_per_load * i + lane // (D // 8)) % ROW_KEYS
                        xk = min(x0k + rin, NW - 1) - x0k
                        assert 0 <= base + xk < NT * NH * NW
                        assert (wave & 3) * loads * 1024 + jj * 1024 + 16 * lane < 2 * ROW_KEYS * row_bytes
    return BT


CASES = [((1, 1, 1), (1, 1, 1)), ((1, 3, 5), (3, 3, 3)), ((2, 8, 32), (3, 3, 3)), ((3, 9, 33), (3, 5, 7)),
         ((2, 7, 63), (1, 7, 13)), ((1, 12, 65), (1, 11, 11)), ((3, 5, 100), (3, 3, 13)),
         ((2, 17, 24), (3, 31, 5)), ((5, 4, 12), (9, 3, 21)), ((6, 10, 70), (11, 11, 11)),
         ((2, 9, 48), (3, 3, 13)), ((1, 8, 47), (1, 5, 11)), ((16, 32, 64), (11, 11, 11))]


@pytest.mark.parametrize("grid,window", CASES, ids=[f"{g}-{w}" for g, w in CASES])
@pytest.mark.parametrize("BT", [None, 1, 2, 4], ids=["chosen", "bt1", "bt2", "bt4"])
def test_windows_covered_and_accesses_in_bounds(grid, window, BT):
    check_grid(grid, window, 128, BT)


def test_x_widths_and_frame_counts():
    for NW in range(1, 100, 3):
        for KW in (1, 5, 11, 13):
            check_grid((1, 5, NW), (1, 3, KW), 64)
    for NT in range(1, 10):
        for KT in (1, 3, 11):
            check_grid((NT, 9, 40), (KT, 5, 11), 128)


def test_brick_shape_choice():
    assert brick_frames(16, 32, 11, 11) == 4   # 14 x 12 key rows beat 11 x 18
    assert brick_frames(1, 32, 11, 11) == 1    # a single frame
    assert brick_frames(16, 32, 1, 11) == 1    # a one-frame t window


@pytest.mark.parametrize("nbx,nby,nbt,H", [(2, 16, 4, 8), (1, 5, 3, 2), (3, 1, 7, 1), (2, 8, 1, 3)])
def test_work_item_decode_visits_every_brick_once(nbx, nby, nbt, H):
    n = nbx * nby * nbt * H
    xcds = 8
    per, rem = n // xcds, n % xcds
    # workgroup w runs on XCD w % 8; the XCDs take consecutive work items
    lids = [(w % xcds) * per + min(w % xcds, rem) + w // xcds for w in range(n)]
    assert sorted(lids) == list(range(n))
    seen = set()
    for lid in lids:
        bx = lid % nbx
        by = center_out((lid // nbx) % nby, nby)
        bt = center_out((lid // (nbx * nby)) % nbt, nbt)
        seen.add((bx, by, bt, lid // (nbx * nby * nbt)))
    assert len(seen) == n
    assert all(0 <= by < nby and 0 <= bt < nbt for _, by, bt, _ in seen)
