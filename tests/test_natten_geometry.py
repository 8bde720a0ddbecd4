"""Geometry of the neighbourhood-attention kernel, on the CPU.

A restatement of the kernel's index rules (natten_fwd_kernel.hip): the
per-call brick shape (BT frames x 8/BT rows x 32 columns, BT in 1, 2, 4, 8),
each wave's BT x 8/BT x 4 patch of it, the walk over the key rows of a
brick's window union two rows per step, the 48-key rows staged from the
brick's first window start rounded down to 4, each wave's 16-key block
within each row, the clamp of keys past the grid row, the LDS slot layout,
and the work-item decode (XCD renumbering, then bricks counted from the
middle outward).
For many grids and windows it checks what the kernel relies on: every
query's window lies inside its wave's 16-key block and inside the walked
rows, every copied key and every LDS access is in bounds, the two copying
waves of a row pair fetch rows 2a and 2a + 1 (or repeat row 2a), and the
decode visits every brick once.  No GPU is involved.
"""
import itertools

import pytest

ROW_KEYS = 48        # keys of one staged key row
BRICK_ROWS = 8       # (t, y) query rows of a brick
BRICK_X = 32         # query columns of a brick
PATCH_X = 4          # query columns of a wave
BLOCK_KEYS = 16      # keys of one row a wave multiplies


def win_start(c, k, n):
    keff = min(k, n)
    return min(max(c - k // 2, 0), n - keff)


def swap23(x):
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1)


def brick_frames(NT, NH, KT, KH):
    kt, kh = min(KT, NT), min(KH, NH)
    best, best_rows, best_q = 1, 0, 1
    for bt in (1, 2, 4, 8):
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
            xw = min(x0 + PATCH_X * wave, NW - 1)
            boff = min(win_start(xw, KW, NW) - x0k, ROW_KEYS - BLOCK_KEYS)
            assert 0 <= boff <= ROW_KEYS - BLOCK_KEYS
            for lane in range(64):
                lr, g = lane & 31, lane >> 5
                # K operand row (block key swap23(lr): row m >> 4, key m & 15)
                # and the transposed V rows of both k-steps, inside the slot
                m = swap23(lr)
                assert 0 <= (m >> 4) * ROW_KEYS + boff + (m & 15) < 2 * ROW_KEYS
                key = boff + 8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)
                for kst in range(2):
                    assert key + kst * ROW_KEYS + 4 < 2 * ROW_KEYS
                    assert key % 4 == (key + kst * ROW_KEYS) % 4  # one V swizzle base serves both rows
                tq = t0 + lr // (PATCH_X * BY)
                yq = y0 + (lr // PATCH_X) % BY
                xq = x0 + PATCH_X * wave + lr % PATCH_X
                if not (tq < NT and yq < NH and xq < NW):
                    continue
                xs, ys, tsq = win_start(xq, KW, NW), win_start(yq, KH, NH), win_start(tq, KT, NT)
                # the lane's x window is its 16-key block's keys whose bit is set in xmask
                assert x0k + boff <= xs and xs + kw <= x0k + boff + BLOCK_KEYS
                xrel = x0k + boff + 8 * g - xs
                in_block = [e for e in range(8) if 0 <= xrel + e < kw]
                assert len(in_block) == sum(1 for x in range(x0k + boff + 8 * g, x0k + boff + 8 * g + 8)
                                            if xs <= x < xs + kw)
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
@pytest.mark.parametrize("BT", [None, 1, 2, 4, 8], ids=["chosen", "bt1", "bt2", "bt4", "bt8"])
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
    assert brick_frames(16, 32, 11, 11) == 4   # 14 x 12 key rows beat 11 x 18 (ties with 12 x 14: more frames)
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
