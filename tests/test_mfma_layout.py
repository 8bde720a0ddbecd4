"""GPU probes of the gfx950 instruction semantics the attention kernel relies
on (all single-wave, in-bounds, on buffers of fixed size).  The kernel assumes, for v_mfma_f32_32x32x16_bf16 (D = A B + C, A 32x16,
B 16x32), that lane l holds A[l%32][8*(l//32)+e] and B[8*(l//32)+e][l%32]
(e = 0..7), and accumulator register r holds D[8*(r//4)+4*(l//32)+r%4][l%32].
"""
import ctypes
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "probes", "liblayout_probe.so")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probes(need_gpu):
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"probe library not built: {PROBE_LIB}")
    lib = ctypes.CDLL(PROBE_LIB)
    for name in ("probe_mfma32", "probe_permlane32_swap", "probe_trans", "probe_load_lds",
                 "probe_read_tr"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_mfma_32x32x16_bf16_layout(probes):
    g = torch.Generator().manual_seed(0)
    A = torch.randint(-8, 9, (32, 16), generator=g).float()
    Bm = torch.randint(-8, 9, (16, 32), generator=g).float()
    a_regs = torch.empty(64, 8)
    b_regs = torch.empty(64, 8)
    for l in range(64):
        for e in range(8):
            a_regs[l, e] = A[l % 32, 8 * (l // 32) + e]
            b_regs[l, e] = Bm[8 * (l // 32) + e, l % 32]
    a_d = a_regs.bfloat16().cuda()
    b_d = b_regs.bfloat16().cuda()
    acc = torch.zeros(64, 16, device="cuda")
    print(f"probe_mfma32 start", flush=True)
    assert probes.probe_mfma32(ctypes.c_void_p(a_d.data_ptr()), ctypes.c_void_p(b_d.data_ptr()),
                               ctypes.c_void_p(acc.data_ptr()), _stream()) == 0
    torch.cuda.synchronize()
    acc = acc.cpu()
    Dm = torch.empty(32, 32)
    for l in range(64):
        for r in range(16):
            Dm[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = acc[l, r]
    assert torch.equal(Dm, A @ Bm), "accumulator/operand layout differs from the assumed one"


def test_permlane32_swap_exchanges_halves(probes):
    x = torch.arange(64, dtype=torch.int32, device="cuda") + 1000
    r0 = torch.zeros_like(x)
    r1 = torch.zeros_like(x)
    assert probes.probe_permlane32_swap(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(r0.data_ptr()),
                                        ctypes.c_void_p(r1.data_ptr()), _stream()) == 0
    torch.cuda.synchronize()
    r0 = r0.cpu().numpy() - 1000
    r1 = r1.cpu().numpy() - 1000
    print("permlane32_swap r0:", r0.tolist())
    print("permlane32_swap r1:", r1.tolist())
    for l in range(64):
        assert (l ^ 32) in (r0[l], r1[l])


def test_exp2_and_log2_builtins_accuracy(probes):
    xs = np.concatenate([np.linspace(-126, 40, 200001), np.linspace(-1, 1, 100001)]).astype(np.float32)
    x = torch.from_numpy(xs).cuda()
    ye = torch.empty_like(x)
    pos = torch.from_numpy(np.abs(xs) + np.float32(1e-3)).cuda()
    yl_dummy = torch.empty_like(x)
    ylog = torch.empty_like(x)
    ye2 = torch.empty_like(x)
    n = xs.size
    assert probes.probe_trans(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(ye.data_ptr()),
                              ctypes.c_void_p(yl_dummy.data_ptr()), n, _stream()) == 0
    assert probes.probe_trans(ctypes.c_void_p(pos.data_ptr()), ctypes.c_void_p(ye2.data_ptr()),
                              ctypes.c_void_p(ylog.data_ptr()), n, _stream()) == 0
    torch.cuda.synchronize()
    ye = ye.cpu().numpy().astype(np.float64)
    want = np.exp2(xs.astype(np.float64))
    rel = np.abs(ye - want) / want
    print(f"v_exp_f32 max rel err {rel.max():.3e} ({rel.max() / 2**-23:.2f} ulp)")
    assert rel.max() < 4 * 2.0 ** -23
    pv = pos.cpu().numpy().astype(np.float64)
    yl = ylog.cpu().numpy().astype(np.float64)
    wl = np.log2(pv)
    err = np.abs(yl - wl)
    bound = np.maximum(np.abs(wl), 1.0) * 4 * 2.0 ** -23
    print(f"v_log_f32 max abs err {err.max():.3e}")
    assert np.all(err <= bound)


def test_global_load_lds_dwordx4_places_lane_chunks_contiguously(probes):
    """global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l."""
    src = torch.arange(4 * 64, dtype=torch.int32, device="cuda") * 7 + 3
    perm = torch.tensor([(37 * l + 11) % 64 for l in range(64)], dtype=torch.int32, device="cuda")
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")
    assert probes.probe_load_lds(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(perm.data_ptr()),
                                 ctypes.c_void_p(out.data_ptr()), _stream()) == 0
    torch.cuda.synchronize()
    out = out.cpu().numpy().view(np.uint32)
    srcn = src.cpu().numpy().view(np.uint32)
    pn = perm.cpu().numpy()
    want = np.full(1024, 0xDEADBEEF, dtype=np.uint32)
    for l in range(64):
        want[128 + 4 * l: 128 + 4 * l + 4] = srcn[4 * pn[l]: 4 * pn[l] + 4]
    assert np.array_equal(out, want)


@pytest.mark.parametrize("pattern", ["rows_of_4", "strided_rows"])
def test_ds_read_b64_tr_b16_semantics(probes, pattern):
    """Within each 16-lane group, with X[j][k] the k-th 16-bit element at lane
    j's address, lane i receives Y[i][e] = X[4e + i//4][i % 4]."""
    if pattern == "rows_of_4":
        addr = [4 * l for l in range(64)]
    else:
        addr = [(l % 16) * 64 + (l // 16) * 4 + 1024 * (l % 3 == 0) for l in range(64)]
        addr = [a & ~3 for a in addr]
    a_d = torch.tensor(addr, dtype=torch.int32, device="cuda")
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    assert probes.probe_read_tr(ctypes.c_void_p(a_d.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(64, 4)
    for l in range(64):
        grp, i = l // 16, l % 16
        for e in range(4):
            src_lane = 16 * grp + 4 * e + i // 4
            assert got[l, e] == addr[src_lane] + (i % 4), (l, e)
