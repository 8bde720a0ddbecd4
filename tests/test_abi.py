"""The C ABI boundary (include/vdx_attn.h): the library loads, exports every
declared function, reports versions and status strings, and validates
arguments before any HIP call -- all checkable without a GPU, since
validation never dereferences the (fake, aligned) device addresses used here.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vdx_attn.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vdx_[a-z0-9_]+)\s*\(", src)))


def header_enum():
    src = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(VDX_[A-Z_]+)\s*=\s*(\d+)", src)}


@pytest.fixture(scope="module")
def native():
    from spatiotemporal_attention_amd import _native
    return _native


def test_exports_every_declared_function(native):
    names = header_functions()
    assert names == sorted(["vdx_attn_fwd", "vdx_attn_fwd_ws", "vdx_attn_fwd_workspace_size", "vdx_natten3d_fwd",
                            "vdx_attn_bwd", "vdx_attn_bwd_noalloc", "vdx_attn_bwd_workspace_size",
                            "vdx_rope3d_apply", "vdx_rope3d_attn_fwd", "vdx_rope3d_attn_fwd_ws",
                            "vdx_status_str", "vdx_abi_version"])
    for n in names:
        assert hasattr(native.lib, n), n


def test_abi_version_matches_header(native):
    m = re.search(r"#define\s+VDX_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert native.abi_version() == int(m.group(1))


def test_status_codes_match_header_and_have_names(native):
    enum = header_enum()
    for name, val in enum.items():
        assert getattr(native, name) == val, name
        s = native.status_str(val)
        assert s.startswith(name), (name, s)
    assert native.status_str(12345) == "VDX_ERR_UNKNOWN"


A = 0x10000  # fake, 16-byte aligned device address; never dereferenced here


def call(native, q=A, k=A + 0x100, v=A + 0x200, sq=0, sk=0, out=A + 0x300, lse=A + 0x400,
         B=1, S=128, H=2, D=128, scale=0.125):
    return native.attn_fwd_raw(q, k, v, sq, sk, out, lse, B, S, H, D, scale, 0)


@pytest.mark.parametrize("which", ["q", "k", "v", "out", "lse"])
def test_null_pointer(native, which):
    assert call(native, **{which: 0}) == native.VDX_ERR_NULL_PTR


def test_segment_pair(native):
    assert call(native, sq=A + 0x500) == native.VDX_ERR_SEG_PAIR
    assert call(native, sk=A + 0x500) == native.VDX_ERR_SEG_PAIR


@pytest.mark.parametrize("kw", [dict(B=0), dict(S=0), dict(H=0), dict(B=-1), dict(S=-5),
                                dict(B=2**31 - 1, S=2**31 - 1, H=2**31 - 1),
                                dict(S=1_966_081, sq=A + 0x500, sk=A + 0x600),
                                dict(H=2**18, D=128)])
def test_shape(native, kw):
    assert call(native, **kw) == native.VDX_ERR_SHAPE


@pytest.mark.parametrize("D", [0, 1, 32, 96, 256, -64])
def test_head_dim(native, D):
    assert call(native, D=D) == native.VDX_ERR_HEAD_DIM


@pytest.mark.parametrize("scale", [0.0, -0.1, float("nan"), float("inf"), float("-inf")])
def test_scale(native, scale):
    assert call(native, scale=scale) == native.VDX_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(q=A + 2), dict(k=A + 8), dict(v=A + 4), dict(out=A + 6),
                                dict(lse=A + 0x402), dict(sq=A + 0x501, sk=A + 0x600),
                                dict(sq=A + 0x500, sk=A + 0x602)])
def test_alignment(native, kw):
    assert call(native, **kw) == native.VDX_ERR_ALIGN


def test_validation_order(native):
    # NULL beats everything, then segment pair, shape, head dim, scale, alignment.
    assert call(native, q=0, sq=A, B=0, D=3, scale=-1.0) == native.VDX_ERR_NULL_PTR
    assert call(native, sq=A + 0x500, B=0, D=3, scale=-1.0) == native.VDX_ERR_SEG_PAIR
    assert call(native, B=0, D=3, scale=-1.0, q=A + 1) == native.VDX_ERR_SHAPE
    assert call(native, D=3, scale=-1.0, q=A + 1) == native.VDX_ERR_HEAD_DIM
    assert call(native, scale=-1.0, q=A + 1) == native.VDX_ERR_SCALE


def test_valid_arguments_without_gpu_report_device_error(native):
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this path would launch on fake addresses")
    assert call(native) == native.VDX_ERR_DEVICE


def test_python_wrapper_rejects_bad_tensors():
    import spatiotemporal_attention_amd as vdx
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vdx.attn_fwd(q, q, q)  # CPU tensors are refused before the C call
    with pytest.raises(ValueError):
        vdx.attn_fwd(q.float(), q, q)


@pytest.mark.gpu
def test_error_path_writes_nothing(need_gpu, ):
    from spatiotemporal_attention_amd import _native
    q = torch.randn(1, 64, 1, 64, device="cuda").bfloat16()
    out = torch.full_like(q, 3.0)
    lse = torch.full((1, 1, 64), 5.0, device="cuda")
    rc = _native.attn_fwd_raw(q.data_ptr(), q.data_ptr(), q.data_ptr(), 0, 0, out.data_ptr(),
                              lse.data_ptr(), 1, 64, 1, 64, float("nan"),
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == _native.VDX_ERR_SCALE
    assert torch.all(out == 3.0) and torch.all(lse == 5.0)


@pytest.mark.gpu
def test_runs_on_side_stream(need_gpu):
    import spatiotemporal_attention_amd as vdx
    q = torch.randn(1, 300, 2, 64, device="cuda").bfloat16()
    ref, ref_lse = vdx.attn_fwd(q, q, q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, l = vdx.attn_fwd(q, q, q)
    s.synchronize()
    assert torch.equal(o, ref) and torch.equal(l, ref_lse)


@pytest.mark.gpu
def test_bwd_on_side_stream_with_own_workspace(need_gpu):
    """attn_bwd on a stream other than the current one, allocating its
    workspace and gradients itself: the caller's next allocations on the
    current stream (filled at once) must not land in memory the backward still
    uses, so the gradients equal those of the same call on the current
    stream, bit for bit."""
    import spatiotemporal_attention_amd as vdx
    B, S, H, D = 1, 8192, 4, 128
    g = torch.Generator(device="cuda").manual_seed(31)
    q, k, v, dout = (torch.randn(B, S, H, D, device="cuda", generator=g).bfloat16() for _ in range(4))
    seg = torch.ones(B, S, dtype=torch.int32, device="cuda")
    seg[:, S - 100:] = 0
    out, lse = vdx.attn_fwd(q, k, v, seg, seg)
    ref = vdx.attn_bwd(q, k, v, out, lse, dout, seg, seg)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    got = vdx.attn_bwd(q, k, v, out, lse, dout, seg, seg, stream=s)
    junk = [torch.full((1 << 22,), float("nan"), device="cuda") for _ in range(8)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --- vdx_natten3d_fwd validation (no GPU needed) ----------------------------------
def ncall(native, q=A, k=A + 0x100, v=A + 0x200, out=A + 0x300, lse=A + 0x400, B=1, NT=4, NH=8,
          NW=32, H=2, D=128, KT=3, KH=5, KW=11, scale=0.125):
    return native.natten3d_fwd_raw(q, k, v, out, lse, B, NT, NH, NW, H, D, KT, KH, KW, scale, 0)


@pytest.mark.parametrize("which", ["q", "k", "v", "out", "lse"])
def test_natten_null_pointer(native, which):
    assert ncall(native, **{which: 0}) == native.VDX_ERR_NULL_PTR


@pytest.mark.parametrize("kw", [dict(B=0), dict(NT=0), dict(NH=-1), dict(NW=0), dict(H=0),
                                dict(NT=2048, NH=2048, NW=1024), dict(H=1 << 18)])
def test_natten_shape(native, kw):
    assert ncall(native, **kw) == native.VDX_ERR_SHAPE


@pytest.mark.parametrize("D", [0, 32, 96, 256])
def test_natten_head_dim(native, D):
    assert ncall(native, D=D) == native.VDX_ERR_HEAD_DIM


@pytest.mark.parametrize("kw", [dict(KT=0), dict(KH=4), dict(KW=2), dict(KT=-3), dict(KW=15),
                                dict(KW=21, NW=64)])
def test_natten_window(native, kw):
    assert ncall(native, **kw) == native.VDX_ERR_WINDOW


def test_natten_wide_window_on_narrow_axis_is_accepted(native):
    # min(KW, NW) is what counts: a 21-wide window on an 8-wide grid is the
    # whole axis, so validation passes and only the device check remains
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this path would launch on fake addresses")
    assert ncall(native, KW=21, NW=8) == native.VDX_ERR_DEVICE


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan"), float("inf")])
def test_natten_scale(native, scale):
    assert ncall(native, scale=scale) == native.VDX_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(q=A + 2), dict(k=A + 8), dict(v=A + 4), dict(out=A + 6),
                                dict(lse=A + 2)])
def test_natten_alignment(native, kw):
    assert ncall(native, **kw) == native.VDX_ERR_ALIGN


def test_natten_validation_order(native):
    # NULL beats shape beats head dim beats window beats scale beats alignment
    assert ncall(native, q=0, B=0, D=3, KW=2, scale=-1.0) == native.VDX_ERR_NULL_PTR
    assert ncall(native, B=0, D=3, KW=2, scale=-1.0, k=A + 1) == native.VDX_ERR_SHAPE
    assert ncall(native, D=3, KW=2, scale=-1.0, k=A + 1) == native.VDX_ERR_HEAD_DIM
    assert ncall(native, KW=2, scale=-1.0, k=A + 1) == native.VDX_ERR_WINDOW
    assert ncall(native, scale=-1.0, k=A + 1) == native.VDX_ERR_SCALE
    assert ncall(native, k=A + 1) == native.VDX_ERR_ALIGN


def test_natten_python_wrapper_rejects_bad_grid():
    import spatiotemporal_attention_amd as vdx
    q = torch.zeros(1, 10, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vdx.natten3d_fwd(q, q, q, grid=(2, 2, 2), window=(1, 1, 1))


# --- vdx_attn_fwd_ws validation (no GPU needed) ---------------------------------------
def wcall(native, ws=A + 0x900, ws_bytes=None, q=A, k=A + 0x100, v=A + 0x200, sq=A + 0x500, sk=A + 0x600,
          out=A + 0x300, lse=A + 0x400, B=1, S=128, H=2, D=128, scale=0.125):
    if ws_bytes is None:
        ws_bytes = native.lib.vdx_attn_fwd_workspace_size(B, S, H)
    return native.attn_fwd_ws_raw(q, k, v, sq, sk, out, lse, ws, ws_bytes, B, S, H, D, scale, 0)


def test_fwd_workspace_size(native):
    size = native.lib.vdx_attn_fwd_workspace_size
    r = lambda x: (x + 255) // 256 * 256
    # counters, then per batch int4 tile summaries, block counts, block orders,
    # then 256 part records of the split last round (256 rows x (128 + 2) fp32)
    recs = 256 * 256 * (128 + 2) * 4
    assert size(1, 61440, 16) == 256 + r(16 * 960) + r(4 * 240) + r(4 * 240) + recs
    assert size(2, 17920, 24) == 256 + r(16 * 2 * 280) + r(4 * 2 * 70) + r(4 * 2 * 70) + recs
    assert size(1, 1, 1) == 256 + 256 + 256 + 256 + recs
    assert size(3, 1000, 1) == size(3, 1000, 40)  # H does not enter
    for bad in ((0, 1, 1), (1, 0, 1), (1, 1, 0)):
        assert size(*bad) == 0


def test_fwd_ws_validation(native):
    # the checks of vdx_attn_fwd, in its order, then the workspace (masked calls only)
    assert wcall(native, q=0, ws=0) == native.VDX_ERR_NULL_PTR
    assert wcall(native, sk=0, ws=0) == native.VDX_ERR_SEG_PAIR
    assert wcall(native, B=0, ws=0) == native.VDX_ERR_SHAPE
    assert wcall(native, D=96, ws=0) == native.VDX_ERR_HEAD_DIM
    assert wcall(native, scale=0.0, ws=0) == native.VDX_ERR_SCALE
    assert wcall(native, sq=A + 0x502, ws=0) == native.VDX_ERR_ALIGN
    assert wcall(native, ws=0) == native.VDX_ERR_WORKSPACE
    assert wcall(native, ws=A + 0x908) == native.VDX_ERR_WORKSPACE
    need = native.lib.vdx_attn_fwd_workspace_size(1, 128, 2)
    assert wcall(native, ws_bytes=need - 1) == native.VDX_ERR_WORKSPACE
    # without segment IDs a workspace is optional, but one that is given is checked
    assert wcall(native, sq=0, sk=0, ws_bytes=need - 1) == native.VDX_ERR_WORKSPACE
    assert wcall(native, sq=0, sk=0, ws=A + 0x908) == native.VDX_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert wcall(native) == native.VDX_ERR_DEVICE
        assert wcall(native, sq=0, sk=0, ws=0, ws_bytes=0) == native.VDX_ERR_DEVICE
        assert wcall(native, sq=0, sk=0) == native.VDX_ERR_DEVICE


# --- vdx_attn_bwd validation (no GPU needed) -------------------------------------
def bcall(native, q=A, k=A + 0x100, v=A + 0x200, sq=0, sk=0, out=A + 0x300, lse=A + 0x400,
          dout=A + 0x500, dq=A + 0x600, dk=A + 0x700, dv=A + 0x800, ws=A + 0x900, ws_bytes=None,
          B=1, S=128, H=2, D=128, scale=0.125):
    if ws_bytes is None:
        ws_bytes = max(native.attn_bwd_workspace_size(B, S, H), 0)
    return native.attn_bwd_raw(q, k, v, sq, sk, out, lse, dout, dq, dk, dv, ws, ws_bytes,
                               B, S, H, D, scale, 0)


def test_bwd_workspace_size(native):
    # two fp32 rows per (b, h), S padded to a multiple of 64, then per batch
    # four int32 per 128-row block (counts and orders of both sweeps)
    assert native.attn_bwd_workspace_size(1, 75600, 40) == 2 * 40 * 75648 * 4 + 4 * 591 * 4
    assert native.attn_bwd_workspace_size(2, 1, 3) == 2 * 6 * 64 * 4 + 2 * 4 * 1 * 4
    assert native.attn_bwd_workspace_size(1, 64, 1) == 2 * 64 * 4 + 4 * 1 * 4
    for bad in ((0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 2**31 - 1, 1)):
        assert native.attn_bwd_workspace_size(*bad) == 0


@pytest.mark.parametrize("which", ["q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv"])
def test_bwd_null_pointer(native, which):
    assert bcall(native, **{which: 0}) == native.VDX_ERR_NULL_PTR


def test_bwd_segment_pair(native):
    assert bcall(native, sq=A + 0xa00) == native.VDX_ERR_SEG_PAIR
    assert bcall(native, sk=A + 0xa00) == native.VDX_ERR_SEG_PAIR


@pytest.mark.parametrize("kw", [dict(B=0), dict(S=0), dict(H=-1), dict(S=2**31 - 64),
                                dict(S=896_001, sq=A + 0xa00, sk=A + 0xb00),
                                dict(H=2**18, D=128)])
def test_bwd_shape(native, kw):
    kw.setdefault("ws_bytes", 1 << 40)
    assert bcall(native, **kw) == native.VDX_ERR_SHAPE


@pytest.mark.parametrize("D", [0, 32, 96, 256])
def test_bwd_head_dim(native, D):
    assert bcall(native, D=D) == native.VDX_ERR_HEAD_DIM


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan"), float("inf")])
def test_bwd_scale(native, scale):
    assert bcall(native, scale=scale) == native.VDX_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(q=A + 2), dict(dout=A + 0x508), dict(dq=A + 0x604),
                                dict(dk=A + 0x702), dict(dv=A + 0x80a), dict(out=A + 0x306),
                                dict(lse=A + 0x402), dict(sq=A + 0xa01, sk=A + 0xb00)])
def test_bwd_alignment(native, kw):
    assert bcall(native, **kw) == native.VDX_ERR_ALIGN


@pytest.mark.parametrize("kw", [dict(ws=0), dict(ws=A + 0x908), dict(ws_bytes=2 * 2 * 128 * 4 - 4)])
def test_bwd_workspace(native, kw):
    assert bcall(native, **kw) == native.VDX_ERR_WORKSPACE


def test_bwd_validation_order(native):
    # NULL -> segment pair -> shape -> head dim -> scale -> alignment -> workspace
    assert bcall(native, dv=0, sq=A, B=0, D=3, scale=-1.0, ws=0) == native.VDX_ERR_NULL_PTR
    assert bcall(native, sq=A + 0xa00, B=0, D=3, scale=-1.0, ws=0) == native.VDX_ERR_SEG_PAIR
    assert bcall(native, B=0, D=3, scale=-1.0, q=A + 1, ws=0) == native.VDX_ERR_SHAPE
    assert bcall(native, D=3, scale=-1.0, q=A + 1, ws=0) == native.VDX_ERR_HEAD_DIM
    assert bcall(native, scale=-1.0, q=A + 1, ws=0) == native.VDX_ERR_SCALE
    assert bcall(native, q=A + 1, ws=0) == native.VDX_ERR_ALIGN


def test_bwd_valid_arguments_without_gpu_report_device_error(native):
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this path would launch on fake addresses")
    assert bcall(native) == native.VDX_ERR_DEVICE
    # the largest masked sequence passes validation
    assert bcall(native, S=896_000, sq=A + 0xa00, sk=A + 0xb00, ws_bytes=1 << 40) == native.VDX_ERR_DEVICE


def test_bwd_python_wrapper_rejects_bad_tensors():
    import spatiotemporal_attention_amd as vdx
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        vdx.attn_bwd(q, q, q, q, lse, q)  # CPU tensors are refused before the C call


@pytest.mark.gpu
def test_bwd_error_path_writes_nothing(need_gpu):
    import spatiotemporal_attention_amd as vdx
    from spatiotemporal_attention_amd import _native
    q = torch.randn(1, 64, 1, 64, device="cuda").bfloat16()
    lse = torch.zeros(1, 1, 64, device="cuda")
    g = [torch.full_like(q, 3.0) for _ in range(3)]
    ws = torch.full((vdx.attn_bwd_workspace_size(1, 64, 1),), 7, dtype=torch.uint8, device="cuda")
    rc = _native.attn_bwd_raw(q.data_ptr(), q.data_ptr(), q.data_ptr(), 0, 0, q.data_ptr(),
                              lse.data_ptr(), q.data_ptr(), g[0].data_ptr(), g[1].data_ptr(),
                              g[2].data_ptr(), ws.data_ptr(), ws.numel() - 1, 1, 64, 1, 64, 0.125,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == _native.VDX_ERR_WORKSPACE
    assert all(torch.all(t == 3.0) for t in g) and torch.all(ws == 7)


# --- vdx_attn_bwd_noalloc validation (no GPU needed) ------------------------------------
def ncall_bwd(native, q=A, k=A + 0x100, v=A + 0x200, sq=0, sk=0, out=A + 0x300, lse=A + 0x400,
              dout=A + 0x500, dq=A + 0x600, dk=A + 0x700, dv=A + 0x800, B=1, S=128, H=2, D=128, scale=0.125):
    return native.attn_bwd_noalloc_raw(q, k, v, sq, sk, out, lse, dout, dq, dk, dv, B, S, H, D, scale, 0)


def test_bwd_noalloc_validation(native):
    for w in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv"):
        assert ncall_bwd(native, **{w: 0}) == native.VDX_ERR_NULL_PTR, w
    assert ncall_bwd(native, sq=A + 0x900) == native.VDX_ERR_SEG_PAIR
    assert ncall_bwd(native, S=0) == native.VDX_ERR_SHAPE
    assert ncall_bwd(native, D=96) == native.VDX_ERR_HEAD_DIM
    assert ncall_bwd(native, scale=-1.0) == native.VDX_ERR_SCALE
    assert ncall_bwd(native, dq=A + 0x602) == native.VDX_ERR_ALIGN


def test_bwd_noalloc_rejects_calls_beyond_its_scratch(native):
    """The 720p layer fits the 32 MiB array; a call needing more is refused
    before any HIP call (and after the alignment check)."""
    import spatiotemporal_attention_amd as vdx
    assert vdx.attn_bwd_workspace_size(1, 75600, 40) <= native.NOALLOC_SCRATCH_BYTES
    B, S, H = 1, 1 << 20, 4
    assert vdx.attn_bwd_workspace_size(B, S, H) > native.NOALLOC_SCRATCH_BYTES
    assert ncall_bwd(native, B=B, S=S, H=H) == native.VDX_ERR_SCRATCH
    assert ncall_bwd(native, B=B, S=S, H=H, dq=A + 0x602) == native.VDX_ERR_ALIGN
    if not torch.cuda.is_available():
        assert ncall_bwd(native) == native.VDX_ERR_DEVICE


# --- vdx_rope3d_apply / vdx_rope3d_attn_fwd validation (no GPU needed) ----------------
def rdesc(native, pos=A + 0x800, cos=(A + 0x900, A + 0xa00, A + 0xb00), sin=(A + 0xc00, A + 0xd00, A + 0xe00),
          n=(4, 5, 6), dims=(44, 42, 42), interleaved=True):
    return native.rope3d_desc(pos, cos, sin, n, dims, interleaved)


def rapply(native, x=A, y=A + 0x100, rope="default", B=1, S=64, H=2, D=128):
    r = rdesc(native) if rope == "default" else rope
    return native.rope3d_apply_raw(x, y, r, B, S, H, D, 0)


def rattn(native, q=A, k=A + 0x100, v=A + 0x200, sq=0, sk=0, rope="default", k_rot=A + 0x600,
          out=A + 0x300, lse=A + 0x400, B=1, S=128, H=2, D=128, scale=0.125):
    r = rdesc(native) if rope == "default" else rope
    return native.rope3d_attn_fwd_raw(q, k, v, sq, sk, r, k_rot, out, lse, B, S, H, D, scale, 0)


@pytest.mark.parametrize("kw", [dict(pos=0), dict(pos=A + 0x802), dict(dims=(43, 43, 42)),
                                dict(dims=(-2, 66, 64)), dict(dims=(44, 44, 42)), dict(n=(4, -1, 6)),
                                dict(cos=(A + 0x900, 0, A + 0xb00)), dict(sin=(A + 0xc00, A + 0xd00, 0)),
                                dict(cos=(A + 0x902, A + 0xa00, A + 0xb00))])
def test_rope_description_rejected(native, kw):
    assert rapply(native, rope=rdesc(native, **kw)) == native.VDX_ERR_ROPE
    assert rattn(native, rope=rdesc(native, **kw)) == native.VDX_ERR_ROPE


def test_rope_missing_description(native):
    assert rapply(native, rope=None) == native.VDX_ERR_ROPE
    assert rattn(native, rope=None) == native.VDX_ERR_ROPE


def test_rope_zero_width_section_needs_no_table(native):
    r = rdesc(native, cos=(A + 0x900, 0, A + 0xb00), sin=(A + 0xc00, 0, A + 0xe00), dims=(64, 0, 64))
    want = native.VDX_ERR_DEVICE if not torch.cuda.is_available() else None
    if want is None:
        pytest.skip("a GPU is visible; this path would launch on fake addresses")
    assert rapply(native, rope=r) == want
    assert rattn(native, rope=r) == want


def test_rope_apply_validation(native):
    assert rapply(native, x=0) == native.VDX_ERR_NULL_PTR
    assert rapply(native, y=0) == native.VDX_ERR_NULL_PTR
    assert rapply(native, S=0) == native.VDX_ERR_SHAPE
    assert rapply(native, D=96) == native.VDX_ERR_HEAD_DIM
    assert rapply(native, D=64) == native.VDX_ERR_ROPE  # 44 + 42 + 42 > 64
    assert rapply(native, x=A + 4) == native.VDX_ERR_ALIGN
    # order: NULL -> shape -> head dim -> alignment -> rope
    assert rapply(native, x=0, S=0, D=3, rope=None) == native.VDX_ERR_NULL_PTR
    assert rapply(native, S=0, D=3, y=A + 2, rope=None) == native.VDX_ERR_SHAPE
    assert rapply(native, D=3, y=A + 2, rope=None) == native.VDX_ERR_HEAD_DIM
    assert rapply(native, y=A + 2, rope=None) == native.VDX_ERR_ALIGN


def test_rope_attn_validation(native):
    for w in ("q", "k", "v", "out", "lse", "k_rot"):
        assert rattn(native, **{w: 0}) == native.VDX_ERR_NULL_PTR, w
    assert rattn(native, sq=A + 0x500) == native.VDX_ERR_SEG_PAIR
    assert rattn(native, B=0) == native.VDX_ERR_SHAPE
    assert rattn(native, D=32) == native.VDX_ERR_HEAD_DIM
    assert rattn(native, scale=0.0) == native.VDX_ERR_SCALE
    assert rattn(native, k_rot=A + 0x608) == native.VDX_ERR_ALIGN
    # order: NULL -> segment pair -> shape -> head dim -> scale -> alignment -> rope
    assert rattn(native, k_rot=0, sq=A, B=0, rope=None) == native.VDX_ERR_NULL_PTR
    assert rattn(native, sq=A, B=0, rope=None) == native.VDX_ERR_SEG_PAIR
    assert rattn(native, B=0, D=3, rope=None) == native.VDX_ERR_SHAPE
    assert rattn(native, D=3, scale=-1.0, rope=None) == native.VDX_ERR_HEAD_DIM
    assert rattn(native, scale=-1.0, k_rot=A + 2, rope=None) == native.VDX_ERR_SCALE
    assert rattn(native, k_rot=A + 2, rope=None) == native.VDX_ERR_ALIGN


def rattn_ws(native, ws=A + 0xe00, ws_bytes=None, sq=A + 0x500, sk=A + 0x700, rope="default", k_rot=A + 0x600,
             B=1, S=128, H=2, D=128, **kw):
    r = rdesc(native) if rope == "default" else rope
    if ws_bytes is None:
        ws_bytes = native.lib.vdx_attn_fwd_workspace_size(B, S, H)
    return native.rope3d_attn_fwd_ws_raw(kw.get("q", A), kw.get("k", A + 0x100), kw.get("v", A + 0x200), sq, sk, r,
                                         k_rot, kw.get("out", A + 0x300), kw.get("lse", A + 0x400), ws, ws_bytes,
                                         B, S, H, D, kw.get("scale", 0.125), 0)


def test_rope_attn_ws_validation(native):
    # vdx_rope3d_attn_fwd's checks in its order, then the workspace (masked calls only)
    assert rattn_ws(native, k_rot=0, ws=0) == native.VDX_ERR_NULL_PTR
    assert rattn_ws(native, sk=0, ws=0) == native.VDX_ERR_SEG_PAIR
    assert rattn_ws(native, B=0, ws=0) == native.VDX_ERR_SHAPE
    assert rattn_ws(native, D=32, ws=0) == native.VDX_ERR_HEAD_DIM
    assert rattn_ws(native, scale=0.0, ws=0) == native.VDX_ERR_SCALE
    assert rattn_ws(native, k_rot=A + 0x608, ws=0) == native.VDX_ERR_ALIGN
    assert rattn_ws(native, rope=None, ws=0) == native.VDX_ERR_ROPE
    assert rattn_ws(native, ws=0) == native.VDX_ERR_WORKSPACE
    assert rattn_ws(native, ws=A + 0xe04) == native.VDX_ERR_WORKSPACE
    need = native.lib.vdx_attn_fwd_workspace_size(1, 128, 2)
    assert rattn_ws(native, ws_bytes=need - 1) == native.VDX_ERR_WORKSPACE
    assert rattn_ws(native, sq=0, sk=0, ws_bytes=need - 1) == native.VDX_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert rattn_ws(native) == native.VDX_ERR_DEVICE
        assert rattn_ws(native, sq=0, sk=0, ws=0, ws_bytes=0) == native.VDX_ERR_DEVICE
        assert rattn_ws(native, sq=0, sk=0) == native.VDX_ERR_DEVICE


def test_rope_valid_arguments_without_gpu_report_device_error(native):
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this path would launch on fake addresses")
    assert rapply(native) == native.VDX_ERR_DEVICE
    assert rattn(native) == native.VDX_ERR_DEVICE
    assert rapply(native, rope=rdesc(native, dims=(0, 0, 0), cos=(0, 0, 0), sin=(0, 0, 0))) == \
        native.VDX_ERR_DEVICE


C_CLIENT = r"""
#include "vdx_attn.h"
#include <stdio.h>

/* A plain C99 caller: the header must need no C++ and every entry point must
 * link; only argument validation runs (NULL tensors), so no GPU is touched. */
int main(void) {
    int fails = 0;
    if (vdx_abi_version() != VDX_ABI_VERSION) fails |= 1;
    if (vdx_attn_fwd(0, 0, 0, 0, 0, 0, 0, 1, 64, 1, 64, 0.125f, 0) != VDX_ERR_NULL_PTR) fails |= 2;
    if (vdx_natten3d_fwd(0, 0, 0, 0, 0, 1, 1, 1, 64, 1, 64, 1, 1, 1, 0.125f, 0) != VDX_ERR_NULL_PTR)
        fails |= 4;
    if (vdx_attn_bwd(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 64, 1, 64, 0.125f, 0) != VDX_ERR_NULL_PTR)
        fails |= 8;
    if (vdx_attn_bwd_workspace_size(1, 64, 1) == 0) fails |= 16;
    if (vdx_attn_bwd_noalloc(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 64, 1, 64, 0.125f, 0) != VDX_ERR_NULL_PTR)
        fails |= 256;
    if (vdx_status_str(VDX_OK) == NULL) fails |= 32;
    if (vdx_attn_fwd_ws(0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 64, 1, 64, 0.125f, 0) != VDX_ERR_NULL_PTR) fails |= 512;
    if (vdx_attn_fwd_workspace_size(1, 64, 1) == 0) fails |= 1024;
    {
        vdx_rope3d r = {0};
        if (vdx_rope3d_attn_fwd_ws(0, 0, 0, 0, 0, &r, 0, 0, 0, 0, 0, 1, 64, 1, 64, 0.125f, 0) != VDX_ERR_NULL_PTR)
            fails |= 2048;
    }
    {
        vdx_rope3d r = {0};
        if (vdx_rope3d_apply(0, 0, &r, 1, 64, 1, 64, 0) != VDX_ERR_NULL_PTR) fails |= 64;
        if (vdx_rope3d_attn_fwd(0, 0, 0, 0, 0, &r, 0, 0, 0, 1, 64, 1, 64, 0.125f, 0) != VDX_ERR_NULL_PTR)
            fails |= 128;
    }
    printf("%d %s\n", fails, vdx_status_str(VDX_ERR_NULL_PTR));
    return fails;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """A C99 program includes the header, links the built library and calls
    every entry point (validation paths only)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    from spatiotemporal_attention_amd import _native
    libdir = os.path.dirname(_native.LIB_PATH)
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    cmd = [gcc, "-std=c99", "-Wall", "-Werror=implicit-function-declaration", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-o", str(exe),
           "-L", libdir, "-lvdx_attn", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr[-2000:])
    assert "VDX_ERR_NULL_PTR" in r.stdout
