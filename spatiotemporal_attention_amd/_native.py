"""ctypes binding of the C ABI in include/vdx_attn.h (argument marshalling only).

Loads the in-tree ``libvdx_attn.so``; there is no fallback path: if the
library is missing or fails to load, import of the binding raises.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

VDX_OK = 0
VDX_ERR_NULL_PTR = 1
VDX_ERR_SEG_PAIR = 2
VDX_ERR_SHAPE = 3
VDX_ERR_HEAD_DIM = 4
VDX_ERR_SCALE = 5
VDX_ERR_ALIGN = 6
VDX_ERR_DEVICE = 7
VDX_ERR_LAUNCH = 8
VDX_ERR_WINDOW = 9
VDX_ERR_WORKSPACE = 10
VDX_ERR_ROPE = 11
VDX_ERR_SCRATCH = 12

EXPORTED = ("vdx_attn_fwd", "vdx_attn_fwd_ws", "vdx_attn_fwd_workspace_size", "vdx_natten3d_fwd",
            "vdx_attn_bwd", "vdx_attn_bwd_noalloc", "vdx_attn_bwd_workspace_size", "vdx_rope3d_apply",
            "vdx_rope3d_attn_fwd", "vdx_rope3d_attn_fwd_ws", "vdx_status_str", "vdx_abi_version")


class Rope3D(ctypes.Structure):
    """struct vdx_rope3d of include/vdx_attn.h (device pointers as integers)."""
    _fields_ = [("pos", ctypes.c_void_p), ("cos_tab", ctypes.c_void_p * 3), ("sin_tab", ctypes.c_void_p * 3),
                ("n", ctypes.c_int * 3), ("dims", ctypes.c_int * 3), ("interleaved", ctypes.c_int)]


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"HIP library not built: {path} (build it with python spatiotemporal_attention_amd/build.py)")
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i = ctypes.c_int
    lib.vdx_attn_fwd.restype = i
    lib.vdx_attn_fwd.argtypes = [p, p, p, p, p, p, p, i, i, i, i, ctypes.c_float, p]
    lib.vdx_attn_fwd_ws.restype = i
    lib.vdx_attn_fwd_ws.argtypes = [p] * 8 + [ctypes.c_size_t] + [i] * 4 + [ctypes.c_float, p]
    lib.vdx_attn_fwd_workspace_size.restype = ctypes.c_size_t
    lib.vdx_attn_fwd_workspace_size.argtypes = [i, i, i]
    lib.vdx_natten3d_fwd.restype = i
    lib.vdx_natten3d_fwd.argtypes = [p, p, p, p, p] + [i] * 9 + [ctypes.c_float, p]
    lib.vdx_attn_bwd.restype = i
    lib.vdx_attn_bwd.argtypes = [p] * 12 + [ctypes.c_size_t] + [i] * 4 + [ctypes.c_float, p]
    lib.vdx_attn_bwd_noalloc.restype = i
    lib.vdx_attn_bwd_noalloc.argtypes = [p] * 11 + [i] * 4 + [ctypes.c_float, p]
    lib.vdx_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.vdx_attn_bwd_workspace_size.argtypes = [i, i, i]
    lib.vdx_rope3d_apply.restype = i
    lib.vdx_rope3d_apply.argtypes = [p, p, ctypes.POINTER(Rope3D), i, i, i, i, p]
    lib.vdx_rope3d_attn_fwd.restype = i
    lib.vdx_rope3d_attn_fwd.argtypes = [p, p, p, p, p, ctypes.POINTER(Rope3D), p, p, p, i, i, i, i,
                                        ctypes.c_float, p]
    lib.vdx_rope3d_attn_fwd_ws.restype = i
    lib.vdx_rope3d_attn_fwd_ws.argtypes = [p, p, p, p, p, ctypes.POINTER(Rope3D), p, p, p, p, ctypes.c_size_t,
                                           i, i, i, i, ctypes.c_float, p]
    lib.vdx_status_str.restype = ctypes.c_char_p
    lib.vdx_status_str.argtypes = [i]
    lib.vdx_abi_version.restype = i
    lib.vdx_abi_version.argtypes = []
    return lib


lib = _load()


def status_str(rc: int) -> str:
    return lib.vdx_status_str(int(rc)).decode()


def abi_version() -> int:
    return int(lib.vdx_abi_version())


def attn_fwd_raw(q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale, stream) -> int:
    """Direct C call with integer device addresses (0 for NULL)."""
    return int(lib.vdx_attn_fwd(q or None, k or None, v or None, seg_q or None, seg_kv or None,
                                out or None, lse or None, int(B), int(S), int(H), int(D),
                                float(scale), stream or None))


def attn_fwd_ws_raw(q, k, v, seg_q, seg_kv, out, lse, ws, ws_bytes, B, S, H, D, scale, stream) -> int:
    """Direct C call with integer device addresses (0 for NULL)."""
    return int(lib.vdx_attn_fwd_ws(q or None, k or None, v or None, seg_q or None, seg_kv or None,
                                   out or None, lse or None, ws or None, int(ws_bytes), int(B), int(S),
                                   int(H), int(D), float(scale), stream or None))


def natten3d_fwd_raw(q, k, v, out, lse, B, NT, NH, NW, H, D, KT, KH, KW, scale, stream) -> int:
    """Direct C call with integer device addresses (0 for NULL)."""
    return int(lib.vdx_natten3d_fwd(q or None, k or None, v or None, out or None, lse or None,
                                    int(B), int(NT), int(NH), int(NW), int(H), int(D),
                                    int(KT), int(KH), int(KW), float(scale), stream or None))


def attn_bwd_raw(q, k, v, seg_q, seg_kv, out, lse, dout, dq, dk, dv, ws, ws_bytes, B, S, H, D,
                 scale, stream) -> int:
    """Direct C call with integer device addresses (0 for NULL)."""
    return int(lib.vdx_attn_bwd(q or None, k or None, v or None, seg_q or None, seg_kv or None,
                                out or None, lse or None, dout or None, dq or None, dk or None,
                                dv or None, ws or None, int(ws_bytes), int(B), int(S), int(H),
                                int(D), float(scale), stream or None))


def attn_bwd_noalloc_raw(q, k, v, seg_q, seg_kv, out, lse, dout, dq, dk, dv, B, S, H, D, scale,
                        stream) -> int:
    """Direct C call with integer device addresses (0 for NULL)."""
    return int(lib.vdx_attn_bwd_noalloc(q or None, k or None, v or None, seg_q or None, seg_kv or None,
                                        out or None, lse or None, dout or None, dq or None, dk or None,
                                        dv or None, int(B), int(S), int(H), int(D), float(scale),
                                        stream or None))


NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_bwd_workspace_size(B, S, H) -> int:
    return int(lib.vdx_attn_bwd_workspace_size(int(B), int(S), int(H)))


def rope3d_desc(pos, cos, sin, n, dims, interleaved) -> Rope3D:
    """A struct vdx_rope3d from integer device addresses (0 for NULL)."""
    r = Rope3D()
    r.pos = pos or None
    for a in range(3):
        r.cos_tab[a] = cos[a] or None
        r.sin_tab[a] = sin[a] or None
        r.n[a] = int(n[a])
        r.dims[a] = int(dims[a])
    r.interleaved = 1 if interleaved else 0
    return r


def rope3d_apply_raw(x, y, rope: Rope3D, B, S, H, D, stream) -> int:
    """Direct C call with integer device addresses (0 for NULL); rope may be None."""
    return int(lib.vdx_rope3d_apply(x or None, y or None, None if rope is None else ctypes.byref(rope),
                                    int(B), int(S), int(H), int(D), stream or None))


def rope3d_attn_fwd_raw(q, k, v, seg_q, seg_kv, rope: Rope3D, k_rot, out, lse, B, S, H, D, scale,
                        stream) -> int:
    """Direct C call with integer device addresses (0 for NULL); rope may be None."""
    return int(lib.vdx_rope3d_attn_fwd(q or None, k or None, v or None, seg_q or None, seg_kv or None,
                                       None if rope is None else ctypes.byref(rope), k_rot or None,
                                       out or None, lse or None, int(B), int(S), int(H), int(D),
                                       float(scale), stream or None))


def rope3d_attn_fwd_ws_raw(q, k, v, seg_q, seg_kv, rope: Rope3D, k_rot, out, lse, ws, ws_bytes, B, S, H, D,
                           scale, stream) -> int:
    """Direct C call with integer device addresses (0 for NULL); rope may be None."""
    return int(lib.vdx_rope3d_attn_fwd_ws(q or None, k or None, v or None, seg_q or None, seg_kv or None,
                                          None if rope is None else ctypes.byref(rope), k_rot or None,
                                          out or None, lse or None, ws or None, int(ws_bytes), int(B), int(S),
                                          int(H), int(D), float(scale), stream or None))
