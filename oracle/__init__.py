"""CPU oracles for segment-masked, non-causal softmax self-attention (forward
and gradient) and for 3D neighbourhood (windowed) self-attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library.

The arithmetic lives in ``attn_oracle.c`` (scalar fp64, plain definition of
softmax(scale * Q K^T, masked by segment IDs) V -- vidax paper, section 2
"3D RoPE, 3D VAEs, and flash attention" with its reference [2], and Appendix A,
Table 4, group 2 for SegmentIds) and ``natten_oracle.c`` (the same softmax
restricted to each query's 3D neighbourhood window -- section 2 for the
windowed-attention fallback of the neighbourhood-attention VAE decoder,
Appendix A, Table 4, group 4 for its 11 x 11 x 11 window) and
``attn_bwd_oracle.c`` (the exact gradients of the segment-masked forward with
respect to q, k, v -- section 5 lists training as future work) and
``rope_oracle.c`` (the 3D rotary position embedding of queries and keys that
section 2 places right before attention, with the per-axis angle tables and
section widths, the pairing of features and the positions all given by the
caller).  This wrapper only marshals numpy arrays.

Every function here has pins in ``tests/test_oracle.py``,
``tests/test_natten_oracle.py``, ``tests/test_bwd_oracle.py`` and
``tests/test_rope_oracle.py``; their module docstrings say what pins what.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from .build import LIB_PATH, build_oracle

_lib = None


def _load(path: Optional[str] = None):
    """Load (once) the oracle library; ``path`` swaps in another build of the
    same source (the mutation tests use this to check that the pins bite)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is None:
        path = LIB_PATH
        if not os.path.exists(path):
            build_oracle()
    lib = ctypes.CDLL(path)
    f = lib.vdx_oracle_attn_fwd
    f.restype = ctypes.c_int
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    f.argtypes = [p, p, p, p, p, i64, i64, i64, i64, ctypes.c_double,
                  p, i64, p, p, p, p, ctypes.c_int]
    bw = lib.vdx_oracle_attn_bwd
    bw.restype = ctypes.c_int
    bw.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_double, p, p, p, p, p, p,
                   ctypes.c_int]
    br = lib.vdx_oracle_attn_bwd_dq_rows
    br.restype = ctypes.c_int
    br.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_double, p, i64, p, p, ctypes.c_int]
    r = lib.vdx_oracle_rope3d
    r.restype = ctypes.c_int
    r.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                  i64, i64, i64, i64, p, p]
    rb = lib.vdx_oracle_round_bf16
    rb.restype = None
    rb.argtypes = [p, i64, p]
    g = lib.vdx_oracle_natten3d_fwd
    g.restype = ctypes.c_int
    g.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double,
                  p, i64, p, p, p, ctypes.c_int]
    _lib = lib
    return lib


def use_library(path: Optional[str]) -> None:
    """Point the wrappers at another oracle build (None -> the default one)."""
    global _lib
    _lib = None
    _load(path)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def attn_fwd(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
             seg_q: Optional[np.ndarray], seg_kv: Optional[np.ndarray],
             scale: float, rows: Optional[np.ndarray] = None,
             n_threads: Optional[int] = None, want_probs: bool = False,
             sens: Optional[np.ndarray] = None
             ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """fp64 attention on bf16 bit patterns.

    q_bits/k_bits/v_bits: uint16 [B, S, H, D] (bf16 bits).
    seg_q/seg_kv: int32 [B, S] or both None.
    rows: optional int64 [n, 3] of (b, h, i); then out is [n, D] and lse [n];
          else out is [B, S, H, D] and lse [B, H, S].
    sens: optional fp64 array shaped like out, filled with the rounding
          sensitivity sum_j P_ij |v_jd| of each output element.
    Returns (out fp64, lse fp64, probs fp64 or None).
    """
    lib = _load()
    for a in (q_bits, k_bits, v_bits):
        assert a.dtype == np.uint16 and a.ndim == 4
    B, S, H, D = q_bits.shape
    assert k_bits.shape == q_bits.shape and v_bits.shape == q_bits.shape
    q_bits = np.ascontiguousarray(q_bits)
    k_bits = np.ascontiguousarray(k_bits)
    v_bits = np.ascontiguousarray(v_bits)
    if (seg_q is None) != (seg_kv is None):
        raise ValueError("seg_q and seg_kv must both be given or both be None")
    if seg_q is not None:
        seg_q = np.ascontiguousarray(seg_q, dtype=np.int32)
        seg_kv = np.ascontiguousarray(seg_kv, dtype=np.int32)
        assert seg_q.shape == (B, S) and seg_kv.shape == (B, S)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        out = np.zeros((n, D), dtype=np.float64)
        lse = np.zeros((n,), dtype=np.float64)
        n_prob_rows = n
    else:
        n = 0
        out = np.zeros((B, S, H, D), dtype=np.float64)
        lse = np.zeros((B, H, S), dtype=np.float64)
        n_prob_rows = B * H * S
    probs = np.zeros((n_prob_rows, S), dtype=np.float64) if want_probs else None
    if sens is not None:
        assert sens.shape == out.shape and sens.dtype == np.float64 and sens.flags.c_contiguous
    rc = lib.vdx_oracle_attn_fwd(
        _ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(seg_q), _ptr(seg_kv),
        B, S, H, D, float(scale), _ptr(rows), n, _ptr(out), _ptr(lse), _ptr(probs), _ptr(sens),
        int(n_threads if n_threads is not None else default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    return out, lse, probs


def natten3d_fwd(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                 grid: Tuple[int, int, int], window: Tuple[int, int, int], scale: float,
                 rows: Optional[np.ndarray] = None, n_threads: Optional[int] = None,
                 sens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 3D neighbourhood attention on bf16 bit patterns.

    q_bits/k_bits/v_bits: uint16 [B, S, H, D], S = NT*NH*NW, tokens (t, y, x)
    row-major.  grid = (NT, NH, NW); window = (KT, KH, KW), odd sizes.
    rows: optional int64 [n, 3] of (b, h, i); then out is [n, D] and lse [n];
    else out is [B, S, H, D] and lse [B, H, S].  sens: optional fp64 array
    shaped like out, filled with sum over the window of P_ij |v_jd|.
    """
    lib = _load()
    for a in (q_bits, k_bits, v_bits):
        assert a.dtype == np.uint16 and a.ndim == 4
    B, S, H, D = q_bits.shape
    NT, NH, NW = (int(x) for x in grid)
    KT, KH, KW = (int(x) for x in window)
    if NT * NH * NW != S:
        raise ValueError("grid does not match the sequence length")
    assert k_bits.shape == q_bits.shape and v_bits.shape == q_bits.shape
    q_bits = np.ascontiguousarray(q_bits)
    k_bits = np.ascontiguousarray(k_bits)
    v_bits = np.ascontiguousarray(v_bits)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        out = np.zeros((n, D), dtype=np.float64)
        lse = np.zeros((n,), dtype=np.float64)
    else:
        n = 0
        out = np.zeros((B, S, H, D), dtype=np.float64)
        lse = np.zeros((B, H, S), dtype=np.float64)
    if sens is not None:
        assert sens.shape == out.shape and sens.dtype == np.float64 and sens.flags.c_contiguous
    rc = lib.vdx_oracle_natten3d_fwd(
        _ptr(q_bits), _ptr(k_bits), _ptr(v_bits), B, NT, NH, NW, H, D, KT, KH, KW,
        float(scale), _ptr(rows), n, _ptr(out), _ptr(lse), _ptr(sens),
        int(n_threads if n_threads is not None else default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    return out, lse


def attn_bwd(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, dout_bits: np.ndarray,
             seg_q: Optional[np.ndarray], seg_kv: Optional[np.ndarray], scale: float,
             n_threads: Optional[int] = None, sensitivity: bool = False):
    """fp64 gradients (dq, dk, dv), each [B, S, H, D], of sum(dout * out) for
    the segment-masked forward, on bf16 bit patterns.  Dense S x S per head:
    for S up to a few thousand.  With sensitivity=True also returns (tq, tk,
    tv): per element, the sum of |terms| whose one-time rounding to relative
    precision u moves the result by at most u * t."""
    lib = _load()
    for a in (q_bits, k_bits, v_bits, dout_bits):
        assert a.dtype == np.uint16 and a.ndim == 4
    B, S, H, D = q_bits.shape
    arrs = [np.ascontiguousarray(a) for a in (q_bits, k_bits, v_bits, dout_bits)]
    if (seg_q is None) != (seg_kv is None):
        raise ValueError("seg_q and seg_kv must both be given or both be None")
    if seg_q is not None:
        seg_q = np.ascontiguousarray(seg_q, dtype=np.int32)
        seg_kv = np.ascontiguousarray(seg_kv, dtype=np.int32)
    dq = np.zeros((B, S, H, D), dtype=np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    ts = [np.zeros_like(dq) for _ in range(3)] if sensitivity else [None] * 3
    rc = lib.vdx_oracle_attn_bwd(*[_ptr(a) for a in arrs], _ptr(seg_q), _ptr(seg_kv),
                                 B, S, H, D, float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                 *[_ptr(t) for t in ts],
                                 int(n_threads if n_threads is not None else default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    if sensitivity:
        return dq, dk, dv, ts[0], ts[1], ts[2]
    return dq, dk, dv


def attn_bwd_dq_rows(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                     dout_bits: np.ndarray, seg_q: Optional[np.ndarray],
                     seg_kv: Optional[np.ndarray], scale: float, rows: np.ndarray,
                     n_threads: Optional[int] = None, sensitivity: bool = False):
    """fp64 dq [n_rows, D] of the listed (b, h, i) rows only, any S (O(S D)
    per row); with sensitivity=True also tq [n_rows, D] (see attn_bwd)."""
    lib = _load()
    for a in (q_bits, k_bits, v_bits, dout_bits):
        assert a.dtype == np.uint16 and a.ndim == 4
    B, S, H, D = q_bits.shape
    arrs = [np.ascontiguousarray(a) for a in (q_bits, k_bits, v_bits, dout_bits)]
    if (seg_q is None) != (seg_kv is None):
        raise ValueError("seg_q and seg_kv must both be given or both be None")
    if seg_q is not None:
        seg_q = np.ascontiguousarray(seg_q, dtype=np.int32)
        seg_kv = np.ascontiguousarray(seg_kv, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    dq = np.zeros((rows.shape[0], D), dtype=np.float64)
    tq = np.zeros_like(dq) if sensitivity else None
    rc = lib.vdx_oracle_attn_bwd_dq_rows(*[_ptr(a) for a in arrs], _ptr(seg_q), _ptr(seg_kv),
                                         B, S, H, D, float(scale), _ptr(rows), rows.shape[0],
                                         _ptr(dq), _ptr(tq),
                                         int(n_threads if n_threads is not None else default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    return (dq, tq) if sensitivity else dq


def rope3d(x_bits: np.ndarray, pos: np.ndarray, cos: Tuple[np.ndarray, np.ndarray, np.ndarray],
           sin: Tuple[np.ndarray, np.ndarray, np.ndarray], dims: Tuple[int, int, int],
           interleaved: bool) -> Tuple[np.ndarray, np.ndarray]:
    """3D rotary position embedding of bf16 bit patterns x [B, S, H, D].

    pos: int32 [B, S, 3], the (t, y, x) of every token; cos / sin: per axis
    (t, y, x) fp32 tables [n_a, d_a / 2]; dims: the section widths (d_t, d_h,
    d_w); interleaved: pairs (2p, 2p + 1) of a section, else (p, p + d_a / 2).
    Returns (bf16 bits uint16 [B, S, H, D], the fp64 values before rounding)."""
    lib = _load()
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 4
    B, S, H, D = x_bits.shape
    x_bits = np.ascontiguousarray(x_bits)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert pos.shape == (B, S, 3)
    cs = [np.ascontiguousarray(c, dtype=np.float32) for c in cos]
    sn = [np.ascontiguousarray(c, dtype=np.float32) for c in sin]
    for a in range(3):
        assert cs[a].ndim == 2 and cs[a].shape == sn[a].shape and cs[a].shape[1] == dims[a] // 2
    y = np.zeros((B, S, H, D), dtype=np.uint16)
    yd = np.zeros((B, S, H, D), dtype=np.float64)
    tabs = []
    for a in range(3):
        tabs += [_ptr(cs[a]) if cs[a].size else None, _ptr(sn[a]) if sn[a].size else None]
    rc = lib.vdx_oracle_rope3d(_ptr(x_bits), _ptr(pos), *tabs, cs[0].shape[0], cs[1].shape[0],
                               cs[2].shape[0], int(dims[0]), int(dims[1]), int(dims[2]),
                               1 if interleaved else 0, B, S, H, D, _ptr(y), _ptr(yd))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    return y, yd


def round_bf16(v: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) of fp64 values, rounded to nearest, ties to even."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    lib.vdx_oracle_round_bf16(_ptr(v), v.size, _ptr(out))
    return out


def rope3d_attn_fwd(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, pos: np.ndarray,
                    cos, sin, dims, interleaved: bool, seg_q: Optional[np.ndarray],
                    seg_kv: Optional[np.ndarray], scale: float, rows: Optional[np.ndarray] = None,
                    n_threads: Optional[int] = None,
                    sens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention (attn_fwd) of the 3D-rotary-embedded queries and keys: q and
    k go through rope3d (rounded to bf16), v is used as given; sens as for
    attn_fwd."""
    qr, _ = rope3d(q_bits, pos, cos, sin, dims, interleaved)
    kr, _ = rope3d(k_bits, pos, cos, sin, dims, interleaved)
    out, lse, _ = attn_fwd(qr, kr, v_bits, seg_q, seg_kv, scale, rows=rows, n_threads=n_threads, sens=sens)
    return out, lse
