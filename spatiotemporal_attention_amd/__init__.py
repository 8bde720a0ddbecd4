"""spatiotemporal_attention_amd -- segment-masked, non-causal flash-attention
forward for video-DiT token volumes on MI355X (gfx950), and 3D neighbourhood
(windowed) attention over a t x h x w token grid.

``attn_fwd`` computes, for q, k, v of shape [B, S, H, D] (bf16):
    out[b,i,h,:] = softmax_j(scale * q[b,i,h,:] . k[b,j,h,:]) v[b,j,h,:]
over the keys j whose segment ID equals the query's (ID 0 = padding, matched
by nothing), and lse[b,h,i] = log sum_j exp(scale * q . k) over those keys
(vidax paper, arXiv:2609.18077: section 2 "3D RoPE, 3D VAEs, and flash
attention"; Appendix A, Table 4, group 2 for SegmentIds).

``natten3d_fwd`` computes the same softmax restricted, for each query of a
t x h x w grid (tokens flattened (t, y, x), x fastest), to its neighbourhood
window: along an axis of length n an odd window k covers min(k, n) positions
starting at clamp(c - k//2, 0, n - min(k, n)) (section 2 for the
windowed-attention primitive of the neighbourhood-attention VAE decoder;
Appendix A, Table 4, group 4 for its 11 x 11 x 11 window).

``attn_bwd`` returns the gradients (dq, dk, dv) of ``attn_fwd`` for a given
dout, recomputing the probabilities from the forward's lse (section 5 lists
training and fine-tuning, which need them).

``rope3d_apply`` rotates a [B, S, H, D] tensor by a 3D rotary position
embedding over (t, y, x) whose conventions the caller gives (per-axis
cos/sin tables, head-dim section widths, pairing, per-token positions);
``rope3d_attn_fwd`` is ``attn_fwd`` on the rotated queries and keys, with the
queries rotated as the attention kernel loads them (section 2 places the 3D
RoPE right before attention and keeps each family's convention).

Every step runs in the hand-written HIP kernels behind the C ABI
(include/vdx_attn.h); this module only checks arguments and passes device
pointers and the current stream.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _native
from ._native import abi_version, status_str

__all__ = ["attn_fwd", "attn_fwd_workspace_size", "attn_bwd", "attn_bwd_workspace_size", "natten3d_fwd", "rope3d_apply",
           "rope3d_attn_fwd", "abi_version", "status_str", "VdxError"]


class VdxError(ValueError):
    def __init__(self, rc: int):
        super().__init__(status_str(rc))
        self.rc = rc


def _outputs(q: torch.Tensor, out: Optional[torch.Tensor], lse: Optional[torch.Tensor],
             stream: torch.cuda.Stream) -> Tuple[torch.Tensor, torch.Tensor]:
    """Checks caller-given out / lse, or allocates them on the launch stream
    (so the caching allocator orders their reuse after the kernel)."""
    B, S, H, D = q.shape
    if out is not None and (out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous()
                            or out.device != q.device):
        raise ValueError("out must be a contiguous bf16 tensor like q")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S)
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, S]")
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    return out, lse


def attn_fwd_workspace_size(B: int, S: int, H: int) -> int:
    """Bytes of workspace the masked forward (vdx_attn_fwd_ws) needs."""
    return int(_native.lib.vdx_attn_fwd_workspace_size(int(B), int(S), int(H)))


def _workspace(workspace: Optional[torch.Tensor], B: int, S: int, H: int, device, stream) -> torch.Tensor:
    """Checks a caller's forward workspace, or allocates one on the launch stream."""
    need = attn_fwd_workspace_size(B, S, H)
    if workspace is None:
        with torch.cuda.stream(stream):
            return torch.empty(need, dtype=torch.uint8, device=device)
    if (workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.numel() < need
            or workspace.device != device):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of >= {need} bytes on {device}")
    return workspace


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             seg_q: Optional[torch.Tensor] = None, seg_kv: Optional[torch.Tensor] = None,
             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None,
             workspace: Optional[torch.Tensor] = None,
             scheduled: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """Segment-masked attention forward on the current (or given) HIP stream.

    q, k, v: bf16 [B, S, H, D] contiguous on one GPU.  seg_q, seg_kv: int32
    [B, S] or both None (unmasked).  Returns (out bf16 [B,S,H,D], lse fp32 [B,H,S]).

    With segment IDs the call goes to vdx_attn_fwd_ws (work counters, a
    longest-first block order and the partial results of split items in
    a workspace; ``workspace``, a uint8 CUDA tensor of at least
    attn_fwd_workspace_size(B, S, H) bytes, or one allocated here on the
    launch stream); ``scheduled=False`` calls vdx_attn_fwd, one workgroup per
    block in index order.  Without segment IDs the call goes to
    vdx_attn_fwd_ws only when a ``workspace`` is given (and ``scheduled``).
    The two entry points give the same bits except on the query blocks whose
    keys vdx_attn_fwd_ws splits (equal up to rounding).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, S, H, D]")
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of shape {tuple(q.shape)}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if (seg_q is None) != (seg_kv is None):
        raise VdxError(_native.VDX_ERR_SEG_PAIR)
    for name, t in (("seg_q", seg_q), ("seg_kv", seg_kv)):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (B, S) or not t.is_cuda
                              or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous int32 CUDA tensor of shape {(B, S)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    out, lse = _outputs(q, out, lse, stream)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), 0 if seg_q is None else seg_q.data_ptr(),
            0 if seg_kv is None else seg_kv.data_ptr(), out.data_ptr(), lse.data_ptr())
    with torch.cuda.device(q.device):
        if scheduled and (seg_q is not None or workspace is not None):
            workspace = _workspace(workspace, B, S, H, q.device, stream)
            rc = _native.attn_fwd_ws_raw(*ptrs, workspace.data_ptr(), workspace.numel(), B, S, H, D, scale,
                                         stream.cuda_stream)
        else:
            rc = _native.attn_fwd_raw(*ptrs, B, S, H, D, scale, stream.cuda_stream)
    if rc != 0:
        raise VdxError(rc)
    return out, lse


def natten3d_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 grid: Tuple[int, int, int], window: Tuple[int, int, int],
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """3D neighbourhood attention forward on the current (or given) HIP stream.

    q, k, v: bf16 [B, S, H, D] contiguous on one GPU with S = NT*NH*NW for
    grid = (NT, NH, NW); window = (KT, KH, KW), odd sizes.  Returns
    (out bf16 [B,S,H,D], lse fp32 [B,H,S]).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, S, H, D]")
    B, S, H, D = q.shape
    NT, NH, NW = (int(x) for x in grid)
    KT, KH, KW = (int(x) for x in window)
    if NT * NH * NW != S:
        raise ValueError(f"grid {grid} does not hold S={S} tokens")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of shape {tuple(q.shape)}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    out, lse = _outputs(q, out, lse, stream)
    with torch.cuda.device(q.device):
        rc = _native.natten3d_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), B, NT, NH, NW, H, D, KT, KH, KW, scale,
                                      stream.cuda_stream)
    if rc != 0:
        raise VdxError(rc)
    return out, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
             lse: torch.Tensor, dout: torch.Tensor,
             seg_q: Optional[torch.Tensor] = None, seg_kv: Optional[torch.Tensor] = None,
             scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradient of ``attn_fwd`` on the current (or given) HIP stream.

    q, k, v, seg_q, seg_kv, scale: as passed to attn_fwd; out, lse: its
    outputs; dout: bf16 [B, S, H, D].  workspace: optional uint8 CUDA tensor of
    at least ``attn_bwd_workspace_size(B, S, H)`` bytes (allocated here if
    None).  Returns (dq, dk, dv), bf16 [B, S, H, D].
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, S, H, D]")
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of shape {tuple(q.shape)}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, S]")
    if (seg_q is None) != (seg_kv is None):
        raise VdxError(_native.VDX_ERR_SEG_PAIR)
    for name, t in (("seg_q", seg_q), ("seg_kv", seg_kv)):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (B, S) or not t.is_cuda
                              or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous int32 CUDA tensor of shape {(B, S)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None and (t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous bf16 tensor like q")
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()
                                  or workspace.device != q.device):
        raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
    need = _native.attn_bwd_workspace_size(B, S, H)
    # Tensors made here belong to the launch stream: the caching allocator
    # then hands a freed block (the workspace, when this function allocated
    # it, is freed on return) to later work only in that stream's order, never
    # while the kernels still use it.
    with torch.cuda.stream(stream):
        grads = [torch.empty_like(q) if t is None else t for t in (dq, dk, dv)]
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        rc = _native.attn_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  0 if seg_q is None else seg_q.data_ptr(),
                                  0 if seg_kv is None else seg_kv.data_ptr(),
                                  out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                  grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                                  workspace.data_ptr(), ws_bytes, B, S, H, D, scale,
                                  stream.cuda_stream)
    if rc != 0:
        raise VdxError(rc)
    return grads[0], grads[1], grads[2]


def attn_bwd_workspace_size(B: int, S: int, H: int) -> int:
    """Bytes of workspace ``attn_bwd`` needs for (B, S, H)."""
    return _native.attn_bwd_workspace_size(B, S, H)


def _rope_desc(q: torch.Tensor, pos: torch.Tensor, cos, sin, dims, interleaved: bool):
    """Checks the rotary-embedding tensors against q [B, S, H, D] and returns
    the C description (the tensors must outlive the call's stream work)."""
    B, S, H, D = q.shape
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B, S, 3) or not pos.is_cuda or not pos.is_contiguous() \
            or pos.device != q.device:
        raise ValueError(f"pos must be a contiguous int32 CUDA tensor of shape {(B, S, 3)}")
    if len(cos) != 3 or len(sin) != 3 or len(dims) != 3:
        raise ValueError("cos, sin and dims need one entry per axis (t, y, x)")
    n = []
    for a in range(3):
        c, s_ = cos[a], sin[a]
        for name, t in (("cos", c), ("sin", s_)):
            if t.dtype != torch.float32 or t.dim() != 2 or not t.is_cuda or not t.is_contiguous() \
                    or t.device != q.device or t.shape[1] != int(dims[a]) // 2:
                raise ValueError(f"{name}[{a}] must be a contiguous fp32 CUDA tensor [n, dims[{a}] / 2]")
        if c.shape != s_.shape:
            raise ValueError(f"cos[{a}] and sin[{a}] differ in shape")
        n.append(int(c.shape[0]))
    ptr = lambda t: t.data_ptr() if t.numel() else 0
    return _native.rope3d_desc(pos.data_ptr(), [ptr(c) for c in cos], [ptr(s_) for s_ in sin], n,
                               [int(d) for d in dims], interleaved)


def rope3d_apply(x: torch.Tensor, pos: torch.Tensor, cos, sin, dims, interleaved: bool = True,
                 out: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """3D rotary position embedding of x (bf16 [B, S, H, D], contiguous).

    pos: int32 [B, S, 3], the (t, y, x) of every token (a token outside the
    tables is left as is); cos / sin: per axis (t, y, x) an fp32 [n_a, d_a / 2]
    table; dims: section widths (d_t, d_h, d_w); interleaved: pairs
    (2p, 2p + 1) of a section, else (p, p + d_a / 2).  out may be x (in place).
    """
    if x.dim() != 4 or x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 CUDA tensor [B, S, H, D]")
    B, S, H, D = x.shape
    desc = _rope_desc(x, pos, cos, sin, dims, interleaved)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    if out is None:
        with torch.cuda.stream(stream):
            out = torch.empty_like(x)
    elif out.dtype != torch.bfloat16 or out.shape != x.shape or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous bf16 tensor like x")
    with torch.cuda.device(x.device):
        rc = _native.rope3d_apply_raw(x.data_ptr(), out.data_ptr(), desc, B, S, H, D, stream.cuda_stream)
    if rc != 0:
        raise VdxError(rc)
    return out


def rope3d_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, cos, sin, dims,
                    interleaved: bool = True, seg_q: Optional[torch.Tensor] = None,
                    seg_kv: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                    k_rot: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None,
                    workspace: Optional[torch.Tensor] = None,
                    scheduled: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """``attn_fwd`` on the 3D-rotary-embedded queries and keys (see
    ``rope3d_apply``; v is used as given).  k_rot: bf16 like k, receives the
    rotated keys (allocated here if None; may be k itself).  With segment IDs
    the call goes to vdx_rope3d_attn_fwd_ws with ``workspace`` (as for
    ``attn_fwd``) unless ``scheduled=False``.  Returns (out bf16 [B,S,H,D],
    lse fp32 [B,H,S])."""
    if q.dim() != 4:
        raise ValueError("q must be [B, S, H, D]")
    B, S, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of shape {tuple(q.shape)}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if (seg_q is None) != (seg_kv is None):
        raise VdxError(_native.VDX_ERR_SEG_PAIR)
    for name, t in (("seg_q", seg_q), ("seg_kv", seg_kv)):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (B, S) or not t.is_cuda
                              or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous int32 CUDA tensor of shape {(B, S)}")
    desc = _rope_desc(q, pos, cos, sin, dims, interleaved)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    out, lse = _outputs(q, out, lse, stream)
    if k_rot is None:
        with torch.cuda.stream(stream):
            k_rot = torch.empty_like(k)
    elif k_rot.dtype != torch.bfloat16 or k_rot.shape != k.shape or not k_rot.is_contiguous() \
            or k_rot.device != q.device:
        raise ValueError("k_rot must be a contiguous bf16 tensor like k")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), 0 if seg_q is None else seg_q.data_ptr(),
            0 if seg_kv is None else seg_kv.data_ptr(), desc, k_rot.data_ptr(), out.data_ptr(), lse.data_ptr())
    with torch.cuda.device(q.device):
        if scheduled and (seg_q is not None or workspace is not None):
            workspace = _workspace(workspace, B, S, H, q.device, stream)
            rc = _native.rope3d_attn_fwd_ws_raw(*ptrs, workspace.data_ptr(), workspace.numel(), B, S, H, D, scale,
                                                stream.cuda_stream)
        else:
            rc = _native.rope3d_attn_fwd_raw(*ptrs, B, S, H, D, scale, stream.cuda_stream)
    if rc != 0:
        raise VdxError(rc)
    return out, lse
