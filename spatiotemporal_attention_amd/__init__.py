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

__all__ = ["attn_fwd", "attn_bwd", "attn_bwd_workspace_size", "natten3d_fwd", "abi_version", "status_str", "VdxError"]


class VdxError(ValueError):
    def __init__(self, rc: int):
        super().__init__(status_str(rc))
        self.rc = rc


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             seg_q: Optional[torch.Tensor] = None, seg_kv: Optional[torch.Tensor] = None,
             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Segment-masked attention forward on the current (or given) HIP stream.

    q, k, v: bf16 [B, S, H, D] contiguous on one GPU.  seg_q, seg_kv: int32
    [B, S] or both None (unmasked).  Returns (out bf16 [B,S,H,D], lse fp32 [B,H,S]).
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
    if out is None:
        out = torch.empty_like(q)
    elif out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bf16 tensor like q")
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, S]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        rc = _native.attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  0 if seg_q is None else seg_q.data_ptr(),
                                  0 if seg_kv is None else seg_kv.data_ptr(),
                                  out.data_ptr(), lse.data_ptr(), B, S, H, D, scale,
                                  stream.cuda_stream)
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
    if out is None:
        out = torch.empty_like(q)
    elif out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bf16 tensor like q")
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, S]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
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
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        elif t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 tensor like q")
        grads.append(t)
    need = _native.attn_bwd_workspace_size(B, S, H)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
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
