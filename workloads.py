"""Seeded synthetic workloads for segment-masked video-DiT self-attention.

This module only *generates inputs*: shapes, seeds, value distributions and
per-token segment-ID layouts.  It contains none of the attention arithmetic,
so both the CPU oracle (``oracle/``) and the HIP path may be fed from it.

Provenance of the shapes (vidax paper, arXiv:2609.18077):
  * the token volume is frames x h x w latent patches flattened into one
    sequence that reaches tens of thousands of tokens (section 1,
    "Spatiotemporal constraints in video generation");
  * padding and packed clips are expressed as per-token SegmentIds instead of a
    dense (B, H, Sq, Sk) mask (Appendix A, Table 4, group 2, HunyuanVideo-1.5
    row);
  * classifier-free guidance doubles the internal batch (section 4,
    "Experimental setup").
The latent grids, head counts and head dims below are synthetic stand-ins for
the layers of Table 5's models; the pages print no activation statistics, so
Q/K/V are drawn i.i.d. normal and rounded to bf16 (round-to-nearest-even).

Generation recipe (fixed; the same bits go to the oracle and the GPU):
  Q, K, V are drawn one after the other, each from its own
  ``torch.Generator().manual_seed(seed_x)`` as float32 ``randn`` of shape
  [B, S, H, D], multiplied by sigma, then cast to bfloat16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import torch

# A segment layout is a list of (start, stop, seg_id) runs covering [0, S).
SegRuns = List[Tuple[int, int, int]]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int
    D: int
    scale: float
    seeds: Tuple[int, int, int]
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    # None -> no segment arrays (unmasked); otherwise the per-batch runs.
    seg_runs: Optional[SegRuns] = None
    note: str = ""

    @property
    def masked(self) -> bool:
        return self.seg_runs is not None


def _runs_cover(runs: SegRuns, S: int) -> bool:
    pos = 0
    for a, b, _ in runs:
        if a != pos or b <= a:
            return False
        pos = b
    return pos == S


# --- the five workloads ------------------------------------------------------
# tiny_ref: 4x16x16 patch grid, small enough for the full oracle in seconds.
TINY_REF = Workload(
    name="tiny_ref", B=1, S=1024, H=4, D=64, scale=1.0 / 8.0,
    seeds=(1000, 1001, 1002), seg_runs=[(0, 1024, 1)],
    note="4x16x16 patch grid, single segment passed as arrays")

# 480p small-DiT layer: 21x30x52 latent patch grid (Wan2.1 1.3B at 832x480,
# 81 frames is the page workload it stands for; Table 5).
SMALL_DIT_480P = Workload(
    name="dit480p_small", B=1, S=32760, H=12, D=128,
    scale=1.0 / math.sqrt(128.0), seeds=(2000, 2001, 2002), seg_runs=None,
    note="21x30x52 latent patch grid, no mask")

# Joint video+text attention with padding (CogVideoX 5B at 720x480, 49 frames,
# CFG batch 2): 13x30x45 video tokens + 226 text tokens, padded to 17,920.
JOINT_VIDEO_TEXT = Workload(
    name="joint_video_text_pad", B=2, S=17920, H=24, D=128,
    scale=1.0 / math.sqrt(128.0), seeds=(3000, 3001, 3002),
    seg_runs=[(0, 17550, 1), (17550, 17776, 1), (17776, 17920, 0)],
    note="17,550 video + 226 text tokens (seg 1), 144 pad tokens (seg 0)")

# 720p large-DiT layer: 21x45x80 latent patch grid, all 40 heads on one GPU
# (Wan2.1 14B at 1280x720, 81 frames; Table 5 and section 4's offload sweep).
LARGE_DIT_720P = Workload(
    name="dit720p_large", B=1, S=75600, H=40, D=128,
    scale=1.0 / math.sqrt(128.0), seeds=(4000, 4001, 4002), seg_runs=None,
    note="21x45x80 latent patch grid, no mask")

# Packed variable-length clips: 4 clips + 14 pad tokens, distinct seg IDs,
# Q/K with sigma 3 to stress the softmax range.
PACKED_CLIPS = Workload(
    name="packed_clips", B=1, S=61440, H=16, D=128,
    scale=1.0 / math.sqrt(128.0), seeds=(5000, 5001, 5002), sigma_qk=3.0,
    seg_runs=[(0, 4096, 1), (4096, 12286, 2), (12286, 28666, 3),
              (28666, 61426, 4), (61426, 61440, 0)],
    note="clips of 4,096 / 8,190 / 16,380 / 32,760 tokens + 14 pad")

WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in (TINY_REF, SMALL_DIT_480P, JOINT_VIDEO_TEXT,
                        LARGE_DIT_720P, PACKED_CLIPS)
}
# The workload the throughput line is quoted on.
HEADLINE = LARGE_DIT_720P.name

for _w in WORKLOADS.values():
    if _w.seg_runs is not None:
        assert _runs_cover(_w.seg_runs, _w.S), _w.name


# --- 3D neighbourhood attention ----------------------------------------------
@dataclass(frozen=True)
class NattenWorkload:
    """A t x h x w token grid (flattened (t, y, x), x fastest) with an odd
    per-axis window.  The pages give the window of the neighbourhood-attention
    VAE decoder (11 x 11 x 11, Appendix A, Table 4, group 4) but no grid,
    head count or head dim, so those are synthetic stand-ins."""
    name: str
    B: int
    grid: Tuple[int, int, int]
    window: Tuple[int, int, int]
    H: int
    D: int
    scale: float
    seeds: Tuple[int, int, int]
    note: str = ""

    @property
    def S(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]


NATTEN_TINY = NattenWorkload(
    "natten_tiny", B=1, grid=(4, 6, 40), window=(3, 5, 11), H=2, D=64, scale=1.0 / 8.0,
    seeds=(6000, 6001, 6002), note="small grid the oracle finishes in seconds; border-heavy")
NATTEN_VAE = NattenWorkload(
    "natten_vae_decoder", B=1, grid=(16, 32, 64), window=(11, 11, 11), H=8, D=128,
    scale=1.0 / math.sqrt(128.0), seeds=(7000, 7001, 7002),
    note="synthetic stand-in for a video VAE decoder stage with an 11x11x11 window")
NATTEN_WORKLOADS: Dict[str, NattenWorkload] = {w.name: w for w in (NATTEN_TINY, NATTEN_VAE)}


def make_natten_inputs(w: NattenWorkload) -> Dict[str, torch.Tensor]:
    """CPU tensors q, k, v (bf16 [B, S, H, D]), same recipe as the workloads."""
    shape = (w.B, w.S, w.H, w.D)
    return {"q": randn_bf16(shape, w.seeds[0]), "k": randn_bf16(shape, w.seeds[1]),
            "v": randn_bf16(shape, w.seeds[2])}


# --- generators --------------------------------------------------------------
def randn_bf16(shape: Sequence[int], seed: int, sigma: float = 1.0) -> torch.Tensor:
    """float32 N(0, sigma^2) from a seeded CPU generator, rounded to bf16."""
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def seg_from_runs(runs: SegRuns, B: int, S: int) -> torch.Tensor:
    """int32 [B, S] segment IDs, the same runs in every batch row."""
    seg = torch.empty(S, dtype=torch.int32)
    for a, b, sid in runs:
        seg[a:b] = sid
    return seg.unsqueeze(0).expand(B, S).contiguous()


def make_inputs(w: Workload) -> Dict[str, Optional[torch.Tensor]]:
    """CPU tensors q, k, v (bf16 [B,S,H,D]) and seg_q, seg_kv (int32 [B,S] or None)."""
    shape = (w.B, w.S, w.H, w.D)
    q = randn_bf16(shape, w.seeds[0], w.sigma_qk)
    k = randn_bf16(shape, w.seeds[1], w.sigma_qk)
    v = randn_bf16(shape, w.seeds[2], w.sigma_v)
    seg = seg_from_runs(w.seg_runs, w.B, w.S) if w.seg_runs is not None else None
    return {"q": q, "k": k, "v": v, "seg_q": seg,
            "seg_kv": None if seg is None else seg.clone()}


def make_random(B: int, S: int, H: int, D: int, seed: int, sigma_qk: float = 1.0,
                sigma_v: float = 1.0) -> Dict[str, torch.Tensor]:
    """Ad-hoc seeded q, k, v for shape sweeps (same recipe as the workloads)."""
    shape = (B, S, H, D)
    return {"q": randn_bf16(shape, seed, sigma_qk),
            "k": randn_bf16(shape, seed + 1, sigma_qk),
            "v": randn_bf16(shape, seed + 2, sigma_v)}


def random_segments(B: int, S: int, seed: int, kind: str) -> torch.Tensor:
    """Seeded int32 [B, S] segment layouts used by the parity sweeps.

    kinds: "single" (all 1), "padded" (ones then a pad tail of 0),
    "packed" (contiguous runs of random length, IDs 1..n, pad tail),
    "interleaved" (random IDs in {0,1,2,3} per token, so segments are
    non-contiguous), "singletons" (every token its own ID),
    "allpad" (every token 0), "negative" (contiguous runs of random length
    with negative IDs -1, -2, ..., interrupted by pad runs of 0, and a run of
    ID 1 that shares no token with a negative run), "extreme" (runs of the
    int32 extremes -2^31 and 2^31 - 1, their neighbours -2^31 + 1 and
    2^31 - 2, -1, 1 and 0 in random order and lengths, each ID possibly in
    several non-adjacent runs).
    """
    g = torch.Generator().manual_seed(int(seed))
    seg = torch.zeros(B, S, dtype=torch.int32)
    for b in range(B):
        if kind == "single":
            seg[b] = 1
        elif kind == "padded":
            n_pad = int(torch.randint(0, max(1, S // 4) + 1, (1,), generator=g))
            seg[b, : S - n_pad] = 1
        elif kind == "packed":
            pos, sid = 0, 1
            n_pad = int(torch.randint(0, max(1, S // 8) + 1, (1,), generator=g))
            real = S - n_pad
            while pos < real:
                ln = int(torch.randint(1, max(2, real // 3) + 1, (1,), generator=g))
                seg[b, pos: min(real, pos + ln)] = sid
                pos += ln
                sid += 1
        elif kind == "interleaved":
            seg[b] = torch.randint(0, 4, (S,), generator=g, dtype=torch.int32)
        elif kind == "singletons":
            seg[b] = torch.arange(1, S + 1, dtype=torch.int32)
        elif kind == "allpad":
            pass
        elif kind == "negative":
            pos, sid = 0, -1
            while pos < S:
                ln = int(torch.randint(1, max(2, S // 4) + 1, (1,), generator=g))
                r = int(torch.randint(0, 5, (1,), generator=g))
                seg[b, pos: pos + ln] = 0 if r == 0 else (1 if r == 1 else sid)
                if r >= 2:
                    sid -= 1
                pos += ln
        elif kind == "extreme":
            ids = torch.tensor([-2 ** 31, 2 ** 31 - 1, -2 ** 31 + 1, 2 ** 31 - 2, -1, 1, 0],
                               dtype=torch.int64)
            pos = 0
            while pos < S:
                ln = int(torch.randint(1, max(2, S // 6) + 1, (1,), generator=g))
                sid = int(ids[int(torch.randint(0, len(ids), (1,), generator=g))])
                seg[b, pos: pos + ln] = sid
                pos += ln
        else:
            raise ValueError(kind)
    return seg


def bf16_bits(t: torch.Tensor):
    """uint16 numpy view of a CPU bf16 tensor (the exact bits)."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view("uint16")


# --- 3D rotary position embedding of queries and keys -----------------------------
# The pages say the video DiTs rotate queries and keys by a 3D rotary position
# embedding over (t, y, x) before attention, with per-family conventions
# (vidax paper, section 2, "3D RoPE, 3D VAEs, and flash attention"), and give
# no formula, head-dim split or frequency schedule.  The inputs below are
# synthetic: per-axis angle tables from the geometric frequency schedule of
# the rotary position embedding (angle(pos, p) = pos * theta^(-2p / d_a),
# theta = 10,000), a split of the head dim into three even sections whose pair
# counts are not multiples of 8, and the (t, y, x) of every video token of
# each clip's latent grid; other tokens (text, padding) get (-1, -1, -1) and
# stay unrotated.

@dataclass(frozen=True)
class Rope3D:
    """Per-token positions and per-axis tables of a 3D rotary embedding."""
    pos: torch.Tensor                 # int32 [B, S, 3]
    cos: Tuple[torch.Tensor, ...]     # fp32 [n_a, d_a / 2] for a = t, y, x
    sin: Tuple[torch.Tensor, ...]
    dims: Tuple[int, int, int]        # (d_t, d_h, d_w)
    interleaved: bool = True

    def numpy(self):
        """(pos, cos, sin) as numpy arrays, for the oracle."""
        return (self.pos.numpy(), tuple(c.numpy() for c in self.cos),
                tuple(s.numpy() for s in self.sin))


ROPE_DIMS = {64: (20, 22, 22), 128: (44, 42, 42)}
ROPE_THETA = 10000.0

# Latent grids (t, y, x) of the video tokens of each workload: (first token, grid).
ROPE_GRIDS: Dict[str, List[Tuple[int, Tuple[int, int, int]]]] = {
    "tiny_ref": [(0, (4, 16, 16))],
    "dit480p_small": [(0, (21, 30, 52))],
    "joint_video_text_pad": [(0, (13, 30, 45))],     # the 226 text tokens and the padding stay unrotated
    "dit720p_large": [(0, (21, 45, 80))],
    "packed_clips": [(0, (16, 16, 16)), (4096, (7, 30, 39)), (12286, (13, 30, 42)),
                     (28666, (21, 30, 52))],
}


def rope3d_tables(n: int, d: int, theta: float = ROPE_THETA) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp32 cos / sin [n, d/2] of angle(pos, p) = pos * theta^(-2p/d),
    evaluated in fp64 and rounded to fp32."""
    half = d // 2
    p = torch.arange(half, dtype=torch.float64)
    freq = theta ** (-2.0 * p / d) if d > 0 else p
    ang = torch.arange(n, dtype=torch.float64)[:, None] * freq[None, :]
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def grid_positions(B: int, S: int, grids: Sequence[Tuple[int, Tuple[int, int, int]]]) -> torch.Tensor:
    """int32 [B, S, 3]: (t, y, x) of token start + (t*NH + y)*NW + x of each
    grid, (-1, -1, -1) for every other token; the same in every batch row."""
    pos = torch.full((S, 3), -1, dtype=torch.int32)
    for start, (nt, nh, nw) in grids:
        n = nt * nh * nw
        assert start + n <= S
        idx = torch.arange(n, dtype=torch.int32)
        pos[start:start + n, 0] = idx // (nh * nw)
        pos[start:start + n, 1] = (idx // nw) % nh
        pos[start:start + n, 2] = idx % nw
    return pos.unsqueeze(0).expand(B, S, 3).contiguous()


def make_rope3d(B: int, S: int, D: int, grids: Sequence[Tuple[int, Tuple[int, int, int]]],
                interleaved: bool = True, dims: Optional[Tuple[int, int, int]] = None) -> Rope3D:
    """Positions of the given grids and tables covering the largest extent of
    each axis."""
    dims = ROPE_DIMS[D] if dims is None else tuple(dims)
    n = [max(g[1][a] for g in grids) if grids else 1 for a in range(3)]
    tabs = [rope3d_tables(n[a], dims[a]) for a in range(3)]
    return Rope3D(pos=grid_positions(B, S, grids), cos=tuple(t[0] for t in tabs),
                  sin=tuple(t[1] for t in tabs), dims=dims, interleaved=interleaved)


def workload_rope3d(w: "Workload", interleaved: bool = True) -> Rope3D:
    return make_rope3d(w.B, w.S, w.D, ROPE_GRIDS[w.name], interleaved)


def random_positions(B: int, S: int, n: Tuple[int, int, int], seed: int,
                     outside: float = 0.1) -> torch.Tensor:
    """int32 [B, S, 3] seeded positions inside tables of n = (n_t, n_h, n_w)
    rows, with about a fraction `outside` of the tokens given a coordinate
    outside them (negative or >= n_a) on one random axis."""
    g = torch.Generator().manual_seed(int(seed))
    pos = torch.stack([torch.randint(0, max(1, n[a]), (B, S), generator=g, dtype=torch.int32)
                       for a in range(3)], dim=-1)
    sel = torch.rand(B, S, generator=g) < outside
    axis = torch.randint(0, 3, (B, S), generator=g)
    big = torch.rand(B, S, generator=g) < 0.5
    for a in range(3):
        m = sel & (axis == a)
        pos[..., a] = torch.where(m & big, torch.tensor(n[a] + 3, dtype=torch.int32), pos[..., a])
        pos[..., a] = torch.where(m & ~big, torch.tensor(-1 - a, dtype=torch.int32), pos[..., a])
    return pos.contiguous()
