"""vdx_attn_bwd_noalloc (the backward with its scratch in the library's static
per-GPU array, for callers that cannot allocate) against vdx_attn_bwd with a
caller workspace, through the C ABI: bit for bit on two calls in a row, the
second on a smaller input (the array keeps the first call's contents), with
and without segment IDs."""
import math

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _inputs(B, S, H, D, seed, kind):
    import spatiotemporal_attention_amd as vdx
    x = W.make_random(B, S, H, D, seed=seed)
    d = {n: x[n].cuda() for n in ("q", "k", "v")}
    seg = None if kind is None else W.random_segments(B, S, seed + 1, kind).cuda()
    d["dout"] = W.randn_bf16((B, S, H, D), seed + 2).cuda()
    d["seg"] = seg
    d["out"], d["lse"] = vdx.attn_fwd(d["q"], d["k"], d["v"], seg, seg, scale=1.0 / math.sqrt(D))
    return d


def _noalloc(d, scale):
    from spatiotemporal_attention_amd import _native
    B, S, H, D = d["q"].shape
    g = [torch.full_like(d["q"], float("nan")) for _ in range(3)]
    seg = 0 if d["seg"] is None else d["seg"].data_ptr()
    rc = _native.attn_bwd_noalloc_raw(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), seg, seg,
                                      d["out"].data_ptr(), d["lse"].data_ptr(), d["dout"].data_ptr(),
                                      g[0].data_ptr(), g[1].data_ptr(), g[2].data_ptr(), B, S, H, D, scale,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _native.status_str(rc)
    return g


def _with_workspace(d, scale):
    import spatiotemporal_attention_amd as vdx
    return vdx.attn_bwd(d["q"], d["k"], d["v"], d["out"], d["lse"], d["dout"], d["seg"], d["seg"], scale=scale)


@pytest.mark.parametrize("kind", [None, "packed"], ids=str)
def test_noalloc_matches_workspace_variant_twice(need_gpu, kind):
    for B, S, H, D, seed in ((2, 3000, 3, 128, 61), (1, 700, 2, 64, 71)):
        print(f"case noalloc B={B} S={S} H={H} D={D} kind={kind}", flush=True)
        d = _inputs(B, S, H, D, seed, kind)
        scale = 1.0 / math.sqrt(D)
        got = _noalloc(d, scale)
        ref = _with_workspace(d, scale)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))

