// rope3d.h -- device pieces of the 3D rotary position embedding of queries and
// keys: which feature pairs an axis rotates, the rotation of one feature, and
// the rounding of its fp64 value to bf16.  Shared by the key pre-pass
// (rope3d_kernel.hip) and the query prologue of the attention kernel, so that
// both produce the same bits for the same feature.
//
// The operation (vidax paper, arXiv:2609.18077, section 2 "3D RoPE, 3D VAEs,
// and flash attention"; section 3.1 for the 3D-RoPE DiT families): queries and
// keys are rotated by a rotary position embedding over time, height and width
// right before attention, each family with its own convention; no formula is
// printed.  The caller supplies every family-specific choice:
//   * features [0, d_t), [d_t, d_t + d_h), [d_t + d_h, d_t + d_h + d_w) belong
//     to the t, y and x axes (later features are not rotated);
//   * pair p of an axis section at offset o and width w is (o + 2p, o + 2p + 1)
//     (interleaved) or (o + p, o + p + w/2) (split halves);
//   * its angle is given by cos / sin tables [n_a][w/2] (fp32) at the token's
//     coordinate on that axis;
//   * (x0, x1) -> (x0 c - x1 s, x0 s + x1 c), formed in fp64 (a bf16 times an
//     fp32 value is exact there, so the sum is rounded once) and rounded once
//     to bf16, to nearest, ties to even;
//   * a token with any coordinate outside its table (< 0 or >= n_a) is not
//     rotated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_launch.h"

namespace vdx {

namespace {

// Role of feature f of a token inside the tables: whether it is rotated, the
// index of its pair partner, whether it is the pair's first feature, and the
// table and entry its angle comes from.
struct RopeFeature {
    bool rot;
    bool first;
    int partner;
    int axis;
    int entry;  // row * (d_a / 2) + p
};

__device__ __forceinline__ RopeFeature rope_feature(const Rope3DDev& r, int f, const int (&pos)[3]) {
    RopeFeature out{false, false, f, 0, 0};
    int off = 0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const int w = r.d[a], half = w >> 1;
        if (!out.rot && f >= off && f < off + w) {
            const int l = f - off;
            int p;
            if (r.interleaved) {
                p = l >> 1;
                out.first = (l & 1) == 0;
                out.partner = out.first ? f + 1 : f - 1;
            } else {
                out.first = l < half;
                p = out.first ? l : l - half;
                out.partner = out.first ? f + half : f - half;
            }
            out.rot = true;
            out.axis = a;
            out.entry = pos[a] * half + p;
        }
        off += w;
    }
    return out;
}

// Angle of a rotated feature (selects instead of an indexed kernel-argument
// array, which would be copied to scratch memory).
__device__ __forceinline__ float rope_cos(const Rope3DDev& r, const RopeFeature& ft) {
    const float* t = ft.axis == 0 ? r.cs[0] : (ft.axis == 1 ? r.cs[1] : r.cs[2]);
    return t[ft.entry];
}
__device__ __forceinline__ float rope_sin(const Rope3DDev& r, const RopeFeature& ft) {
    const float* t = ft.axis == 0 ? r.sn[0] : (ft.axis == 1 ? r.sn[1] : r.sn[2]);
    return t[ft.entry];
}

// Whether (t, y, x) lies inside all three tables.
__device__ __forceinline__ bool rope_inside(const Rope3DDev& r, const int (&pos)[3]) {
    return pos[0] >= 0 && pos[0] < r.n[0] && pos[1] >= 0 && pos[1] < r.n[1] && pos[2] >= 0 &&
           pos[2] < r.n[2];
}

// bf16 bits of y rounded to nearest, ties to even, in two exact steps: y to
// fp32 with round-to-odd (the fp32 truncation with its last bit set whenever
// the conversion is inexact), then fp32 to bf16 by round-to-nearest-even.
// fp32 keeps 16 more significand bits than bf16 (at least 2 more in the
// subnormal range), so the odd last bit only breaks ties that the exact value
// would not have had.
__device__ __forceinline__ uint16_t bf16_rne_from_f64(double y) {
    const float f = (float)y;
    uint32_t u = __float_as_uint(f);
    const double back = (double)f;
    if (back != y) {
        if (fabs(back) > fabs(y)) u -= 1u;
        u |= 1u;
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Rotated value of a feature with value x whose pair partner has value xp.
__device__ __forceinline__ uint16_t rope_rotate(float x, float xp, float c, float s, bool first) {
    const double xd = x, pd = xp, cd = c, sd = s;
    const double y = first ? xd * cd - pd * sd : pd * sd + xd * cd;
    return bf16_rne_from_f64(y);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace
}  // namespace vdx
