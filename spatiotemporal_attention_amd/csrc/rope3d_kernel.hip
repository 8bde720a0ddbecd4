// rope3d_kernel.hip -- the 3D rotary position embedding of one bf16 [B, S, H, D]
// tensor (the rule is stated in rope3d.h), and the key pre-pass of the
// rotary-embedded attention forward.
//
// One (token, head) row of D features is handled by D/2 lanes, two adjacent
// features (4 bytes) a lane, so a row is one coalesced D*2-byte load and store.
// A feature's pair partner is fetched from the lane that holds it with a
// cross-lane permute; the row groups never straddle a wave (64 is a multiple
// of D/2), so every lane of a row has its inputs before any lane stores, and
// the output may be the input itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "attn_fwd_launch.h"
#include "rope3d.h"

namespace vdx {
namespace {

template <int D>
__global__ __launch_bounds__(256) void rope3d_apply_kernel(const uint32_t* x, uint32_t* y,
                                                           Rope3DDev r, int S, int H, int64_t n_rows) {
    constexpr int L = D / 2;  // lanes per row
    const int lane = threadIdx.x & 63;
    const int sub = lane % L;            // this lane's feature pair (2 sub, 2 sub + 1)
    const int base = lane - sub;         // first lane of the row within the wave
    const int64_t rows_per_block = 256 / L;
    for (int64_t row0 = (int64_t)blockIdx.x * rows_per_block; row0 < n_rows;
         row0 += (int64_t)gridDim.x * rows_per_block) {
        const int64_t row = row0 + threadIdx.x / L;
        const bool live = row < n_rows;
        const uint32_t w = live ? x[row * L + sub] : 0u;
        // Every lane of the wave takes part in the permutes below.
        int pos[3] = {-1, -1, -1};
        if (live) {
            const int64_t tok = row / H;  // b * S + s
#pragma unroll
            for (int a = 0; a < 3; ++a) pos[a] = r.pos[tok * 3 + a];
        }
        const bool inside = live && rope_inside(r, pos);
        uint32_t outw = w;
        uint32_t half[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int f = 2 * sub + e;
            const RopeFeature ft = rope_feature(r, f, pos);
            const int src = base + (ft.partner >> 1);
            const uint32_t pw = (uint32_t)__shfl((int)w, src, 64);
            half[e] = (w >> (16 * e)) & 0xffffu;
            if (inside && ft.rot) {
                const uint32_t pb = (pw >> (16 * (ft.partner & 1))) & 0xffffu;
                const float c = rope_cos(r, ft), s = rope_sin(r, ft);
                half[e] = rope_rotate(bf16_bits_to_f32(half[e]), bf16_bits_to_f32(pb), c, s, ft.first);
            }
        }
        outw = half[0] | (half[1] << 16);
        if (live) y[row * L + sub] = outw;
    }
}

}  // namespace

hipError_t launch_rope3d_apply(const void* x, void* y, const Rope3DDev& r, int B, int S, int H, int D,
                               hipStream_t stream) {
    const int64_t n_rows = (int64_t)B * S * H;
    const int64_t rows_per_block = 256 / (D / 2);
    const int64_t blocks = std::min<int64_t>((n_rows + rows_per_block - 1) / rows_per_block, 1 << 16);
    if (D == 128)
        hipLaunchKernelGGL(rope3d_apply_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t*>(x), reinterpret_cast<uint32_t*>(y), r, S, H,
                           n_rows);
    else
        hipLaunchKernelGGL(rope3d_apply_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t*>(x), reinterpret_cast<uint32_t*>(y), r, S, H,
                           n_rows);
    return hipGetLastError();
}

}  // namespace vdx
