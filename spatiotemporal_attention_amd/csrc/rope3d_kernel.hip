// rope3d_kernel.hip -- the 3D rotary position embedding of one bf16 [B, S, H, D]
// tensor (the rule is stated in rope3d.h), and the key pre-pass of the
// rotary-embedded attention forward.
//
// A wave takes one token at a time: its position and each lane's angles are
// looked up once and serve all H heads of the token (the tables are read per
// token, not per element).  The heads go 64/(D/8) at a time, D/8 lanes a head
// and 8 features (16 bytes) a lane, so every head row is one coalesced load
// and one store.  A feature's pair partner is in the lane's own 16 bytes when
// pairs are interleaved (sections start at even offsets); for split halves it
// is read back from a per-wave copy of the rows in LDS.  Each row is read in
// full before it is written, so the output may be the input itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "attn_fwd_launch.h"
#include "rope3d.h"

namespace vdx {
namespace {

constexpr int kRopeWaves = 4;  // waves per block

template <int D>
__global__ __launch_bounds__(64 * kRopeWaves) void rope3d_apply_kernel(const uint4* x, uint4* y, Rope3DDev r,
                                                                       int H, int64_t n_tok) {
    constexpr int L = D / 8;   // lanes per head row
    constexpr int R = 64 / L;  // head rows per wave step
    __shared__ uint4 stage[kRopeWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane % L, rr = lane / L;
    const uint16_t* sh = reinterpret_cast<const uint16_t*>(&stage[wave][rr * L]);  // this lane's row
    for (int64_t tok = (int64_t)blockIdx.x * kRopeWaves + wave; tok < n_tok;
         tok += (int64_t)gridDim.x * kRopeWaves) {
        int pos[3];
#pragma unroll
        for (int a = 0; a < 3; ++a) pos[a] = r.pos[tok * 3 + a];
        const bool inside = rope_inside(r, pos);
        RopeFeature ft[8];
        float cs[8], sn[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ft[e] = rope_feature(r, 8 * c + e, pos);
            cs[e] = 1.f;
            sn[e] = 0.f;
            if (inside && ft[e].rot) {
                cs[e] = rope_cos(r, ft[e]);
                sn[e] = rope_sin(r, ft[e]);
            }
        }
        for (int h0 = 0; h0 < H; h0 += R) {
            const int h = h0 + rr;
            const bool live = h < H;
            const int64_t idx = (tok * H + h) * L + c;
            uint4 w = live ? x[idx] : uint4{0u, 0u, 0u, 0u};
            if (inside) {
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
                uint16_t v[8], pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (uint16_t)(wd[e >> 1] >> (16 * (e & 1)));
                if (r.interleaved) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv[e] = v[e ^ 1];
                } else {
                    stage[wave][lane] = w;
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv[e] = sh[ft[e].partner];
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                }
                uint16_t o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[e] = ft[e].rot ? rope_rotate(bf16_bits_to_f32(v[e]), bf16_bits_to_f32(pv[e]), cs[e], sn[e],
                                                   ft[e].first)
                                     : v[e];
                w = uint4{o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16),
                          o[4] | ((uint32_t)o[5] << 16), o[6] | ((uint32_t)o[7] << 16)};
            }
            if (live) y[idx] = w;
        }
    }
}

}  // namespace

hipError_t launch_rope3d_apply(const void* x, void* y, const Rope3DDev& r, int B, int S, int H, int D,
                               hipStream_t stream) {
    const int64_t n_tok = (int64_t)B * S;
    const int64_t blocks = std::min<int64_t>((n_tok + kRopeWaves - 1) / kRopeWaves, 1 << 16);
    if (D == 128)
        hipLaunchKernelGGL(rope3d_apply_kernel<128>, dim3((unsigned)blocks), dim3(64 * kRopeWaves), 0, stream,
                           reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), r, H, n_tok);
    else
        hipLaunchKernelGGL(rope3d_apply_kernel<64>, dim3((unsigned)blocks), dim3(64 * kRopeWaves), 0, stream,
                           reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), r, H, n_tok);
    return hipGetLastError();
}

}  // namespace vdx
