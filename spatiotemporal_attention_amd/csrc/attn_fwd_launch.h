// attn_fwd_launch.h -- internal interface between the C ABI layer and the
// gfx950 kernel launcher.  Not installed; the public interface is
// include/vdx_attn.h.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace vdx {

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seg_q;   // nullptr together with seg_kv -> unmasked
    const int32_t* seg_kv;
    void* out;
    float* lse;
    int B, S, H, D;
    float scale;
};

// Enqueue the forward kernel; arguments are already validated.
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);

// Largest S accepted with segment IDs (the LDS key-tile table bound).
int64_t max_masked_seq();

// Queries per workgroup (sets the grid size).
int64_t queries_per_workgroup();

}  // namespace vdx
