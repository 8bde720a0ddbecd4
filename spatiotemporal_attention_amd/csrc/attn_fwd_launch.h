// attn_fwd_launch.h -- internal interface between the C ABI layer and the
// gfx950 kernel launcher.  Not installed; the public interface is
// include/vdx_attn.h.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace vdx {

// Kernel-argument form of a 3D rotary position embedding (device pointers;
// the rule is stated in rope3d.h).
struct Rope3DDev {
    const int32_t* pos;  // [B, S, 3]: (t, y, x) of every token
    const float* cs[3];  // cos tables [n_a][d_a / 2] of the t, y, x axes
    const float* sn[3];  // sin tables, same shape
    int n[3];            // table rows per axis
    int d[3];            // even section widths, d[0] + d[1] + d[2] <= D
    int interleaved;     // 1: pairs (2p, 2p + 1); 0: (p, p + d_a / 2)
};

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

// The forward with a caller workspace of attn_fwd_workspace_bytes(B, S)
// bytes (16-byte aligned): masked calls run on a persistent grid with per-XCD
// work counters and longest-first block order, ending with a pool of items
// shared by all XCDs; unmasked calls with more items than the persistent grid
// claim items through per-XCD counters with work stealing.  Either way the
// last items are split along the keys and merged by a last kernel.  An
// unmasked call with a NULL workspace is launch_attn_fwd.
hipError_t launch_attn_fwd_sched(const AttnArgs& a, void* workspace, hipStream_t stream);

size_t attn_fwd_workspace_bytes(int64_t B, int64_t S);

// The forward kernel on 3D-rotary-embedded queries (rotated in registers as
// they are loaded) and keys (a.k must already hold the rotated keys).
hipError_t launch_rope3d_attn_fwd(const AttnArgs& a, const Rope3DDev& rope, hipStream_t stream);

// launch_rope3d_attn_fwd on the schedule of launch_attn_fwd_sched (same
// workspace; an unmasked call with a NULL workspace is launch_rope3d_attn_fwd).
hipError_t launch_rope3d_attn_fwd_sched(const AttnArgs& a, const Rope3DDev& rope, void* workspace,
                                        hipStream_t stream);

// y = the 3D rotary embedding of x (bf16 [B, S, H, D]; y may be x).
hipError_t launch_rope3d_apply(const void* x, void* y, const Rope3DDev& r, int B, int S, int H, int D,
                               hipStream_t stream);

// Largest S accepted with segment IDs (the LDS key-tile table bound).
int64_t max_masked_seq();

// Queries per workgroup (sets the grid size).
int64_t queries_per_workgroup();

}  // namespace vdx

namespace vdx {

// 3D neighbourhood attention over a t x h x w grid (tokens (t, y, x), x fastest).
struct NattenArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int B, NT, NH, NW, H, D;
    int KT, KH, KW;  // odd window sizes
    float scale;
};

// Largest effective window along x the neighbourhood kernel supports.
constexpr int kNattenMaxWindowX = 13;

// Enqueue the neighbourhood-attention kernel; arguments are already validated.
hipError_t launch_natten_fwd(const NattenArgs& a, hipStream_t stream);

// Workgroups the neighbourhood kernel launches for a call.
int64_t natten_workgroups(const NattenArgs& a);

}  // namespace vdx

namespace vdx {

// Backward of segment-masked attention.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seg_q;  // nullptr together with seg_kv -> unmasked
    const int32_t* seg_kv;
    const void* out;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    void* workspace;  // attn_bwd_workspace_bytes(B, S, H) bytes
    int B, S, H, D;
    float scale;
};

// Workspace the backward needs: per (b, h) two fp32 rows (lse2, delta) of S
// rounded up to a multiple of 64.
size_t attn_bwd_workspace_bytes(int64_t B, int64_t S, int64_t H);

// Enqueue the three backward kernels; arguments are already validated.
hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t stream);

// Largest S accepted with segment IDs, and rows per workgroup (grid size).
int64_t bwd_max_masked_seq();
int64_t bwd_rows_per_workgroup();

}  // namespace vdx
