// vdx_attn_api.hip -- the C ABI declared in include/vdx_attn.h: argument
// validation (before any HIP call), the per-device architecture check, and
// the hand-off to the gfx950 launchers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "attn_fwd_launch.h"
#include "vdx_attn.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = something else / query failed.
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VDX_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int c = g_arch_ok[dev].load(std::memory_order_acquire);
        if (c == 1) return VDX_OK;
        if (c == 2) return VDX_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    int ok = 2;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
        ok = 1;
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok, std::memory_order_release);
    return ok == 1 ? VDX_OK : VDX_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int validate(const void* q, const void* k, const void* v, const int32_t* seg_q,
             const int32_t* seg_kv, const void* out, const float* lse, int B, int S, int H, int D,
             float scale) {
    if (!q || !k || !v || !out || !lse) return VDX_ERR_NULL_PTR;
    if ((seg_q == nullptr) != (seg_kv == nullptr)) return VDX_ERR_SEG_PAIR;
    if (B < 1 || S < 1 || H < 1) return VDX_ERR_SHAPE;
    if (D > 0) {
        const __int128 n = (__int128)B * S * H * D;
        if (n > (__int128)INT64_MAX / 2) return VDX_ERR_SHAPE;
    }
    const int64_t bq = vdx::queries_per_workgroup();
    const int64_t n_wg = (int64_t)B * H * ((S + bq - 1) / bq);
    if (n_wg > INT32_MAX) return VDX_ERR_SHAPE;
    if (seg_q && (int64_t)S > vdx::max_masked_seq()) return VDX_ERR_SHAPE;
    // Per-tile element offsets (64 tokens x H*D) are kept in 32 bits.
    if (D > 0 && (int64_t)64 * H * D > INT32_MAX) return VDX_ERR_SHAPE;
    if (D != 64 && D != 128) return VDX_ERR_HEAD_DIM;
    if (!std::isfinite(scale) || !(scale > 0.f)) return VDX_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return VDX_ERR_ALIGN;
    if (!aligned(lse, 4) || (seg_q && (!aligned(seg_q, 4) || !aligned(seg_kv, 4))))
        return VDX_ERR_ALIGN;
    return VDX_OK;
}

int validate_natten(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    int B, int NT, int NH, int NW, int H, int D, int KT, int KH, int KW, float scale) {
    if (!q || !k || !v || !out || !lse) return VDX_ERR_NULL_PTR;
    if (B < 1 || NT < 1 || NH < 1 || NW < 1 || H < 1) return VDX_ERR_SHAPE;
    const int64_t S = (int64_t)NT * NH * NW;
    if (S > INT32_MAX) return VDX_ERR_SHAPE;
    if (D > 0) {
        const __int128 n = (__int128)B * S * H * D;
        if (n > (__int128)INT64_MAX / 2) return VDX_ERR_SHAPE;
        if ((int64_t)64 * H * D > INT32_MAX) return VDX_ERR_SHAPE;
    }
    vdx::NattenArgs a{q, k, v, nullptr, nullptr, B, NT, NH, NW, H, D, KT, KH, KW, scale};
    if (vdx::natten_workgroups(a) > INT32_MAX) return VDX_ERR_SHAPE;
    if (D != 64 && D != 128) return VDX_ERR_HEAD_DIM;
    if (KT < 1 || KH < 1 || KW < 1 || KT % 2 == 0 || KH % 2 == 0 || KW % 2 == 0) return VDX_ERR_WINDOW;
    if ((KW < NW ? KW : NW) > vdx::kNattenMaxWindowX) return VDX_ERR_WINDOW;
    if (!std::isfinite(scale) || !(scale > 0.f)) return VDX_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return VDX_ERR_ALIGN;
    if (!aligned(lse, 4)) return VDX_ERR_ALIGN;
    return VDX_OK;
}

int validate_bwd_args(const void* q, const void* k, const void* v, const int32_t* seg_q,
                      const int32_t* seg_kv, const void* out, const float* lse, const void* dout,
                      const void* dq, const void* dk, const void* dv, int B, int S, int H, int D,
                      float scale) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return VDX_ERR_NULL_PTR;
    if ((seg_q == nullptr) != (seg_kv == nullptr)) return VDX_ERR_SEG_PAIR;
    if (B < 1 || S < 1 || H < 1) return VDX_ERR_SHAPE;
    if (S > INT32_MAX - 64) return VDX_ERR_SHAPE;
    if (D > 0) {
        const __int128 n = (__int128)B * S * H * D;
        if (n > (__int128)INT64_MAX / 2) return VDX_ERR_SHAPE;
        if ((int64_t)64 * H * D > INT32_MAX) return VDX_ERR_SHAPE;
    }
    const int64_t rows = vdx::bwd_rows_per_workgroup();
    if ((int64_t)B * H * ((S + rows - 1) / rows) > INT32_MAX) return VDX_ERR_SHAPE;
    if (seg_q && (int64_t)S > vdx::bwd_max_masked_seq()) return VDX_ERR_SHAPE;
    if (D != 64 && D != 128) return VDX_ERR_HEAD_DIM;
    if (!std::isfinite(scale) || !(scale > 0.f)) return VDX_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return VDX_ERR_ALIGN;
    if (!aligned(lse, 4) || (seg_q && (!aligned(seg_q, 4) || !aligned(seg_kv, 4))))
        return VDX_ERR_ALIGN;
    return VDX_OK;
}

int validate_bwd(const void* q, const void* k, const void* v, const int32_t* seg_q,
                 const int32_t* seg_kv, const void* out, const float* lse, const void* dout,
                 const void* dq, const void* dk, const void* dv, const void* ws, size_t ws_bytes,
                 int B, int S, int H, int D, float scale) {
    const int rc = validate_bwd_args(q, k, v, seg_q, seg_kv, out, lse, dout, dq, dk, dv, B, S, H, D, scale);
    if (rc != VDX_OK) return rc;
    if (!ws || !aligned(ws, 16) || ws_bytes < vdx::attn_bwd_workspace_bytes(B, S, H))
        return VDX_ERR_WORKSPACE;
    return VDX_OK;
}

// ---- the allocation-free backward's scratch ---------------------------------------
// One file-scope device array: every GPU the library runs on holds its own copy
// (at its own address) until the process ends.  Host code never uses the
// array's name as an address: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) unsigned char scratch[VDX_BWD_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VDX_ERR_DEVICE;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return VDX_ERR_DEVICE;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return VDX_OK;
}

int validate_rope(const vdx_rope3d* r, int D, vdx::Rope3DDev& dev) {
    if (!r || !r->pos || !aligned(r->pos, 4)) return VDX_ERR_ROPE;
    int64_t sum = 0;
    for (int a = 0; a < 3; ++a) {
        if (r->dims[a] < 0 || r->dims[a] % 2 != 0 || r->n[a] < 0) return VDX_ERR_ROPE;
        if (r->dims[a] > 0 && (!r->cos_tab[a] || !r->sin_tab[a] || !aligned(r->cos_tab[a], 4) ||
                               !aligned(r->sin_tab[a], 4)))
            return VDX_ERR_ROPE;
        sum += r->dims[a];
    }
    if (sum > D) return VDX_ERR_ROPE;
    dev.pos = r->pos;
    for (int a = 0; a < 3; ++a) {
        dev.cs[a] = r->cos_tab[a];
        dev.sn[a] = r->sin_tab[a];
        // A section of width 0 reads no table; its rows only decide which
        // tokens are inside.
        dev.n[a] = r->n[a];
        dev.d[a] = r->dims[a];
    }
    dev.interleaved = r->interleaved ? 1 : 0;
    return VDX_OK;
}

int validate_rope_apply(const void* x, const void* y, const vdx_rope3d* r, int B, int S, int H, int D,
                        vdx::Rope3DDev& dev) {
    if (!x || !y) return VDX_ERR_NULL_PTR;
    if (B < 1 || S < 1 || H < 1) return VDX_ERR_SHAPE;
    if (D > 0) {
        const __int128 n = (__int128)B * S * H * D;
        if (n > (__int128)INT64_MAX / 2) return VDX_ERR_SHAPE;
    }
    if (D != 64 && D != 128) return VDX_ERR_HEAD_DIM;
    if (!aligned(x, 16) || !aligned(y, 16)) return VDX_ERR_ALIGN;
    return validate_rope(r, D, dev);
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int vdx_attn_fwd(
    const void* q, const void* k, const void* v, const int32_t* seg_q, const int32_t* seg_kv,
    void* out, float* lse, int B, int S, int H, int D, float scale, hipStream_t stream) {
    int rc = validate(q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale);
    if (rc != VDX_OK) return rc;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    vdx::AttnArgs a{q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale};
    if (vdx::launch_attn_fwd(a, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) int vdx_attn_fwd_ws(
    const void* q, const void* k, const void* v, const int32_t* seg_q, const int32_t* seg_kv,
    void* out, float* lse, void* workspace, size_t workspace_bytes, int B, int S, int H, int D, float scale,
    hipStream_t stream) {
    int rc = validate(q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale);
    if (rc != VDX_OK) return rc;
    if ((seg_q || workspace) &&
        (!workspace || !aligned(workspace, 16) || workspace_bytes < vdx::attn_fwd_workspace_bytes(B, S)))
        return VDX_ERR_WORKSPACE;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    vdx::AttnArgs a{q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale};
    if (vdx::launch_attn_fwd_sched(a, workspace, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) size_t vdx_attn_fwd_workspace_size(int B, int S, int H) {
    if (B < 1 || S < 1 || H < 1) return 0;
    return vdx::attn_fwd_workspace_bytes(B, S);
}

__attribute__((visibility("default"))) int vdx_natten3d_fwd(
    const void* q, const void* k, const void* v, void* out, float* lse, int B, int NT, int NH, int NW,
    int H, int D, int KT, int KH, int KW, float scale, hipStream_t stream) {
    int rc = validate_natten(q, k, v, out, lse, B, NT, NH, NW, H, D, KT, KH, KW, scale);
    if (rc != VDX_OK) return rc;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    vdx::NattenArgs a{q, k, v, out, lse, B, NT, NH, NW, H, D, KT, KH, KW, scale};
    if (vdx::launch_natten_fwd(a, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) int vdx_attn_bwd(
    const void* q, const void* k, const void* v, const int32_t* seg_q, const int32_t* seg_kv,
    const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
    void* workspace, size_t workspace_bytes, int B, int S, int H, int D, float scale,
    hipStream_t stream) {
    int rc = validate_bwd(q, k, v, seg_q, seg_kv, out, lse, dout, dq, dk, dv, workspace,
                          workspace_bytes, B, S, H, D, scale);
    if (rc != VDX_OK) return rc;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    vdx::BwdArgs a{q, k, v, seg_q, seg_kv, out, lse, dout, dq, dk, dv, workspace, B, S, H, D, scale};
    if (vdx::launch_attn_bwd(a, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) int vdx_rope3d_apply(const void* x, void* y, const vdx_rope3d* rope,
                                                            int B, int S, int H, int D, hipStream_t stream) {
    vdx::Rope3DDev dev{};
    int rc = validate_rope_apply(x, y, rope, B, S, H, D, dev);
    if (rc != VDX_OK) return rc;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    if (vdx::launch_rope3d_apply(x, y, dev, B, S, H, D, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) int vdx_rope3d_attn_fwd(
    const void* q, const void* k, const void* v, const int32_t* seg_q, const int32_t* seg_kv,
    const vdx_rope3d* rope, void* k_rot, void* out, float* lse, int B, int S, int H, int D, float scale,
    hipStream_t stream) {
    if (!k_rot && q && k && v && out && lse) return VDX_ERR_NULL_PTR;
    int rc = validate(q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale);
    if (rc != VDX_OK) return rc;
    if (!aligned(k_rot, 16)) return VDX_ERR_ALIGN;
    vdx::Rope3DDev dev{};
    rc = validate_rope(rope, D, dev);
    if (rc != VDX_OK) return rc;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    if (vdx::launch_rope3d_apply(k, k_rot, dev, B, S, H, D, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    vdx::AttnArgs a{q, k_rot, v, seg_q, seg_kv, out, lse, B, S, H, D, scale};
    if (vdx::launch_rope3d_attn_fwd(a, dev, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) int vdx_rope3d_attn_fwd_ws(
    const void* q, const void* k, const void* v, const int32_t* seg_q, const int32_t* seg_kv,
    const vdx_rope3d* rope, void* k_rot, void* out, float* lse, void* workspace, size_t workspace_bytes, int B,
    int S, int H, int D, float scale, hipStream_t stream) {
    if (!k_rot && q && k && v && out && lse) return VDX_ERR_NULL_PTR;
    int rc = validate(q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale);
    if (rc != VDX_OK) return rc;
    if (!aligned(k_rot, 16)) return VDX_ERR_ALIGN;
    vdx::Rope3DDev dev{};
    rc = validate_rope(rope, D, dev);
    if (rc != VDX_OK) return rc;
    if ((seg_q || workspace) &&
        (!workspace || !aligned(workspace, 16) || workspace_bytes < vdx::attn_fwd_workspace_bytes(B, S)))
        return VDX_ERR_WORKSPACE;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    if (vdx::launch_rope3d_apply(k, k_rot, dev, B, S, H, D, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    vdx::AttnArgs a{q, k_rot, v, seg_q, seg_kv, out, lse, B, S, H, D, scale};
    if (vdx::launch_rope3d_attn_fwd_sched(a, dev, workspace, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) int vdx_attn_bwd_noalloc(
    const void* q, const void* k, const void* v, const int32_t* seg_q, const int32_t* seg_kv,
    const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int S,
    int H, int D, float scale, hipStream_t stream) {
    int rc = validate_bwd_args(q, k, v, seg_q, seg_kv, out, lse, dout, dq, dk, dv, B, S, H, D, scale);
    if (rc != VDX_OK) return rc;
    if (vdx::attn_bwd_workspace_bytes(B, S, H) > (size_t)VDX_BWD_NOALLOC_SCRATCH_BYTES) return VDX_ERR_SCRATCH;
    rc = check_device();
    if (rc != VDX_OK) return rc;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != VDX_OK) return rc;
    vdx::BwdArgs a{q, k, v, seg_q, seg_kv, out, lse, dout, dq, dk, dv, ws, B, S, H, D, scale};
    if (vdx::launch_attn_bwd(a, stream) != hipSuccess) return VDX_ERR_LAUNCH;
    return VDX_OK;
}

__attribute__((visibility("default"))) size_t vdx_attn_bwd_workspace_size(int B, int S, int H) {
    if (B < 1 || S < 1 || H < 1 || S > INT32_MAX - 64) return 0;
    const __int128 n = (__int128)B * H * (((int64_t)S + 63) / 64 * 64) * 8 +
                       (__int128)B * (((int64_t)S + 127) / 128) * 16;
    if (n > (__int128)INT64_MAX) return 0;
    return vdx::attn_bwd_workspace_bytes(B, S, H);
}

__attribute__((visibility("default"))) const char* vdx_status_str(int status) {
    switch (status) {
        case VDX_OK: return "VDX_OK";
        case VDX_ERR_NULL_PTR: return "VDX_ERR_NULL_PTR: q, k, v, out or lse is NULL";
        case VDX_ERR_SEG_PAIR: return "VDX_ERR_SEG_PAIR: exactly one of seg_q/seg_kv is NULL";
        case VDX_ERR_SHAPE: return "VDX_ERR_SHAPE: batch, sequence, grid or head count out of range";
        case VDX_ERR_HEAD_DIM: return "VDX_ERR_HEAD_DIM: D must be 64 or 128";
        case VDX_ERR_SCALE: return "VDX_ERR_SCALE: scale must be finite and > 0";
        case VDX_ERR_ALIGN: return "VDX_ERR_ALIGN: q/k/v/out need 16-byte, seg/lse 4-byte alignment";
        case VDX_ERR_DEVICE: return "VDX_ERR_DEVICE: current device is not gfx950";
        case VDX_ERR_LAUNCH: return "VDX_ERR_LAUNCH: kernel launch failed";
        case VDX_ERR_WINDOW:
            return "VDX_ERR_WINDOW: window sizes must be odd and >= 1, the x window at most 13";
        case VDX_ERR_WORKSPACE:
            return "VDX_ERR_WORKSPACE: workspace NULL, misaligned or smaller than the call's workspace size";
        case VDX_ERR_SCRATCH:
            return "VDX_ERR_SCRATCH: the call needs more scratch than vdx_attn_bwd_noalloc's static buffer holds";
        case VDX_ERR_ROPE:
            return "VDX_ERR_ROPE: rotary embedding description NULL, or a section width, row count, table or "
                   "position pointer invalid";
        default: return "VDX_ERR_UNKNOWN";
    }
}

__attribute__((visibility("default"))) int vdx_abi_version(void) { return VDX_ABI_VERSION; }

}  // extern "C"
