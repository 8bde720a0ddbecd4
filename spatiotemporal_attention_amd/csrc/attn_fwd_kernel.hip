// attn_fwd_kernel.hip -- gfx950 flash-attention forward with segment-ID
// masking, for the flattened spatiotemporal token volume of a video DiT.
//
// What it computes: softmax(scale * Q K^T restricted to equal, nonzero
// segment IDs) V, plus the natural-log log-sum-exp per row (vidax paper,
// arXiv:2609.18077: section 1 "Spatiotemporal constraints in video
// generation" for full self-attention over the token volume; section 2
// "3D RoPE, 3D VAEs, and flash attention" for the flash-attention dispatch of
// its reference [2]; Appendix A, Table 4, group 2 for SegmentIds that skip
// invalid key blocks; Table 4, group 1 for masking padding).
//
// Design (CDNA4 first; the TPU Pallas kernel of the pages is prior art only):
//   * one workgroup = 8 wave64s = 256 queries of one (batch, head); each wave
//     owns 32 queries whose Q slice stays in VGPRs for the whole sweep;
//   * K and V stream through LDS in 64-key tiles, double buffered: the next
//     active tile's global loads are in flight while the current one is used;
//   * scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: every lane then owns one query column, so
//     the row max/sum need one exchange with lane^32 only, and the fp32 score
//     registers become the bf16 B operand of O^T += V^T P^T without any data
//     movement (the key order inside a 32-key block is permuted so the
//     accumulator rows line up with the operand's contraction index);
//   * V is transposed once per tile while it is copied to LDS, so each lane
//     reads its V^T operand as one 16-byte ds_read;
//   * online softmax in fp32 with exp2 and scale*log2(e) folded into one FMA;
//     the O rescale is skipped for a wave unless one of its rows' maxima grew;
//   * with segment IDs, a prologue classifies every 64-key tile against the
//     workgroup's query segments as skip / full / partial and compacts the
//     active ones into an LDS list, so fully masked tiles cost nothing and
//     only partial tiles pay for element masks;
//   * workgroups are renumbered so that each XCD (own L2) runs consecutive
//     query blocks of the same head, which then share K/V tiles in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_launch.h"

namespace vdx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBq = 32 * kWaves;  // queries per workgroup
constexpr int kBk = 64;           // keys per tile
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kMaxKvTiles = 32768;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Tile {
    static constexpr int kChunks = D / 8;               // 16-byte chunks per K row
    static constexpr int kKBytes = kBk * D * 2;         // K tile, row-major, swizzled
    static constexpr int kVBytes = D * kBk * 2;         // V^T tile, d-major, swizzled
    static constexpr int kSegOff = kKBytes + kVBytes;   // int32 seg_kv of the tile
    static constexpr int kBufBytes = kSegOff + kBk * 4;
    static constexpr int kSteps = D / 16;               // MFMA k-steps over D
    static constexpr int kDBlocks = D / 32;             // 32-row blocks of O^T
    static constexpr int kKUnits = kBk * kChunks / kThreads;      // K chunks per thread
    static constexpr int kVUnits = (kBk / 2) * kChunks;           // (key pair, chunk) units
    static_assert(kKUnits >= 1, "tile too small for the workgroup");
    static_assert(kVUnits <= kThreads, "one V unit per thread at most");
};

// Swap bits 2 and 3: maps an MFMA accumulator row inside a 32-key block to the
// physical key it holds (and back; the map is an involution).
__device__ __forceinline__ int swap23(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// LDS swizzles (16-byte chunk position inside a row) that keep the operand
// reads of one wave on distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) { return swap23(row & 31) & (Tile<D>::kChunks - 1); }
__device__ __forceinline__ int v_swz(int drow) { return (drow + (drow >> 3)) & 7; }

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

struct Staged {
    u32x4 k[4];
    u32x4 v0, v1;
    int seg;
};

// Global -> registers for key tile `t` (rows past S read as zero).
template <int D, bool SEG>
__device__ __forceinline__ void stage_load(Staged& st, const __bf16* __restrict__ kp,
                                           const __bf16* __restrict__ vp,
                                           const int32_t* __restrict__ segkv, int t, int S,
                                           int64_t tok_stride, int tid) {
    using T = Tile<D>;
    const int key0 = t * kBk;
#pragma unroll
    for (int u = 0; u < T::kKUnits; ++u) {
        const int unit = tid + u * kThreads;
        const int row = unit / T::kChunks, ch = unit % T::kChunks;
        const int key = key0 + row;
        st.k[u] = (key < S) ? ld16(kp + (int64_t)key * tok_stride + ch * 8) : u32x4{0, 0, 0, 0};
    }
    if (tid < T::kVUnits) {
        const int pair = tid / T::kChunks, ch = tid % T::kChunks;
        const int key = key0 + 2 * pair;
        st.v0 = (key < S) ? ld16(vp + (int64_t)key * tok_stride + ch * 8) : u32x4{0, 0, 0, 0};
        st.v1 = (key + 1 < S) ? ld16(vp + (int64_t)(key + 1) * tok_stride + ch * 8)
                              : u32x4{0, 0, 0, 0};
    }
    if (SEG && tid < kBk) {
        const int key = key0 + tid;
        st.seg = (key < S) ? segkv[key] : 0;
    }
}

// Registers -> LDS buffer: K row-major (swizzled), V transposed to V^T.
template <int D, bool SEG>
__device__ __forceinline__ void stage_store(const Staged& st, char* buf, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int u = 0; u < T::kKUnits; ++u) {
        const int unit = tid + u * kThreads;
        const int row = unit / T::kChunks, ch = unit % T::kChunks;
        *reinterpret_cast<u32x4*>(buf + row * (D * 2) + ((ch ^ k_swz<D>(row)) << 4)) = st.k[u];
    }
    if (tid < T::kVUnits) {
        const int pair = tid / T::kChunks, ch = tid % T::kChunks;
        const int j = 2 * pair;  // key inside the tile (even)
        char* vt = buf + T::kKBytes;
        const uint32_t a[4] = {st.v0.x, st.v0.y, st.v0.z, st.v0.w};
        const uint32_t b[4] = {st.v1.x, st.v1.y, st.v1.z, st.v1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t wa = a[e >> 1], wb = b[e >> 1];
            // (V[j][d], V[j+1][d]) as one dword, key j in the low half.
            const uint32_t pairw = (e & 1) ? ((wb & 0xffff0000u) | (wa >> 16))
                                           : ((wb << 16) | (wa & 0xffffu));
            const int drow = ch * 8 + e;
            const int off = drow * (kBk * 2) + (((j >> 3) ^ v_swz(drow)) << 4) + (j & 7) * 2;
            *reinterpret_cast<uint32_t*>(vt + off) = pairw;
        }
    }
    if (SEG && tid < kBk) reinterpret_cast<int*>(buf + T::kSegOff)[tid] = st.seg;
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}

template <int D, bool SEG>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_kv,
    __bf16* __restrict__ out, float* __restrict__ lse, int S, int H, float c_log2,
    int n_qblk, int n_kvt, int n_wg) {
    using T = Tile<D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    // ---- tile scheduler: XCD-contiguous renumbering of workgroup ids --------
    const int w = blockIdx.x;
    const int per = n_wg / kXcds, rem = n_wg % kXcds;
    const int xcd = w % kXcds;
    const int lid = xcd * per + min(xcd, rem) + w / kXcds;
    const int qblk = lid % n_qblk;
    const int bh = lid / n_qblk;
    const int h = bh % H;
    const int b = bh / H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, g = lane >> 5;
    const int q0 = qblk * kBq;
    const int qi = q0 + wave * 32 + lr;
    const bool wave_live = (q0 + wave * 32) < S;

    const int64_t tok_stride = (int64_t)H * D;
    const __bf16* kp = k + (int64_t)b * S * tok_stride + (int64_t)h * D;
    const __bf16* vp = v + (int64_t)b * S * tok_stride + (int64_t)h * D;
    const int32_t* segkv_b = SEG ? seg_kv + (int64_t)b * S : nullptr;

    // ---- Q slice -> VGPRs as the B operand of S^T = K Q^T --------------------
    bf16x8 qreg[T::kSteps];
    {
        const __bf16* qrow = q + ((int64_t)b * S + qi) * tok_stride + (int64_t)h * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) {
            if (qi < S)
                qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
            else
                qreg[ks] = bf16x8{};
        }
    }

    char* bufs = smem;                                   // 2 tile buffers
    uint16_t* list = reinterpret_cast<uint16_t*>(smem + 2 * T::kBufBytes);
    int* meta = reinterpret_cast<int*>(smem + ((2 * T::kBufBytes + 2 * (SEG ? n_kvt : 0) + 15) & ~15));
    // meta: [0..7] per-wave q min, [8..15] q max, [16..23] q flags, [24] n_active

    int myseg = 1;
    int n_act = n_kvt;
    if (SEG) {
        // ---- query-block segment summary --------------------------------------
        myseg = (qi < S) ? seg_q[(int64_t)b * S + qi] : 0;
        {
            int mn = (myseg != 0) ? myseg : INT32_MAX;
            int mx = (myseg != 0) ? myseg : INT32_MIN;
            int fl = (myseg == 0) ? 1 : 0;  // pad or out-of-range row present
            mn = wave_min(mn);
            mx = wave_max(mx);
            fl = wave_max(fl);
            if (lane == 0) {
                meta[wave] = mn;
                meta[8 + wave] = mx;
                meta[16 + wave] = fl;
            }
        }
        __syncthreads();
        int qmn = INT32_MAX, qmx = INT32_MIN, qfl = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            qmn = min(qmn, meta[i]);
            qmx = max(qmx, meta[8 + i]);
            qfl |= meta[16 + i];
        }
        // ---- classify every key tile: 0 skip, 1 full, 2 partial ---------------
        uint8_t* cls = reinterpret_cast<uint8_t*>(bufs);  // aliases the tile buffers
        for (int t = wave; t < n_kvt; t += kWaves) {
            const int key = t * kBk + lane;
            const int id = (key < S) ? segkv_b[key] : 0;
            int mn = (id != 0) ? id : INT32_MAX;
            int mx = (id != 0) ? id : INT32_MIN;
            int fl = (id == 0) ? 1 : 0;
            mn = wave_min(mn);
            mx = wave_max(mx);
            fl = wave_max(fl);
            if (lane == 0) {
                uint8_t c;
                if (qmn > qmx || mn > mx || max(qmn, mn) > min(qmx, mx))
                    c = 0;
                else if (!qfl && !fl && qmn == qmx && mn == mx && qmn == mn)
                    c = 1;
                else
                    c = 2;
                cls[t] = c;
            }
        }
        __syncthreads();
        // ---- compact active tiles into the list (wave 0, ballot prefix) -------
        if (wave == 0) {
            int base = 0;
            for (int t0 = 0; t0 < n_kvt; t0 += 64) {
                const int t = t0 + lane;
                const int c = (t < n_kvt) ? cls[t] : 0;
                const uint64_t m = __ballot(c != 0);
                const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
                if (c != 0) list[pos] = (uint16_t)(t | ((c == 2) ? 0x8000 : 0));
                base += __popcll(m);
            }
            if (lane == 0) meta[24] = base;
        }
        __syncthreads();
        n_act = meta[24];
    }

    auto tile_of = [&](int n, bool& partial) -> int {
        if (SEG) {
            const int e = __builtin_amdgcn_readfirstlane((int)list[n]);
            partial = (e & 0x8000) != 0;
            return e & 0x7fff;
        } else {
            partial = (n == n_kvt - 1) && (S % kBk != 0);
            return n;
        }
    };

    // ---- running softmax state and the O^T accumulator -----------------------
    f32x16 oacc[T::kDBlocks];
#pragma unroll
    for (int i = 0; i < T::kDBlocks; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;  // running max of scale*log2(e)*s for this lane's query
    float l_run = 0.f;        // this lane's partial sum (its half of each tile's keys)

    Staged st;
    if (n_act > 0) {
        bool pt;
        const int t0 = tile_of(0, pt);
        stage_load<D, SEG>(st, kp, vp, segkv_b, t0, S, tok_stride, tid);
        stage_store<D, SEG>(st, bufs, tid);
    }
    __syncthreads();

    for (int n = 0; n < n_act; ++n) {
        bool partial;
        const int t = tile_of(n, partial);
        char* buf = bufs + (n & 1) * T::kBufBytes;
        const bool has_next = (n + 1) < n_act;
        if (has_next) {
            bool pn;
            const int tn = tile_of(n + 1, pn);
            stage_load<D, SEG>(st, kp, vp, segkv_b, tn, S, tok_stride, tid);
        }

        if (wave_live) {
            // ---- S^T = K Q^T for two 32-key blocks ----------------------------
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x16{};
                const int row = kb * 32 + swap23(lr);
                const char* krow = buf + row * (D * 2);
                const int sw = lr & (T::kChunks - 1);  // == k_swz<D>(row)
#pragma unroll
                for (int ks = 0; ks < T::kSteps; ++ks) {
                    const int ch = 2 * ks + g;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ((ch ^ sw) << 4));
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[kb], 0, 0, 0);
                }
            }

            // ---- element masks on partial tiles -------------------------------
            if (partial) {
                const int* segt = reinterpret_cast<const int*>(buf + T::kSegOff);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int jl = kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
                        bool ok = (t * kBk + jl) < S;
                        if (SEG) ok = ok && (myseg != 0) && (segt[jl] == myseg);
                        if (!ok) sacc[kb][r] = -INFINITY;
                    }
                }
            }

            // ---- online softmax (log2 domain) ---------------------------------
            float mx = sacc[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mt = mx * c_log2;  // -inf if the whole tile is masked for this row
            const bool grow = mt > m_run;
            if (__ballot(grow) != 0ull) {
                const float m_new = grow ? mt : m_run;
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < T::kDBlocks; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
                m_run = m_new;
            }
            const float msub = (m_run == -INFINITY) ? 0.f : m_run;

            bf16x8 pb[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c_log2, -msub));
                    l_run += p;
                    pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
                }
            }

            // ---- O^T += V^T P^T -----------------------------------------------
            const char* vt = buf + T::kKBytes;
#pragma unroll
            for (int db = 0; db < T::kDBlocks; ++db) {
                const int drow = db * 32 + lr;
                const char* vrow = vt + drow * (kBk * 2);
                const int sw = v_swz(drow);
#pragma unroll
                for (int kst = 0; kst < 4; ++kst) {
                    const int jc = 2 * kst + g;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + ((jc ^ sw) << 4));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kst], oacc[db], 0, 0, 0);
                }
            }
        }

        if (has_next) stage_store<D, SEG>(st, bufs + ((n + 1) & 1) * T::kBufBytes, tid);
        __syncthreads();
    }

    // ---- epilogue: normalise, write out (bf16) and lse (fp32) ----------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qi < S) {
        __bf16* orow = out + ((int64_t)b * S + qi) * tok_stride + (int64_t)h * D;
        float lse_v;
        if (l_tot > 0.f) {
            const float inv = 1.0f / l_tot;
#pragma unroll
            for (int db = 0; db < T::kDBlocks; ++db) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = db * 32 + 8 * r4 + 4 * g;
                    __bf16 o4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][4 * r4 + e] * inv);
                    *reinterpret_cast<uint2*>(orow + d) = *reinterpret_cast<const uint2*>(o4);
                }
            }
            lse_v = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
        } else {
#pragma unroll
            for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *reinterpret_cast<uint2*>(orow + db * 32 + 8 * r4 + 4 * g) = uint2{0u, 0u};
            lse_v = -INFINITY;
        }
        if (g == 0) lse[((int64_t)b * H + h) * S + qi] = lse_v;
    }
}

template <int D, bool SEG>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
    using T = Tile<D>;
    const int n_qblk = (a.S + kBq - 1) / kBq;
    const int n_kvt = (a.S + kBk - 1) / kBk;
    const int64_t n_wg64 = (int64_t)a.B * a.H * n_qblk;
    const int n_wg = (int)n_wg64;
    size_t lds = 2 * (size_t)T::kBufBytes;
    if (SEG) lds += 2 * (size_t)n_kvt;
    lds = (lds + 15) & ~(size_t)15;
    lds += 32 * sizeof(int);  // meta
    const float c_log2 = a.scale * kLog2e;
    hipLaunchKernelGGL((attn_fwd_kernel<D, SEG>), dim3(n_wg), dim3(kThreads), lds, stream,
                       reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const __bf16*>(a.k),
                       reinterpret_cast<const __bf16*>(a.v), a.seg_q, a.seg_kv,
                       reinterpret_cast<__bf16*>(a.out), a.lse, a.S, a.H, c_log2, n_qblk, n_kvt,
                       n_wg);
    return hipGetLastError();
}

}  // namespace

int64_t max_masked_seq() { return (int64_t)kMaxKvTiles * kBk; }
int64_t queries_per_workgroup() { return kBq; }

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    const bool seg = a.seg_q != nullptr;
    if (a.D == 128) return seg ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return seg ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace vdx
