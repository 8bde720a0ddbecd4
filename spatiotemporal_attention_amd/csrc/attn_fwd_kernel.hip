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
//   * one workgroup = 4 wave64s (one per SIMD, 512 registers each) = 256
//     queries of one (batch, head); a wave owns 64 queries as two 32-query
//     halves A and B whose Q slices stay in registers for the whole sweep;
//   * scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: every lane then owns one query column, so the
//     row max/sum need one v_permlane32_swap with lane^32 only, and the fp32
//     score registers become the bf16 B operand of O^T += V^T P^T without any
//     data movement (the key order inside a 32-key block is permuted so the
//     accumulator rows line up with the operand's contraction index);
//   * in-wave software pipeline: half B runs half a key tile behind half A.
//     Each phase issues one half's MFMAs (P V of the previous tile and K Q^T
//     of the current one) while the VALU runs the other half's online
//     softmax, so matrix cores and vector ALUs work concurrently inside one
//     wave;
//   * K and V arrive in LDS by direct global->LDS DMA (global_load_lds, 16 B
//     per lane) into three-slot rings, two tiles ahead, with one workgroup
//     barrier per tile; K rows are XOR-swizzled by 16-byte chunk, V stays
//     row-major (32-byte chunks XOR-swizzled) and is read transposed with
//     ds_read_b64_tr_b16, so no VALU work is spent on staging;
//   * online softmax in fp32 with exp2 and scale*log2(e) folded into one FMA;
//     O is rescaled only when some row's running maximum grew;
//   * with segment IDs, a prologue classifies every 64-key tile against the
//     workgroup's query segments as skip / full / partial and compacts the
//     active ones into an LDS list, so fully masked tiles cost nothing and
//     only partial tiles pay for element masks;
//   * workgroups are renumbered so that each XCD (own L2) runs consecutive
//     query blocks of the same head, which then share K/V tiles in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_fwd_launch.h"

namespace vdx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBq = 64 * kWaves;  // queries per workgroup
constexpr int kBk = 64;           // keys per tile
constexpr int kSlots = 3;         // ring depth of the K, V and segment-ID stages
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kMaxKvTiles = 30720;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Tile {
    static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBk * kRowBytes;           // one K or V tile
    static constexpr int kKRegion = 0;
    static constexpr int kVRegion = kSlots * kTileBytes;
    static constexpr int kSegRegion = kVRegion + kSlots * kTileBytes;
    static constexpr int kRingBytes = kSegRegion + kSlots * kBk * 4;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;        // rows per wave DMA
    static constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;
    static constexpr int kSteps = D / 16;                        // MFMA k-steps over D
    static constexpr int kDBlocks = D / 32;                      // 32-row blocks of O^T
    static_assert(kLoadsPerWave >= 1, "tile too small for the workgroup");
};

// Swap bits 2 and 3: maps an MFMA accumulator row inside a 32-key block to the
// physical key it holds (and back; the map is an involution).
__device__ __forceinline__ int swap23(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}
// K tile: 16-byte chunk c of row r sits at position c ^ k_swz(r).
template <int D>
__device__ __forceinline__ int k_swz(int r) { return swap23(r & 31) & (Tile<D>::kChunks - 1); }
// V tile: 32-byte chunk h of row r sits at position h ^ v_swz(r).
template <int D>
__device__ __forceinline__ int v_swz(int r) { return (2 * (r & 3)) & (Tile<D>::kChunks / 2 - 1); }

__device__ __forceinline__ float pair_max(float x) {
    // v_permlane32_swap(x, x) yields x[l % 32] and x[l % 32 + 32] in every lane.
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else static_assert(N < 0, "unsupported count");
}

// Direct global->LDS copies: lane l's bytes land at LDS address M0 + size*l.
// Issued as inline asm so that the compiler does not treat every later LDS read
// as a possible alias of the in-flight copy (it would insert vmcnt(0) waits and
// serialise the prefetch); completion is tracked by hand with wait_vm<N>() and
// the workgroup barrier that follows it.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ void dma16(const void* g, char* lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, char* lds) {
    asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_addr(lds)) : "memory");
}

__device__ __forceinline__ bf16x8 tr_read8(const char* p0, const char* p1) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
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

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int D, bool SEG>
struct Attn {
    using T = Tile<D>;
    char* smem;
    const __bf16* kp;   // K of (b, h), token 0
    const __bf16* vp;
    const int32_t* segkv;
    const uint16_t* list;
    int64_t tok_stride;
    int S, n_kvt, wave, lane, lr, g;
    float c_log2;
    int myseg[2];
    int koff[T::kSteps];               // K operand read offsets (slot base, key block 0)
    int voff[T::kDBlocks];             // V transposed-read offsets (slot base, key 0)
    int dmak[T::kLoadsPerWave];        // per-lane element offsets of the K DMA in a tile
    int dmav[T::kLoadsPerWave];
    bf16x8 qreg[2][T::kSteps];
    f32x16 oacc[2][T::kDBlocks];
    f32x16 sacc[2][2];
    bf16x8 pb[2][4];
    float m_run[2], l_run[2], alpha[2];

    __device__ __forceinline__ int tile_of(int n, bool& partial) const {
        if (SEG) {
            const int e = __builtin_amdgcn_readfirstlane((int)list[n]);
            partial = (e & 0x8000) != 0;
            return e & 0x7fff;
        } else {
            partial = (n == n_kvt - 1) && (S % kBk != 0);
            return n;
        }
    }

    // ---- DMA of this wave's share of a K / V tile (rows past S read row S-1,
    // which the masks then exclude) and of a tile's segment IDs ----------------
    __device__ __forceinline__ void dma_tile(const __bf16* base, const int* off, int t, char* dst) {
        const __bf16* src = base + (int64_t)t * kBk * tok_stride;
        if (t * kBk + kBk <= S) {
#pragma unroll
            for (int j = 0; j < T::kLoadsPerWave; ++j) dma16(src + off[j], dst + j * 1024);
        } else {
#pragma unroll
            for (int j = 0; j < T::kLoadsPerWave; ++j) {
                const int i = wave * T::kLoadsPerWave + j;
                const int r = T::kRowsPerLoad * i + lane / T::kChunks;
                const int over = max(0, t * kBk + r - (S - 1));
                dma16(src + off[j] - (int64_t)over * tok_stride, dst + j * 1024);
            }
        }
    }
    __device__ __forceinline__ void dma_k(int n, int slot) {
        bool p;
        const int t = tile_of(n, p);
        dma_tile(kp, dmak, t, smem + T::kKRegion + slot * T::kTileBytes + wave * T::kLoadsPerWave * 1024);
    }
    __device__ __forceinline__ void dma_v(int n, int slot) {
        bool p;
        const int t = tile_of(n, p);
        dma_tile(vp, dmav, t, smem + T::kVRegion + slot * T::kTileBytes + wave * T::kLoadsPerWave * 1024);
    }
    __device__ __forceinline__ void dma_seg(int n, int slot) {
        if (!SEG) return;
        bool p;
        const int t = tile_of(n, p);
        char* sdst = smem + T::kSegRegion + slot * kBk * 4 + wave * 64;
        const int key = min(t * kBk + wave * 16 + (lane & 15), S - 1);
        if (lane < 16) dma4(segkv + key, sdst);
    }

    // ---- MFMA operands ----------------------------------------------------------
    // MFMA i of a phase: first the P V ones (k-step kst, d-block db), then the
    // K Q^T ones (k-step ks, key block kb).
    template <bool PV>
    static constexpr int n_pv() { return PV ? 4 * T::kDBlocks : 0; }
    template <bool PV, int I>
    __device__ __forceinline__ bf16x8 operand(const char* vb, const char* kb) const {
        if constexpr (I < n_pv<PV>()) {
            constexpr int kst = I / T::kDBlocks, db = I % T::kDBlocks;
            const char* p = vb + voff[db] + kst * 16 * T::kRowBytes;
            return tr_read8(p, p + 4 * T::kRowBytes);
        } else {
            constexpr int j = I - n_pv<PV>();
            constexpr int ks = j / 2, kbk = j % 2;
            return *reinterpret_cast<const bf16x8*>(kb + koff[ks] + kbk * 32 * T::kRowBytes);
        }
    }
    template <bool PV, int HM, int I>
    __device__ __forceinline__ void mfma(const bf16x8& a) {
        if constexpr (I < n_pv<PV>()) {
            constexpr int kst = I / T::kDBlocks, db = I % T::kDBlocks;
            oacc[HM][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[HM][kst], oacc[HM][db], 0, 0, 0);
        } else {
            constexpr int j = I - n_pv<PV>();
            constexpr int ks = j / 2, kbk = j % 2;
            if constexpr (ks == 0)
                sacc[HM][kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[HM][0], f32x16{}, 0, 0, 0);
            else
                sacc[HM][kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[HM][ks], sacc[HM][kbk], 0, 0, 0);
        }
    }

    // ---- online softmax, cut into slices that ride in the MFMA shadow ----------
    // Values of half h: v(k) = sacc[h][k / 16][k % 16], k = 0..31.
    float sm_mx0, sm_mx1, sm_msub, sm_ls[4];
    __device__ __forceinline__ float sv(int h, int k) const { return sacc[h][k >> 4][k & 15]; }
    template <int H, int STEP, int NSTEPS>
    __device__ __forceinline__ void softmax_slice() {
        if constexpr (STEP == 0) {
            float m = fmaxf(fmaxf(sv(H, 0), sv(H, 1)), sv(H, 2));
#pragma unroll
            for (int k = 3; k < 15; k += 2) m = fmaxf(fmaxf(m, sv(H, k)), sv(H, k + 1));
            sm_mx0 = fmaxf(m, sv(H, 15));
        } else if constexpr (STEP == 1) {
            float m = fmaxf(fmaxf(sv(H, 16), sv(H, 17)), sv(H, 18));
#pragma unroll
            for (int k = 19; k < 31; k += 2) m = fmaxf(fmaxf(m, sv(H, k)), sv(H, k + 1));
            sm_mx1 = fmaxf(m, sv(H, 31));
        } else if constexpr (STEP == 2) {
            const float mx = pair_max(fmaxf(sm_mx0, sm_mx1));
            const float m_old = m_run[H];
            const float m_new = fmaxf(m_old, mx * c_log2);
            // alpha == 1 exactly when the maximum did not move (exp2(0) = 1).
            alpha[H] = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_old - m_new);
            m_run[H] = m_new;
            sm_msub = (m_new == -INFINITY) ? 0.f : m_new;
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_ls[i] = 0.f;
        }
        // 16 pairs of values spread over steps 3 .. NSTEPS-2.
        static_for<0, 16>([&](auto kc) {
            constexpr int k = kc;
            if constexpr (STEP == 3 + k * (NSTEPS - 4) / 16) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv(H, 2 * k), c_log2, -sm_msub));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv(H, 2 * k + 1), c_log2, -sm_msub));
                sm_ls[(2 * k) & 3] += p0;
                sm_ls[(2 * k + 1) & 3] += p1;
                // value k' sits in pb[h][k'/8][k'%8]
                pb[H][(2 * k) >> 3][(2 * k) & 7] = (__bf16)p0;
                pb[H][(2 * k + 1) >> 3][(2 * k + 1) & 7] = (__bf16)p1;
            }
        });
        if constexpr (STEP == NSTEPS - 1)
            l_run[H] = __builtin_fmaf(alpha[H], l_run[H], (sm_ls[0] + sm_ls[1]) + (sm_ls[2] + sm_ls[3]));
    }

    // One pipeline phase: the MFMAs of half HM (P V of the previous tile if PV,
    // K Q^T of the current tile if QK) issued one per step with their LDS
    // operands fetched PF steps ahead, and, if SM, the online softmax of the
    // other half cut into one slice per step.  A scheduling fence closes every
    // step so the interleaving survives compilation.
    template <int HM, bool PV, bool QK, bool SM>
    __device__ __forceinline__ void phase(const char* vb, const char* kb) {
        constexpr int NM = n_pv<PV>() + (QK ? 2 * T::kSteps : 0);
        constexpr int PF = 3, RING = PF + 1;
        bf16x8 ops[RING];
        static_for<0, PF>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i < NM) ops[i % RING] = operand<PV, i>(vb, kb);
        });
        static_for<0, NM>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i + PF < NM) ops[(i + PF) % RING] = operand<PV, i + PF>(vb, kb);
            mfma<PV, HM, i>(ops[i % RING]);
            if constexpr (SM) softmax_slice<1 - HM, i, NM>();
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (SM) {
            // Pin the softmax results inside this phase: without a use here the
            // optimiser sinks the whole softmax next to its consumers (the next
            // phase's P V), which would serialise it behind those MFMAs.
            constexpr int HS = 1 - HM;
            asm volatile("" ::"v"(pb[HS][0]), "v"(pb[HS][1]), "v"(pb[HS][2]), "v"(pb[HS][3]),
                         "v"(l_run[HS]), "v"(m_run[HS]), "v"(alpha[HS]));
        }
    }

    // Element masks of half h for active tile n (partial tiles only), seg IDs
    // of the tile at sbase.  Key of register r of block b: b*32 + 16*(r>>3) + 8g + (r&7).
    __device__ __forceinline__ void mask(int h, int n, const int* sbase) {
        bool partial;
        const int t = tile_of(n, partial);
        const int lim = S - t * kBk - 8 * g;
        const int* segt = sbase + 8 * g;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int jc = b * 32 + 16 * (r >> 3) + (r & 7);
                bool ok = jc < lim;
                if (SEG) ok = ok && (segt[jc] == myseg[h]) && (myseg[h] != 0);
                if (!ok) sacc[h][b][r] = -INFINITY;
            }
        }
    }

    // O *= alpha for half h when some row's maximum moved.  The accumulators
    // live in AGPRs; the multiply is spelled out on them so that the compiler
    // keeps them there for the MFMAs instead of shuttling them through VGPRs.
    __device__ __forceinline__ void rescale(int h) {
        if (__ballot(alpha[h] != 1.0f) != 0ull) {
#pragma unroll
            for (int db = 0; db < T::kDBlocks; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float t;
                    asm("v_accvgpr_read_b32 %1, %0\n\t"
                        "v_mul_f32 %1, %1, %2\n\t"
                        "v_accvgpr_write_b32 %0, %1"
                        : "+a"(oacc[h][db][r]), "=&v"(t)
                        : "v"(alpha[h]));
                }
            }
        }
    }

    __device__ __forceinline__ const char* kslot(int r) const { return smem + T::kKRegion + r * T::kTileBytes; }
    __device__ __forceinline__ const char* vslot(int r) const { return smem + T::kVRegion + r * T::kTileBytes; }
    __device__ __forceinline__ const int* sslot(int r) const {
        return reinterpret_cast<const int*>(smem + T::kSegRegion) + r * kBk;
    }
    __device__ __forceinline__ bool partial(int n) const {
        bool p;
        tile_of(n, p);
        return p;
    }

    // Steady-state iteration n (1 <= n < n_act), R = n % 3: S(n) of both halves
    // and P V of tile n-1.  Loads issued here: segment IDs of tile n+1, K of
    // tile n+2 and V of tile n+1, into ring slots whose previous tiles were last
    // read in iteration n-1.
    template <int R>
    __device__ __forceinline__ void iteration(int n, int n_act) {
        constexpr int R1 = (R + 1) % kSlots, R2 = (R + 2) % kSlots;
        const bool ld_v = n + 1 < n_act;
        const bool ld_k = n + 2 < n_act;
        if (ld_v) dma_seg(n + 1, R1);
        if (ld_k) dma_k(n + 2, R2);
        if (ld_v) dma_v(n + 1, R1);
        const bool part = partial(n);
        phase<0, true, true, true>(vslot(R2), kslot(R));   // A: P V(n-1), S(n);  B: softmax(n-1)
        rescale(1);
        if (part) mask(0, n, sslot(R));
        phase<1, true, true, true>(vslot(R2), kslot(R));   // B: P V(n-1), S(n);  A: softmax(n)
        rescale(0);
        if (part) mask(1, n, sslot(R));
        constexpr int kv = T::kLoadsPerWave;
        if (ld_k)
            wait_vm<2 * kv>();
        else if (ld_v)
            wait_vm<kv>();
        else
            wait_vm<0>();
        barrier();
    }
};

template <int D, bool SEG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, const int32_t* __restrict__ seg_q,
                     const int32_t* __restrict__ seg_kv, __bf16* __restrict__ out,
                     float* __restrict__ lse, int S, int H, float c_log2, int n_qblk, int n_kvt,
                     int n_wg) {
    using T = Tile<D>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

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
    const int qbase = qblk * kBq + wave * 64;

    Attn<D, SEG> A;
    A.smem = smem;
    A.tok_stride = (int64_t)H * D;
    A.kp = k + (int64_t)b * S * A.tok_stride + (int64_t)h * D;
    A.vp = v + (int64_t)b * S * A.tok_stride + (int64_t)h * D;
    A.segkv = SEG ? seg_kv + (int64_t)b * S : nullptr;
    A.S = S;
    A.n_kvt = n_kvt;
    A.wave = wave;
    A.lane = lane;
    A.lr = lr;
    A.g = g;
    A.c_log2 = c_log2;

    // ---- Q slices -> registers as the B operand of S^T = K Q^T ----------------
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int qi = qbase + 32 * hh + lr;
        const __bf16* qrow = q + ((int64_t)b * S + qi) * A.tok_stride + (int64_t)h * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks)
            A.qreg[hh][ks] = (qi < S) ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16) : bf16x8{};
        A.myseg[hh] = SEG ? ((qi < S) ? seg_q[(int64_t)b * S + qi] : 0) : 1;
    }
    // ---- per-lane LDS offsets ---------------------------------------------------
    {
        const int ksw = lr & (T::kChunks - 1);  // == k_swz(row) for row = swap23(lr)
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks)
            A.koff[ks] = swap23(lr) * T::kRowBytes + (((2 * ks + g) ^ ksw) << 4);
        // Transposed V read: group q = lane/16 takes d = db*32 + 16(q&1) + 4(j&3)
        // and keys 8(q>>1) + (j>>2) (+4 for the second half of the operand).
        const int qg = lane >> 4, j = lane & 15;
        const int key = 8 * (qg >> 1) + (j >> 2);
        const int vsw = v_swz<D>(key);
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) {
            const int h32 = 2 * db + (qg & 1);  // 32-byte chunk of d
            A.voff[db] = key * T::kRowBytes + 32 * (h32 ^ vsw) + 16 * ((j & 3) >> 1) + 8 * (j & 1);
        }
        // DMA: instruction i of the tile covers rows kRowsPerLoad*i .. ; lane lands
        // at LDS position pos of its row and fetches the chunk stored there.
#pragma unroll
        for (int jj = 0; jj < T::kLoadsPerWave; ++jj) {
            const int i = wave * T::kLoadsPerWave + jj;
            const int r = T::kRowsPerLoad * i + lane / T::kChunks;
            const int pos = lane % T::kChunks;
            const int ck = pos ^ k_swz<D>(r);
            const int cv = 2 * ((pos >> 1) ^ v_swz<D>(r)) + (pos & 1);
            A.dmak[jj] = r * (int)A.tok_stride + ck * 8;
            A.dmav[jj] = r * (int)A.tok_stride + cv * 8;
        }
    }

    uint16_t* list = reinterpret_cast<uint16_t*>(smem + T::kRingBytes);
    int* meta = reinterpret_cast<int*>(smem + ((T::kRingBytes + 2 * (SEG ? n_kvt : 0) + 15) & ~15));
    // meta: [0..3] per-wave q min, [4..7] q max, [8..11] q flags, [12] n_active
    A.list = list;

    int n_act = n_kvt;
    if (SEG) {
        // ---- query-block segment summary --------------------------------------
        {
            int mn = INT32_MAX, mx = INT32_MIN, fl = 0;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int s = A.myseg[hh];
                mn = min(mn, (s != 0) ? s : INT32_MAX);
                mx = max(mx, (s != 0) ? s : INT32_MIN);
                fl |= (s == 0) ? 1 : 0;  // pad or out-of-range row present
            }
            mn = wave_min(mn);
            mx = wave_max(mx);
            fl = wave_max(fl);
            if (lane == 0) {
                meta[wave] = mn;
                meta[4 + wave] = mx;
                meta[8 + wave] = fl;
            }
        }
        __syncthreads();
        int qmn = INT32_MAX, qmx = INT32_MIN, qfl = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            qmn = min(qmn, meta[i]);
            qmx = max(qmx, meta[4 + i]);
            qfl |= meta[8 + i];
        }
        // ---- classify every key tile: 0 skip, 1 full, 2 partial ---------------
        uint8_t* cls = reinterpret_cast<uint8_t*>(smem);  // aliases the rings
        for (int t = wave; t < n_kvt; t += kWaves) {
            const int key = t * kBk + lane;
            const int id = (key < S) ? A.segkv[key] : 0;
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
            if (lane == 0) meta[12] = base;
        }
        __syncthreads();
        n_act = meta[12];
    }

    // ---- running softmax state and the O^T accumulators -----------------------
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int i = 0; i < T::kDBlocks; ++i) A.oacc[hh][i] = f32x16{};
#pragma unroll
        for (int i = 0; i < 4; ++i) A.pb[hh][i] = bf16x8{};
        A.m_run[hh] = -INFINITY;  // running max of scale*log2(e)*s for this lane's query
        A.l_run[hh] = 0.f;        // this lane's partial sum (its half of each tile's keys)
        A.alpha[hh] = 1.f;
    }

    // ---- prologue: segment IDs and K of tile 0, K of tile 1, V of tile 0 ---------
    if (n_act > 0) {
        A.dma_seg(0, 0);
        A.dma_k(0, 0);
        A.dma_v(0, 0);
    }
    if (n_act > 1) A.dma_k(1, 1);
    wait_vm<0>();
    barrier();

    // ---- main loop: iteration n computes S(n) and P V of tile n-1 ---------------
    // Ring slots: K, V and segment IDs of tile n all live in slot n % 3.
    if (n_act > 0) {
        // iteration 0: K Q^T of both halves, softmax of half A
        constexpr int kv = T::kLoadsPerWave;
        if (n_act > 1) A.dma_seg(1, 1);
        if (n_act > 2) A.dma_k(2, 2);
        if (n_act > 1) A.dma_v(1, 1);
        const bool part = A.partial(0);
        A.template phase<0, false, true, false>(nullptr, A.kslot(0));
        if (part) A.mask(0, 0, A.sslot(0));
        A.template phase<1, false, true, true>(nullptr, A.kslot(0));
        A.rescale(0);
        if (part) A.mask(1, 0, A.sslot(0));
        if (n_act > 2)
            wait_vm<2 * kv>();
        else if (n_act > 1)
            wait_vm<kv>();
        else
            wait_vm<0>();
        barrier();
    }
    int n = 1;
    for (; n + 2 < n_act; n += 3) {
        A.template iteration<1>(n, n_act);
        A.template iteration<2>(n + 1, n_act);
        A.template iteration<0>(n + 2, n_act);
    }
    if (n < n_act) A.template iteration<1>(n, n_act);
    if (n + 1 < n_act) A.template iteration<2>(n + 1, n_act);
    if (n_act > 0) {
        // final iteration: P V of the last tile for both halves
        const char* vb = A.vslot((n_act - 1) % kSlots);
        A.template phase<0, true, false, true>(vb, nullptr);
        A.rescale(1);
        A.template phase<1, true, false, false>(vb, nullptr);
    }

    // ---- epilogue: normalise, write out (bf16) and lse (fp32) ----------------
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int qi = qbase + 32 * hh + lr;
        const float l_tot = pair_sum(A.l_run[hh]);
        if (qi < S) {
            __bf16* orow = out + ((int64_t)b * S + qi) * A.tok_stride + (int64_t)h * D;
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
                        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(A.oacc[hh][db][4 * r4 + e] * inv);
                        *reinterpret_cast<uint2*>(orow + d) = *reinterpret_cast<const uint2*>(o4);
                    }
                }
                lse_v = (A.m_run[hh] + __builtin_amdgcn_logf(l_tot)) * kLn2;
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
}

template <int D, bool SEG>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
    using T = Tile<D>;
    const int n_qblk = (a.S + kBq - 1) / kBq;
    const int n_kvt = (a.S + kBk - 1) / kBk;
    const int64_t n_wg64 = (int64_t)a.B * a.H * n_qblk;
    const int n_wg = (int)n_wg64;
    size_t lds = (size_t)T::kRingBytes;
    if (SEG) lds += 2 * (size_t)n_kvt;
    lds = (lds + 15) & ~(size_t)15;
    lds += 16 * sizeof(int);  // meta
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
