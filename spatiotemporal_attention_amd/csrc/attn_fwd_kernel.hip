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
//   * one workgroup = 8 wave64s (two per SIMD) = 256 queries of one
//     (batch, head); each wave owns 32 queries whose Q slice stays in
//     registers for the whole sweep;
//   * scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: every lane then owns one query column, so the
//     row max/sum need one v_permlane32_swap with lane^32 only, and the fp32
//     score registers become the bf16 B operand of O^T += V^T P^T without any
//     data movement (the key order inside a 32-key block is permuted so the
//     accumulator rows line up with the operand's contraction index);
//   * ping-pong schedule: the waves form two groups (one wave of each per
//     SIMD) that run one phase apart -- while one group issues its MFMAs
//     (P V of the previous key tile and K Q^T of the current one, operands
//     fetched from LDS a few MFMAs ahead) the other runs the online softmax,
//     so each SIMD's matrix core and vector ALU are fed by different waves;
//     a workgroup barrier separates phases;
//   * K and V arrive in LDS by direct global->LDS DMA (global_load_lds, 16 B
//     per lane) into three-slot rings, issued two phases or more before use;
//     K rows are XOR-swizzled by 16-byte chunk, V stays row-major (32-byte
//     chunks XOR-swizzled) and is read transposed with ds_read_b64_tr_b16, so
//     no VALU work is spent on staging and no LDS bank conflicts occur;
//   * online softmax in fp32 with exp2 and scale*log2(e) folded into one FMA;
//     the reference maximum moves lazily (only when a score exceeds it by a
//     fixed margin), so the O^T accumulators are almost never rescaled;
//   * register budget (two waves per SIMD, 256 VGPRs each): the O^T and S^T
//     accumulators, the Q slice, P and a short operand ring; operand addresses
//     are one swizzled base per phase (XOR with a constant per MFMA) and the
//     tile copies take a wave-uniform SGPR base plus a 32-bit lane offset, so
//     the steady-state loop runs without spills;
//   * with segment IDs, a prologue classifies every 64-key tile against the
//     workgroup's query segments as skip / full / partial and compacts the
//     active ones into an LDS list, so fully masked tiles cost nothing and
//     only partial tiles pay for element masks;
//   * workgroups are renumbered so that each XCD (own L2) runs consecutive
//     query blocks of the same head, which then share K/V tiles in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <tuple>

#include "attn_common.h"
#include "attn_fwd_launch.h"
#include "rope3d.h"

namespace vdx {
namespace {

constexpr int kMaxKvTiles = 30720;  // capacity of the on-chip active-tile list

template <int D, bool SEG, bool PART>
struct Attn {
    using T = Tile<D>;
    static constexpr bool kSeg = SEG;
    char* smem;
    const __bf16* kp;   // K of (b, h), token 0
    const __bf16* vp;
    const int32_t* segkv;
    const uint16_t* list;
    int64_t tok_stride;
    int S, n_kvt, wave, lane, lr, g;
    // Unmasked: a part of a split item sees tiles t0 .. t0 + n_kvt - 1 of
    // the head (n_kvt then counts that range), and holds the ragged last
    // tile only if its range ends the sequence (last_view).
    int t0;
    bool last_view;
    float c_log2;
    int myseg;
    // Active tile a - 1 of the next plan() call (group 0 plans tiles 0, 1,
    // 2, ... in order): its index and partial flag, looked up by the
    // previous call, so the segment-ID copy decision needs no second lookup.
    int prev_t;
    bool prev_part;
    // With segment IDs the partial flags of the planned tiles are kept as
    // bits (the latest plan() call's in bit 0), so that the VALU phase's
    // partial test does not wait on an LDS read of the tile list.
    uint32_t phist;
    // K operand of k-step ks sits at kx ^ (ks << 5) and the transposed V read
    // of d-block db at vx ^ (db << 6) (offsets within a ring slot): the XOR
    // swizzles only touch bits that these bases hold no other data in.
    int kx, vx;
    // Per-lane byte offsets of this wave's share of a tile copy (group 0 waves
    // copy K tiles and segment IDs, group 1 waves V tiles); w4 = wave & 3.
    uint32_t dmo[T::kLoadsPerWave];
    int w4;
    bf16x8 qreg[T::kSteps];
    f32x16 oacc[T::kDBlocks];
    f32x16 sacc[2];
    bf16x8 pb[4];
    bf16x8 ops[kOperandPrefetch + 2];  // MFMA operand ring
    uint32_t vb_next, kb_next;         // operand bases of the prefetched phase
    float m_run, l_run;

    __device__ __forceinline__ int tile_of(int n, bool& partial) const {
        if (SEG) {
            const int e = __builtin_amdgcn_readfirstlane((int)list[n]);
            partial = (e & 0x8000) != 0;
            return e & 0x7fff;
        } else {
            if constexpr (PART) {
                partial = (n == n_kvt - 1) && (S % kBk != 0) && last_view;
                return n + t0;
            } else {
                partial = (n == n_kvt - 1) && (S % kBk != 0);
                return n;
            }
        }
    }
    // Partial test of tile n in the VALU phase of iteration n of group G: the
    // last plan() call of G was for tile n + 2 - G.
    template <int G>
    __device__ __forceinline__ bool partial_planned(int n) const {
        if constexpr (SEG) {
            return ((phist >> (2 - G)) & 1u) != 0;
        } else {
            bool p;
            tile_of(n, p);
            return p;
        }
    }
    __device__ __forceinline__ bool partial(int n) const {
        bool p;
        tile_of(n, p);
        return p;
    }
    // Byte offset of ring slot n % kSlots.  Hidden from the optimiser, which
    // would otherwise keep one strength-reduced induction variable per operand
    // address (dozens of VGPRs) instead of adding the slot base per phase.
    __device__ __forceinline__ static int slot_base(int n) {
        int o = (n % kSlots) * T::kTileBytes;
        asm volatile("" : "+s"(o));
        return o;
    }
    __device__ __forceinline__ const int* sslot(int n) const {
        return reinterpret_cast<const int*>(smem + T::kSegRegion) + (n % kSlots) * kBk;
    }

    // ---- tile copies ---------------------------------------------------------------
    // In its MFMA phase of local iteration n, a wave of group G copies its share
    // of K (G = 0) or V (G = 1) of active tile a = n + 2 - G into ring slot
    // a % 3, and wave 0 of group 0 copies the segment IDs of active tile n + 1
    // if that tile is partial.
    // In global-phase terms (the MFMA phase of iteration n is phase 2n + G):
    // K of tile m+2 and segment IDs of tile m+1 in phase 2m, V of tile m+1 in
    // phase 2m+1.  Slot a % 3 then held tile a-3, whose last reader finished
    // in phase 2m-1 (K, V) or 2m-2 (segment IDs).  Each wave waits for its
    // copies at the end of its next MFMA phase, before the barrier that
    // precedes their first reader.
    struct Copy {
        const __bf16* src;  // tile base in global memory (wave-uniform)
        char* dst;          // this wave's share of the ring slot
        int t;              // key tile index
        int seg_t, seg_a;   // segment-ID copy (tile, active index), seg_a < 0: none
        bool spread;        // full tile: the loads go out between MFMAs
        bool tail;          // last, partial tile: issued at the phase start
        int cnt;            // loads this wave issues for the copy
    };
    // Tile-list entry of active tile a for plan() (SEG; read at the start of
    // a VALU phase, so that its latency passes under the softmax), or 0.
    __device__ __forceinline__ int list_entry(int a, int n_act) const {
        if constexpr (SEG) return a < n_act ? (int)list[a] : 0;
        return 0;
    }
    // Plans the copies of the MFMA phase of iteration a - 2 + G (run in the
    // preceding VALU phase: scalar work only, nothing is issued); ent is
    // list_entry(a, n_act).
    template <int G>
    __device__ __forceinline__ void plan(Copy& c, int a, int n_act, int ent) {
        bool part;
        int pt = 0;
        bool pp = false;
        if constexpr (SEG && G == 0) {
            pt = prev_t;
            pp = prev_part;
        }
        c.cnt = 0;
        c.spread = c.tail = false;
        c.seg_a = -1;
        if constexpr (SEG) phist <<= 1;
        if (a < n_act) {
            if constexpr (SEG) {
                const int e = __builtin_amdgcn_readfirstlane(ent);
                part = (e & 0x8000) != 0;
                c.t = e & 0x7fff;
                phist |= part ? 1u : 0u;
            } else {
                c.t = tile_of(a, part);
            }
            c.src = (G ? vp : kp) + (int64_t)c.t * kBk * tok_stride;
            c.dst = smem + (G ? T::kVRegion : T::kKRegion) + slot_base(a) +
                    w4 * T::kLoadsPerWave * 1024;
            c.spread = c.t * kBk + kBk <= S;
            c.tail = !c.spread;
            c.cnt = T::kLoadsPerWave;
            if constexpr (SEG && G == 0) {
                prev_t = c.t;
                prev_part = part;
            }
        }
        // Only a partial tile's masks read its segment IDs.
        if (SEG && G == 0 && w4 == 0 && a >= 1 && a - 1 < n_act && pp) {
            c.seg_a = a - 1;
            c.seg_t = pt;
            c.cnt += 1;
        }
    }
    // Issued at the start of the MFMA phase: the segment IDs (64 keys, one per
    // lane) and, for the tail tile, the whole K/V share with rows past S
    // reading row S-1 (the masks exclude them).
    __device__ __forceinline__ void copy_start(const Copy& c) {
        if (SEG && c.seg_a >= 0) {
            char* sdst = smem + T::kSegRegion + (c.seg_a % kSlots) * kBk * 4;
            const int key = min(c.seg_t * kBk + lane, S - 1);
            dma4(segkv, 4u * (uint32_t)key, sdst);
        }
        if (c.tail) {
#pragma unroll
            for (int j = 0; j < T::kLoadsPerWave; ++j) {
                const int i = w4 * T::kLoadsPerWave + j;
                const int r = T::kRowsPerLoad * i + lane / T::kChunks;
                const int over = max(0, c.t * kBk + r - (S - 1));
                dma16(c.src, dmo[j] - (uint32_t)over * (uint32_t)(2 * tok_stride), c.dst + j * 1024);
            }
        }
    }
    // Load j of a spread copy goes out after MFMA step j*NM/L + 1 of a phase
    // with NM MFMAs.
    template <int I, int NM>
    __device__ __forceinline__ void copy_step(const Copy& c) {
        constexpr int L = T::kLoadsPerWave;
        static_assert(NM >= L + 1, "too few MFMA steps to spread the copies over");
        static_for<0, L>([&](auto jc) {
            constexpr int j = jc;
            if constexpr (I == j * NM / L + 1) {
                if (c.spread) dma16(c.src, dmo[j], c.dst + j * 1024);
            }
        });
    }

    // ---- MFMA phase ----------------------------------------------------------------
    // MFMA i: first the K Q^T ones of the current tile (k-step ks, key block
    // kbk), then the P V ones of the previous tile (k-step kst, d-block db).
    // Starting with K Q^T lets a wave fetch the first K operands before the
    // barrier that opens the phase: the K tile became visible one phase
    // earlier, the V tile only at that barrier.
    template <bool QK>
    static constexpr int n_qk() { return QK ? 2 * T::kSteps : 0; }
    template <bool PV, bool QK>
    static constexpr int n_mfma() { return n_qk<QK>() + (PV ? 4 * T::kDBlocks : 0); }
    static constexpr int kRing = kOperandPrefetch + 2;
    // vb / kb: LDS byte addresses of this lane's V and K operand bases in the
    // ring slots (slot and region offsets are multiples of 1024, so the swizzle
    // XOR can be applied to the full address).
    __device__ __forceinline__ uint32_t vbase(int vtile) const {
        return lds_addr(smem) + T::kVRegion + slot_base(vtile) + vx;
    }
    __device__ __forceinline__ uint32_t kbase(int ktile) const {
        return lds_addr(smem) + T::kKRegion + slot_base(ktile) + kx;
    }
    template <bool QK, int I>
    __device__ __forceinline__ bf16x8 operand(uint32_t vb, uint32_t kb) const {
        if constexpr (I < n_qk<QK>()) {
            constexpr int ks = I / 2, kbk = I % 2;
            return *reinterpret_cast<const bf16x8*>(lds_ptr((kb ^ (ks << 5)) + kbk * 32 * T::kRowBytes));
        } else {
            constexpr int j = I - n_qk<QK>();
            constexpr int kst = j / T::kDBlocks, db = j % T::kDBlocks;
            const char* p = lds_ptr((vb ^ (db << 6)) + kst * 16 * T::kRowBytes);
            return tr_read8(p, p + 4 * T::kRowBytes);
        }
    }
    template <bool QK, int I>
    __device__ __forceinline__ void mfma(const bf16x8& a) {
        if constexpr (I < n_qk<QK>()) {
            constexpr int ks = I / 2, kbk = I % 2;
            if constexpr (ks == 0)
                sacc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[0], f32x16{}, 0, 0, 0);
            else
                sacc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[kbk], 0, 0, 0);
        } else {
            constexpr int j = I - n_qk<QK>();
            constexpr int kst = j / T::kDBlocks, db = j % T::kDBlocks;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kst], oacc[db], 0, 0, 0);
        }
    }
    // The first kOperandPrefetch operands of an MFMA phase into the ring.
    // The operand bases are kept for the phase, so that its first MFMA does not
    // wait behind their computation.
    template <bool PV, bool QK>
    __device__ __forceinline__ void prefetch(int vtile, int ktile) {
        vb_next = vbase(vtile);
        kb_next = kbase(ktile);
        static_for<0, kOperandPrefetch>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i < n_mfma<PV, QK>()) ops[i % kRing] = operand<QK, i>(vb_next, kb_next);
        });
    }
    // K Q^T of the current tile (if QK) and P V of the previous tile (if PV):
    // one MFMA per step, LDS operands fetched kOperandPrefetch steps ahead into
    // a ring two entries longer, so a register is refilled only after the MFMA
    // that read it has long issued; the planned tile copy goes out in between.
    // With PRE the first operands were fetched before the phase began.  A
    // scheduling fence closes every step.
    template <bool PV, bool QK, bool PRE>
    __device__ __forceinline__ void mfma_phase(int vtile, int ktile, const Copy& cp) {
        constexpr int NM = n_mfma<PV, QK>();
        constexpr int PF = kOperandPrefetch;
        __builtin_amdgcn_s_setprio(1);
        if constexpr (!PRE) prefetch<PV, QK>(vtile, ktile);
        const uint32_t vb = vb_next, kb = kb_next;
        copy_start(cp);
        static_for<0, NM>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i + PF < NM) ops[(i + PF) % kRing] = operand<QK, i + PF>(vb, kb);
            mfma<QK, i>(ops[i % kRing]);
            copy_step<i, NM>(cp);
            __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_s_setprio(0);
    }

    // ---- VALU phase ----------------------------------------------------------------
    // Element masks for active tile n (partial tiles only).  Key of accumulator
    // register r of block b: b*32 + 16*(r>>3) + 8g + (r&7).
    __device__ __forceinline__ void mask(int n) {
        bool partial;
        const int t = tile_of(n, partial);
        const int lim = S - t * kBk - 8 * g;
        const int* segt = sslot(n) + 8 * g;
        const bool live = myseg != 0;
        // The segment IDs of every key of the slot are read unconditionally
        // (the slot always holds 64; past S they repeat key S-1) and combined
        // with bitwise ands, so the masks compile to selects, not branches.
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int jc = b * 32 + 16 * (r >> 3) + (r & 7);
                bool ok = jc < lim;
                if (SEG) ok = ok & (segt[jc] == myseg) & live;
                sacc[b][r] = ok ? sacc[b][r] : -INFINITY;
            }
        }
    }
    // Online softmax of the current scores in the log2 domain, with a lazily
    // moved reference: m_run only moves when some row of the wave sees a
    // scaled score more than kLazyLog2 above it.  Then P = 2^(s*scale*log2(e)
    // - m_run) <= 2^kLazyLog2, and the rescale of O and l by 2^(m_old - m_new)
    // (an exp and 64 multiplies per lane) is skipped on nearly every tile.
    // out = O / l and lse = m_run + log2(l) do not depend on the reference.
    // l is summed in fp32 from the unrounded P (a sum of the bf16 P would
    // carry their 2^-9 rounding into lse).
    __device__ __forceinline__ void softmax() {
        float mx0 = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), sacc[0][2]);
        float mx1 = fmaxf(fmaxf(sacc[1][0], sacc[1][1]), sacc[1][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
            mx0 = fmaxf(fmaxf(mx0, sacc[0][r]), sacc[0][r + 1]);
            mx1 = fmaxf(fmaxf(mx1, sacc[1][r]), sacc[1][r + 1]);
        }
        const float mx = pair_max(fmaxf(fmaxf(mx0, sacc[0][15]), fmaxf(mx1, sacc[1][15]))) * c_log2;
        const bool move = mx > m_run + kLazyLog2;
        if (__ballot(move) != 0ull) {
            // Per row: only rows past their margin move (alpha = 2^0 = 1
            // exactly for the others), so a row's arithmetic never depends on
            // the other rows of the wave.  m_run = -inf (no valid key yet)
            // gives alpha = 2^-inf = 0.
            const float m_new = move ? mx : m_run;
            const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b][r], c_log2, -msub));
                ls[r & 3] += p;
                pb[b * 2 + (r >> 3)][r & 7] = (__bf16)p;
            }
        }
        l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        // Pin the results inside this phase: without a use here the optimiser
        // sinks the softmax next to its consumer (the next MFMA phase), which
        // would serialise it behind those MFMAs.
        asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3]), "v"(l_run), "v"(m_run));
    }
};

// Ping-pong schedule of group G.  Local iteration n: MFMA phase (K Q^T of
// tile n, P V of tile n-1) at global phase 2n + G, then the VALU phase
// (softmax of tile n) at 2n + 1 + G; a workgroup barrier closes every global
// phase.  In its VALU phase a wave also plans the next MFMA phase's tile copy
// and, once the softmax is done, fetches that phase's first K operands, so
// the MFMA phase starts issuing right after its barrier.  The MFMA phase
// issues the copy between its MFMAs and, before its closing barrier, waits for
// the copy of its previous MFMA phase, so a copy has two phases to land.  The
// first and last iterations are peeled so that the steady-state body has a
// single MFMA phase shape.
template <int G, class AT>
__device__ __forceinline__ void main_loop(AT& A, int n_act) {
    typename AT::Copy cp;
    auto valu_phase = [&](int n) {
        // The tile-list read for this phase's plan goes out first; the fence
        // keeps the scheduler from sinking it next to its use.
        const int ent = A.list_entry(n + 3 - G, n_act);
        if (AT::kSeg) __builtin_amdgcn_sched_barrier(0);
        if (A.template partial_planned<G>(n)) A.mask(n);
        A.softmax();
        A.template plan<G>(cp, n + 3 - G, n_act, ent);
        // Operands of the next MFMA phase (K Q^T of tile n+1; stale when n+1 is
        // past the last tile, and then unused).
        A.template prefetch<true, true>(n, n + 1);
        barrier();
    };
    A.template plan<G>(cp, 2 - G, n_act, A.list_entry(2 - G, n_act));
    A.template prefetch<false, true>(0, 0);
    if (G == 1) barrier();  // group 1 idles in global phase 0
    A.template mfma_phase<false, true, true>(0, 0, cp);
    wait_copies<AT::T::kLoadsPerWave>(cp.cnt);
    barrier();
    valu_phase(0);
    for (int n = 1; n < n_act; ++n) {
        const int c = cp.cnt;
        A.template mfma_phase<true, true, true>(n - 1, n, cp);
        wait_copies<AT::T::kLoadsPerWave>(c);
        barrier();
        valu_phase(n);
    }
    {
        const int c = cp.cnt;
        A.template mfma_phase<true, false, false>(n_act - 1, 0, cp);
        wait_copies<AT::T::kLoadsPerWave>(c);
        barrier();
    }
    if (G == 0) barrier();  // group 0 idles in the last global phase
}

// 3D rotary embedding of a workgroup's query block, staged in LDS before the
// K/V ring is in use: the block's kBq rows (D bf16 each, rows kQStage bytes
// apart so that neighbouring rows start in different banks) are copied in,
// two threads per row rewrite its rotated feature pairs in place (alternate
// pairs; the row's position is read once), and each lane then reads its Q
// slice from there.  The rule and its rounding are those of the key pre-pass
// (rope3d.h), so the bits equal a rotated copy of q.  The loops stay rolled,
// which keeps this prologue's registers far below the main loop's.  Rows past
// S stay zero.
template <int D>
struct QStage {
    static constexpr int kRowBytes = D * 2 + 16;
    static_assert(kBq * kRowBytes <= Tile<D>::kRingBytes, "the staged query block must fit in the ring");
    static_assert(kThreads == 2 * kBq, "two threads per staged row");
};

template <int D>
__device__ void rope_stage_q(char* smem, const __bf16* __restrict__ q, const Rope3DDev& r, int b, int h,
                             int S, int64_t tok_stride, int q0, int tid) {
    constexpr int kRowChunks = D / 8;
    constexpr int kStride = QStage<D>::kRowBytes;
#pragma unroll 1
    for (int c = tid; c < kBq * kRowChunks; c += kThreads) {
        const int row = c / kRowChunks, ch = c % kRowChunks;
        const int tok = q0 + row;
        bf16x8 x = {};
        if (tok < S)
            x = *reinterpret_cast<const bf16x8*>(q + ((int64_t)b * S + tok) * tok_stride + (int64_t)h * D + 8 * ch);
        *reinterpret_cast<bf16x8*>(smem + row * kStride + 16 * ch) = x;
    }
    __syncthreads();
    const int row = tid % kBq, hf = tid / kBq;
    const int tok = q0 + row;
    int pos[3] = {-1, -1, -1};
    if (tok < S) {
#pragma unroll
        for (int a = 0; a < 3; ++a) pos[a] = r.pos[((int64_t)b * S + tok) * 3 + a];
    }
    if (tok < S && rope_inside(r, pos)) {
        uint16_t* sb = reinterpret_cast<uint16_t*>(smem + row * kStride);
        const int h0 = r.d[0] >> 1, h1 = r.d[1] >> 1, h2 = r.d[2] >> 1;
        // walk pairs hf, hf + 2, ... of the concatenated sections: (a, p) is
        // the axis and the pair within it, off the section's first feature
        int a = 0, p = hf, off = 0;
#pragma unroll 1
        for (;;) {
            const int half = a == 0 ? h0 : (a == 1 ? h1 : h2);
            if (p >= half) {
                if (a == 2) break;
                p -= half;
                off += 2 * half;
                ++a;
                continue;
            }
            const int i0 = r.interleaved ? off + 2 * p : off + p;
            const int i1 = r.interleaved ? off + 2 * p + 1 : off + p + half;
            const int e = (a == 0 ? pos[0] : (a == 1 ? pos[1] : pos[2])) * half + p;
            const float c = (a == 0 ? r.cs[0] : (a == 1 ? r.cs[1] : r.cs[2]))[e];
            const float sn = (a == 0 ? r.sn[0] : (a == 1 ? r.sn[1] : r.sn[2]))[e];
            const float x0 = bf16_bits_to_f32(sb[i0]), x1 = bf16_bits_to_f32(sb[i1]);
            sb[i0] = rope_rotate(x0, x1, c, sn, true);
            sb[i1] = rope_rotate(x1, x0, c, sn, false);
            p += 2;
        }
    }
    __syncthreads();
}

// Work item w of a grid of n_wg items -> (b, h, query block), renumbered
// XCD-contiguously: item w runs on XCD w % 8 (workgroups are dealt to the
// XCDs round-robin and the persistent grid is a multiple of 8), and the
// items of one XCD are consecutive query blocks of one head, which share K/V
// tiles in that XCD's L2.
struct ItemPos {
    int b, h, qblk;
};
__device__ __forceinline__ ItemPos item_at(int lid, int n_qblk, int H) {
    const int bh = lid / n_qblk;
    return ItemPos{bh / H, bh % H, lid % n_qblk};
}
__device__ __forceinline__ ItemPos decode_item(int w, int n_wg, int n_qblk, int H) {
    const int per = n_wg / kXcds, rem = n_wg % kXcds;
    const int xcd = w % kXcds;
    return item_at(xcd * per + min(xcd, rem) + w / kXcds, n_qblk, H);
}

// Item j of XCD x in the scheduled order -> batch b, head h and longest-first
// rank r of its query block.  When 8 divides H, XCD x takes its heads x,
// x + 8, ... one after the other, each head's blocks batch by batch, longest
// first, so that its workgroups stream one head's K/V at a time; otherwise
// item e = x + 8 j of the list that walks the batches, then the blocks
// longest first, then the heads.
__device__ __forceinline__ void sched_coords(int x, int j, int H, int n_qblk, int n_items, int& b, int& h,
                                             int& r) {
    if (H % kXcds == 0) {
        const int per_head = n_items / H;  // B * n_qblk
        const int hi = j / per_head, rem = j - hi * per_head;
        h = x + kXcds * hi;
        b = rem / n_qblk;
        r = rem - b * n_qblk;
    } else {
        const int e = x + kXcds * j;
        h = e % H;
        const int rb = e / H;
        r = rb % n_qblk;
        b = rb / n_qblk;
    }
}

// ---- split items of a persistent launch --------------------------------------------
// With a workspace for partial results, an item can be split along its active
// key tiles into P parts that run side by side; a combine kernel then merges
// the parts of each split item.  Which items are split is set by tail_plan.
constexpr int kTailMaxParts = 8;
constexpr int kTailRecords = 256;  // part records a workspace holds (one per workgroup of a 256-CU grid)
// Floats of one part record: the unnormalised O^T of the block's kBq rows as
// [D / 8][kBq][8] (row-contiguous 8-float chunks of d), then the reference
// maximum m (log2 units of the scaled score) and the key sum l of every row
// (l = 0: no valid key in the part).  A multiple of 64 floats.
template <int D>
constexpr size_t tail_record_floats() { return (size_t)kBq * D + 2 * kBq; }
static_assert(tail_record_floats<128>() % 64 == 0 && tail_record_floats<64>() % 64 == 0, "records stay 256-byte aligned");

// Persistent schedules.  XCD x holds n_x = per + (x < rem) items
// (per = n / 8, rem = n mod 8; unmasked a contiguous run starting at item
// x per + min(x, rem), masked the XCD's longest-first list of sched_coords),
// handed out by the XCD's own counter, so that its W = G / 8 workgroups take
// neighbouring items of one head together and share its K/V in their L2.
// The XCDs do not run the kernels at the same speed (per-item timestamps put
// the odd-numbered ones 4-5% behind the even ones on two devices, all
// through the launch), and equal shares would leave the faster ones idle at
// the end.  So that the faster XCDs take over the slower ones' last items:
//   - unmasked (tail_plan, claim_unit): work stealing.  A workgroup whose own
//     counter has run out takes units from the other XCDs' counters (x + 1,
//     x + 2, ... in turn) until every counter has, each thief an item of its
//     victim's current head.  The last R items of each XCD are split into
//     P = min(8, W / R) parts along their key tiles (when that makes at least
//     2), after its n_x - R whole ones: R = W / 4 for a long launch
//     (n_x / W >= kLongRounds), else R = n_x mod W, the ragged last round,
//     which the parts then fill (without parts to take, stealing measured
//     0.5% slower than none on a launch of 6 whole rounds; with them 0.6%
//     faster).  Unit u of XCD x: u < n_x - R is whole item
//     u; otherwise t = u - (n_x - R) is part t / R of item n_x - R + t % R,
//     with its partial results in record x W + t.  The shared pool below,
//     tried here too, balanced as well but cost 50 GB more L2 misses per
//     720p call, its workgroups leaving their XCD's head for two rounds;
//   - masked (pool_plan, pool_sched_item): a shared pool.  XCD x's counter
//     hands out its first K W list positions (K = n_x / W - kPoolRounds for a
//     long launch, n_x / W >= kLongRounds, else n_x / W); the rest of
//     every XCD's list forms a pool of n - K G items, XCD-major, pulled
//     through a ninth counter by any workgroup whose own XCD is done, and the
//     pool's last R items (G / 4 for a long launch, else all of them) are
//     split into P = min(8, 256 / R, G / R) parts when that is >= 2, with
//     part t in record t.  Work stealing measured no faster than no balancing
//     here (the slower XCDs' remaining items were mostly already running when
//     the thieves came), the pool 2.4-2.9% faster.
constexpr int kLongRounds = 4;
constexpr int kPoolRounds = 2;
struct TailPlan {
    int n_x;    // items of the XCD
    int R, P;   // split items and parts per item (R = 0: no split)
    __host__ __device__ int units() const { return n_x - R + R * P; }
};
__host__ __device__ inline TailPlan tail_plan(int x, int n_items, int W, int long_rounds) {
    TailPlan t{n_items / kXcds + (x < n_items % kXcds ? 1 : 0), 0, 1};
    if (t.n_x > W) {
        const int R = t.n_x / W >= long_rounds ? W / 4 : t.n_x % W;
        const int P = R > 0 ? min(kTailMaxParts, W / R) : 1;
        if (P >= 2) {
            t.R = R;
            t.P = P;
        }
    }
    return t;
}
struct PoolPlan {
    int per, rem;  // items of XCD x: per + (x < rem)
    int K;         // rounds of every XCD's own items
    int n_pool;    // n - K G
    int R, P;      // pool items split (the last R) and parts per split item (R = 0: none)
    __host__ __device__ int units() const { return n_pool - R + R * P; }
};
__host__ __device__ inline PoolPlan pool_plan(int n_items, int G) {
    const int W = G / kXcds;
    PoolPlan p{n_items / kXcds, n_items % kXcds, 0, 0, 0, 1};
    const int rounds = p.per / W;
    const bool long_launch = rounds >= kLongRounds;
    p.K = long_launch ? rounds - kPoolRounds : rounds;
    p.n_pool = n_items - p.K * G;
    const int R = long_launch ? min(p.n_pool, G / 4) : p.n_pool % G;
    const int P = R > 0 ? min(min(kTailMaxParts, kTailRecords / R), G / R) : 1;
    if (P >= 2) {
        p.R = R;
        p.P = P;
    }
    return p;
}
// Pool item i -> XCD x and list position j: XCD-major (XCD x's t0 + (x < rem)
// pool items, t0 = per - K W, after those of the XCDs below it), so that the
// workgroups that reach the pool together take one XCD's items, one head's
// K/V in their L2 (interleaving the XCDs' items measured the same time and
// 40-60% more L2 misses).
__host__ __device__ inline void pool_sched_item(const PoolPlan& p, int i, int W, int& x, int& j) {
    const int t0 = p.per - p.K * W;
    int k;
    if (i < p.rem * (t0 + 1)) {
        x = i / (t0 + 1);
        k = i - x * (t0 + 1);
    } else {
        const int i2 = i - p.rem * (t0 + 1);
        x = p.rem + i2 / max(t0, 1);
        k = i2 - (x - p.rem) * t0;
    }
    j = p.K * W + k;
}
// Claims the next unit for a workgroup of XCD xcd: from its own counter,
// then (once that has run out) from the others' in turn; v counts the
// counters found empty, so each is skipped afterwards.  Returns false when
// every counter has run out.  The slot in the LDS carries thread 0's
// claim to the whole workgroup; the barriers keep it from being reused
// early.  Unit u of XCD x is returned.
template <class Units>
__device__ __forceinline__ bool claim_unit(uint32_t* __restrict__ ctr, int* slot, int xcd, int& v, int& x, int& u,
                                           Units units) {
    for (; v < kXcds; ++v) {
        x = (xcd + v) % kXcds;
        if (threadIdx.x == 0) *slot = (int)atomicAdd(ctr + x, 1u);
        __syncthreads();
        u = __builtin_amdgcn_readfirstlane(*slot);
        __syncthreads();  // every wave has the slot before it is reused
        if (u < units(x)) return true;
    }
    return false;
}

// What one workgroup of a persistent launch runs: query block it, whole
// (rec == nullptr) or part p of P of its active key tiles with its partial
// results in record rec.
struct TailPart {
    float* rec;
    int p, P;
};

// One query block (256 queries of one (b, h)).  With segment IDs the key
// tiles are classified from the IDs themselves (SUM false) or from the
// per-tile summaries tsum of the batch (SUM true, see attn_fwd_tilesum_kernel).
template <int D, bool SEG, bool ROPE, bool SUM, bool PART>
__device__ __forceinline__ void attn_fwd_item(
    char* smem, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const int32_t* __restrict__ seg_q,
    const int32_t* __restrict__ seg_kv, __bf16* __restrict__ out, float* __restrict__ lse, int S,
    int H, float c_log2, int n_kvt, ItemPos it, const int4* __restrict__ tsum, const Rope3DDev& rope,
    TailPart part = TailPart{nullptr, 0, 1}) {
    using T = Tile<D>;
    const int qblk = it.qblk, h = it.h, b = it.b;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 31, g = lane >> 5;
    const int grp = wave >> 2;  // ping-pong group; waves w and w+4 share a SIMD
    const int qi = qblk * kBq + wave * 32 + lr;

    Attn<D, SEG, PART> A;
    A.smem = smem;
    A.tok_stride = (int64_t)H * D;
    A.kp = k + (int64_t)b * S * A.tok_stride + (int64_t)h * D;
    A.vp = v + (int64_t)b * S * A.tok_stride + (int64_t)h * D;
    A.segkv = SEG ? seg_kv + (int64_t)b * S : nullptr;
    A.S = S;
    A.n_kvt = n_kvt;
    A.t0 = 0;
    A.last_view = true;
    A.wave = wave;
    A.w4 = wave & 3;
    A.lane = lane;
    A.lr = lr;
    A.g = g;
    A.c_log2 = c_log2;

    // ---- Q slice -> registers as the B operand of S^T = K Q^T -----------------
    if constexpr (ROPE) {
        rope_stage_q<D>(smem, q, rope, b, h, S, A.tok_stride, qblk * kBq, tid);
        const char* st = smem + (wave * 32 + lr) * QStage<D>::kRowBytes + 16 * g;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) A.qreg[ks] = *reinterpret_cast<const bf16x8*>(st + ks * 32);
        A.myseg = SEG ? ((qi < S) ? seg_q[(int64_t)b * S + qi] : 0) : 1;
        // The classifier's scratch and the ring copies reuse this LDS.
        __syncthreads();
    } else {
        const __bf16* qrow = q + ((int64_t)b * S + qi) * A.tok_stride + (int64_t)h * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks)
            A.qreg[ks] = (qi < S) ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16) : bf16x8{};
        A.myseg = SEG ? ((qi < S) ? seg_q[(int64_t)b * S + qi] : 0) : 1;
    }
    // ---- per-lane LDS offsets ---------------------------------------------------
    {
        // K: lane (lr, g) of k-step ks reads chunk 2ks+g of row swap23(lr), stored
        // at chunk (2ks+g) ^ ksw = (g ^ ksw) ^ 2ks.
        const int ksw = lr & (T::kChunks - 1);  // == k_swz(row) for row = swap23(lr)
        A.kx = swap23(lr) * T::kRowBytes + ((g ^ ksw) << 4);
        // Transposed V read: group q = lane/16 takes d = db*32 + 16(q&1) + 4(j&3)
        // and keys 8(q>>1) + (j>>2) (+4 for the second half of the operand); the
        // 32-byte chunk 2db + (q&1) sits at (2db + (q&1)) ^ vsw = ((q&1) ^ vsw) ^ 2db
        // (vsw is even).
        const int qg = lane >> 4, j = lane & 15;
        const int key = 8 * (qg >> 1) + (j >> 2);
        const int vsw = v_swz<D>(key);
        A.vx = key * T::kRowBytes + 32 * ((qg & 1) ^ vsw) + 16 * ((j & 3) >> 1) + 8 * (j & 1);
        // Tile copies: instruction i of a tile covers rows kRowsPerLoad*i .. ; a
        // lane lands at LDS position pos of its row and fetches the chunk stored
        // there (K layout for group 0, V layout for group 1).
#pragma unroll
        for (int jj = 0; jj < T::kLoadsPerWave; ++jj) {
            const int i = A.w4 * T::kLoadsPerWave + jj;
            const int r = T::kRowsPerLoad * i + lane / T::kChunks;
            const int pos = lane % T::kChunks;
            const int c = grp ? 2 * ((pos >> 1) ^ v_swz<D>(r)) + (pos & 1) : (pos ^ k_swz<D>(r));
            A.dmo[jj] = 2u * (uint32_t)(r * (int)A.tok_stride + c * 8);
        }
    }

    uint16_t* list = reinterpret_cast<uint16_t*>(smem + T::kRingBytes);
    int* meta = reinterpret_cast<int*>(smem + ((T::kRingBytes + 2 * (SEG ? n_kvt : 0) + 15) & ~15));
    // meta: classify_tiles' scratch (3 kWaves + 1 ints)
    A.list = list;

    int n_act = n_kvt;
    if (SEG) {
        // ---- classify the key tiles against this query block (skip / full /
        // partial) and compact the active ones into the LDS list ----------------
        // Every lane reads the same count from the LDS; readfirstlane states
        // that it is wave-uniform, so the loop bounds and ring-slot offsets
        // derived from it stay in scalar registers.
        if constexpr (SUM)
            n_act = __builtin_amdgcn_readfirstlane(classify_tiles_sum<kWaves, true>(
                A.myseg, tsum, n_kvt, reinterpret_cast<uint8_t*>(smem), list, meta, wave, lane));
        else
            n_act = __builtin_amdgcn_readfirstlane(classify_tiles<kWaves, true>(
                A.myseg, A.segkv, S, n_kvt, reinterpret_cast<uint8_t*>(smem), list, meta, wave, lane));
    }
    if constexpr (PART) {
        if (part.rec != nullptr) {
            // Part p of P: active tiles [n_act p / P, n_act (p + 1) / P).
            const int a0 = (int)((int64_t)n_act * part.p / part.P);
            const int a1 = (int)((int64_t)n_act * (part.p + 1) / part.P);
            n_act = a1 - a0;
            if (SEG) {
                A.list = list + a0;
            } else {
                A.t0 = a0;
                A.n_kvt = n_act;
                A.last_view = a1 == n_kvt;
            }
        }
        // The record address waits in the LDS (meta[28..29], past the
        // classifier's scratch) until the epilogue, so that it holds no
        // registers through the main loop; the barrier after the prologue
        // copies makes it visible.
        if (tid == 0) *reinterpret_cast<float**>(meta + 28) = part.rec;
    }

    // ---- running softmax state and the O^T accumulators -----------------------
#pragma unroll
    for (int i = 0; i < T::kDBlocks; ++i) A.oacc[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < 4; ++i) A.pb[i] = bf16x8{};
    A.m_run = -INFINITY;  // running max of scale*log2(e)*s for this lane's query
    A.l_run = 0.f;        // this lane's partial sum (its half of each tile's keys)

    // ---- prologue: K of tiles 0 and 1, segment IDs of tile 0 (group 0), V of
    // tile 0 (group 1) ---------------------------------------------------------------
    if (SEG) {
        A.prev_t = 0;
        A.prev_part = false;
        A.phist = 0u;
    }
    {
        typename Attn<D, SEG, PART>::Copy c;
        if (grp == 0) {
            for (int a = 0; a < 2; ++a) {
                A.template plan<0>(c, a, n_act, A.list_entry(a, n_act));  // K tile a, segment IDs of tile a-1
                A.copy_start(c);
                if (c.spread) {
#pragma unroll
                    for (int j = 0; j < T::kLoadsPerWave; ++j) dma16(c.src, A.dmo[j], c.dst + j * 1024);
                }
            }
        } else {
            A.template plan<1>(c, 0, n_act, A.list_entry(0, n_act));
            A.copy_start(c);
            if (c.spread) {
#pragma unroll
                for (int j = 0; j < T::kLoadsPerWave; ++j) dma16(c.src, A.dmo[j], c.dst + j * 1024);
            }
        }
    }
    wait_vm(0);
    barrier();
    // A use of the Q registers (and the query's segment ID) here makes the
    // compiler wait for their loads before the loop rather than inside it,
    // where a vmcnt wait would also drain the in-flight tile copies.
    asm volatile("" ::"v"(A.qreg[0]), "v"(A.qreg[T::kSteps - 1]), "v"(A.myseg));

    // ---- ping-pong main loop --------------------------------------------------------
    if (n_act > 0) {
        if (grp == 0)
            main_loop<0>(A, n_act);
        else
            main_loop<1>(A, n_act);
    }

    // ---- epilogue: normalise, write out (bf16) and lse (fp32) ----------------
    const float l_tot = pair_sum(A.l_run);
    float* ro = nullptr;
    if constexpr (PART) {
        ro = *reinterpret_cast<float* const volatile*>(meta + 28);
        uint64_t rv = reinterpret_cast<uint64_t>(ro);
        rv = ((uint64_t)__builtin_amdgcn_readfirstlane((int)(rv >> 32)) << 32) |
             (uint32_t)__builtin_amdgcn_readfirstlane((int)rv);
        ro = reinterpret_cast<float*>(rv);
    }
    if (PART && ro != nullptr) {
        // A part writes its unnormalised state; attn_fwd_combine_kernel
        // finishes the row.  Padding rows (ID 0) report no valid key.
        const int row = wave * 32 + lr;
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<float4*>(ro + ((size_t)(db * 4 + r4) * kBq + row) * 8 + 4 * g) =
                    float4{A.oacc[db][4 * r4], A.oacc[db][4 * r4 + 1], A.oacc[db][4 * r4 + 2],
                           A.oacc[db][4 * r4 + 3]};
        if (g == 0) {
            ro[(size_t)kBq * D + row] = A.m_run;
            ro[(size_t)kBq * D + kBq + row] = A.myseg != 0 ? l_tot : 0.f;
        }
    } else if (qi < S) {
        __bf16* orow = out + ((int64_t)b * S + qi) * A.tok_stride + (int64_t)h * D;
        float lse_v;
        // A padding row (ID 0) may have run through full tiles unmasked (the
        // classifier does not let a block's own padding make a tile partial):
        // it is written as a row without valid keys.
        if (l_tot > 0.f && A.myseg != 0) {
            const float inv = 1.0f / l_tot;
#pragma unroll
            for (int db = 0; db < T::kDBlocks; ++db) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = db * 32 + 8 * r4 + 4 * g;
                    __bf16 o4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(A.oacc[db][4 * r4 + e] * inv);
                    *reinterpret_cast<uint2*>(orow + d) = *reinterpret_cast<const uint2*>(o4);
                }
            }
            lse_v = (A.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
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

// Dynamic LDS of a launch: the K/V/segment-ID ring, then (masked) the
// active-tile list of n_kvt entries and classify_tiles' metadata.
template <int D, bool SEG>
constexpr size_t fwd_lds(int n_kvt) {
    size_t lds = (size_t)Tile<D>::kRingBytes;
    if (SEG) lds += 2 * (size_t)n_kvt;
    lds = (lds + 15) & ~(size_t)15;
    return lds + 32 * sizeof(int);  // meta
}
static_assert(fwd_lds<128, true>(kMaxKvTiles) <= kLdsBytes && fwd_lds<64, true>(kMaxKvTiles) <= kLdsBytes,
              "a full active-tile list must fit in the LDS beside the ring");

// Workgroup p takes items p, p + G, p + 2G, ... (G = the grid size: one per
// item with segment IDs, else a persistent grid, a multiple of 8).  At every
// step the G/8 workgroups of an XCD then work on consecutive query blocks of
// one head, streaming the same K/V tiles at the same time, which keeps them
// in that XCD's L2; with one workgroup per item, CUs that pick up new items
// at different times drift apart and each re-fetches the tiles.  SPLIT (a
// persistent grid with part records recs and eight zeroed counters ctr): the
// same items, claimed through the counters with work stealing and the last
// ones split (tail_plan with kLongRounds, claim_unit); every claim past the
// last counter ends the loop, so all waves exit.
template <int D, bool SEG, bool ROPE, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_kv,
    __bf16* __restrict__ out, float* __restrict__ lse, int S, int H, float c_log2, int n_qblk,
    int n_kvt, int n_wg, Rope3DDev rope, float* __restrict__ recs, uint32_t* __restrict__ ctr) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    if constexpr (!SPLIT) {
        for (int w = blockIdx.x; w < n_wg; w += gridDim.x) {
            attn_fwd_item<D, SEG, ROPE, false, false>(smem, q, k, v, seg_q, seg_kv, out, lse, S, H, c_log2,
                                                      n_kvt, decode_item(w, n_wg, n_qblk, H), nullptr, rope);
            // Every wave is done with the LDS of this item before the next
            // one's copies land there.
            __syncthreads();
        }
    } else {
        // The schedule is recomputed every iteration (the empty asm keeps the
        // compiler from hoisting it), so that only the counter position v is
        // carried through the item, as the loop above carries w.
        int* slot = reinterpret_cast<int*>(smem + fwd_lds<D, SEG>(n_kvt) - sizeof(int));
        int vv = 0;
        for (;;) {
            int xcd = blockIdx.x % kXcds, G = gridDim.x;
            asm volatile("" : "+s"(xcd), "+s"(G));
            const int W = G / kXcds;
            int x, u;
            if (!claim_unit(ctr, slot, xcd, vv, x, u,
                            [&](int y) { return tail_plan(y, n_wg, W, kLongRounds).units(); }))
                break;
            const TailPlan tp = tail_plan(x, n_wg, W, kLongRounds);
            const int n_whole = tp.n_x - tp.R;
            int j = u;
            TailPart part{nullptr, 0, 1};
            if (u >= n_whole) {
                const int t = u - n_whole;
                part = TailPart{recs + (size_t)(x * W + t) * tail_record_floats<D>(), t / tp.R, tp.P};
                j = n_whole + t % tp.R;
            }
            attn_fwd_item<D, SEG, ROPE, false, true>(smem, q, k, v, seg_q, seg_kv, out, lse, S, H, c_log2, n_kvt,
                                                     decode_item(x + kXcds * j, n_wg, n_qblk, H), nullptr, rope,
                                                     part);
            __syncthreads();
        }
    }
}

// Merges the P parts of every split item, d columns 32 blockIdx.z ..
// 32 blockIdx.z + 31: per row, M = the largest reference maximum among the
// parts with valid keys, L = sum_p l_p 2^(m_p - M), O = sum_p O_p 2^(m_p - M);
// out = O / L (bf16) and lse = (M + log2 L) ln 2, or +0 / -inf when L = 0.
// One thread per row; parts are added in index order, so the result is
// deterministic.  SCHED: split item r = blockIdx.x of attn_fwd_sched_kernel's
// pool (pool item n_pool - R + r, longest-first block order ord, part p in
// record r + p R); else split item r of XCD x = blockIdx.y of
// attn_fwd_kernel (item n_x - R + r of the XCD, part p in record
// x W + r + p R).
template <int D, bool SCHED>
__global__ __launch_bounds__(kBq) void attn_fwd_combine_kernel(const float* __restrict__ recs,
                                                               const int* __restrict__ ord,
                                                               __bf16* __restrict__ out, float* __restrict__ lse,
                                                               int S, int H, int n_qblk, int n_items, int G) {
    const int r = blockIdx.x, c0 = 4 * blockIdx.z, W = G / kXcds;
    constexpr size_t RF = tail_record_floats<D>();
    ItemPos it;
    const float* rec0;
    int R, P;
    if (SCHED) {
        const PoolPlan pp = pool_plan(n_items, G);
        if (r >= pp.R) return;
        int x, j, b, h, rr;
        pool_sched_item(pp, pp.n_pool - pp.R + r, W, x, j);
        sched_coords(x, j, H, n_qblk, n_items, b, h, rr);
        const int o = ord[(int64_t)b * n_qblk + rr];
        it = ItemPos{b, h, (unsigned)o < (unsigned)n_qblk ? o : 0};
        rec0 = recs + (size_t)r * RF;
        R = pp.R;
        P = pp.P;
    } else {
        const int x = blockIdx.y;
        const TailPlan tp = tail_plan(x, n_items, W, kLongRounds);
        if (r >= tp.R) return;
        it = decode_item(x + kXcds * (tp.n_x - tp.R + r), n_items, n_qblk, H);
        rec0 = recs + (size_t)(x * W + r) * RF;
        R = tp.R;
        P = tp.P;
    }
    const int row = threadIdx.x;
    const int qi = it.qblk * kBq + row;
    if (qi >= S) return;
    const size_t pstride = (size_t)R * RF;  // part p of this item: R records further
    float M = -INFINITY;
    for (int p = 0; p < P; ++p) {
        const float* rp = rec0 + p * pstride;
        if (rp[(size_t)kBq * D + kBq + row] > 0.f) M = fmaxf(M, rp[(size_t)kBq * D + row]);
    }
    float L = 0.f;
    float acc[4][8] = {};
    for (int p = 0; p < P; ++p) {
        const float* rp = rec0 + p * pstride;
        const float l = rp[(size_t)kBq * D + kBq + row];
        if (!(l > 0.f)) continue;
        const float w = __builtin_amdgcn_exp2f(rp[(size_t)kBq * D + row] - M);
        L += w * l;
        float4 v[4][2];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const float4* src = reinterpret_cast<const float4*>(rp + ((size_t)(c0 + cc) * kBq + row) * 8);
            v[cc][0] = src[0];
            v[cc][1] = src[1];
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            acc[cc][0] += w * v[cc][0].x;
            acc[cc][1] += w * v[cc][0].y;
            acc[cc][2] += w * v[cc][0].z;
            acc[cc][3] += w * v[cc][0].w;
            acc[cc][4] += w * v[cc][1].x;
            acc[cc][5] += w * v[cc][1].y;
            acc[cc][6] += w * v[cc][1].z;
            acc[cc][7] += w * v[cc][1].w;
        }
    }
    __bf16* orow = out + ((int64_t)it.b * S + qi) * H * D + (int64_t)it.h * D + 8 * c0;
    const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        __bf16 o8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = (__bf16)(acc[cc][e] * inv);
        *reinterpret_cast<uint4*>(orow + 8 * cc) = *reinterpret_cast<const uint4*>(o8);
    }
    if (blockIdx.z == 0)
        lse[((int64_t)it.b * H + it.h) * S + qi] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

// ---- scheduled masked forward (caller workspace) -------------------------------------
// With segment IDs, item lengths differ by up to ~10x (a query block of a
// short clip skips most key tiles), and the hardware dispatcher, which hands
// workgroups to the XCDs round-robin in index order, leaves CUs idle behind a
// long item.  The scheduled path instead runs a persistent grid whose
// workgroups pull items from eight work counters (one per XCD, with work
// stealing) in longest-first order, and classifies key tiles from per-tile
// summaries instead of every workgroup re-reading all of the batch's key
// IDs.  Workspace: the eight work counters (256 bytes), then int4 tile
// summaries [B][n_kvt], active-tile counts [B][n_qblk], the longest-first
// block orders [B][n_qblk] and kTailRecords part records of split items
// (sized for D = 128).  An unmasked call uses only the counters and the part
// records.
struct FwdWs {
    uint32_t* ctr;
    int4* tsum;
    int* cnt;
    int* ord;
    float* recs;  // kTailRecords part records of split items
};
__host__ __device__ inline size_t fwd_ws_align(size_t x) { return (x + 255) & ~(size_t)255; }
FwdWs fwd_ws_layout(void* ws, int64_t B, int64_t n_kvt, int64_t n_qblk) {
    char* p = reinterpret_cast<char*>(ws);
    FwdWs w;
    w.ctr = reinterpret_cast<uint32_t*>(p);
    p += 256;
    w.tsum = reinterpret_cast<int4*>(p);
    p += fwd_ws_align((size_t)(B * n_kvt) * sizeof(int4));
    w.cnt = reinterpret_cast<int*>(p);
    p += fwd_ws_align((size_t)(B * n_qblk) * sizeof(int));
    w.ord = reinterpret_cast<int*>(p);
    p += fwd_ws_align((size_t)(B * n_qblk) * sizeof(int));
    w.recs = reinterpret_cast<float*>(p);
    return w;
}

// Summary of every 64-key tile of every batch: {min nonzero ID, max nonzero
// ID, flag (an ID 0 or a key past S), 0}, the quantities classify_tiles
// reduces; 16 lanes a tile, 4 IDs a lane.  Workgroup 0 also zeroes the work
// counters of the launch that follows on the stream.
__global__ __launch_bounds__(256) void attn_fwd_tilesum_kernel(const int32_t* __restrict__ seg_kv, int S,
                                                               int n_kvt, int64_t n_all, int4* __restrict__ tsum,
                                                               uint32_t* __restrict__ ctr) {
    if (blockIdx.x == 0 && threadIdx.x <= kXcds) ctr[threadIdx.x] = 0u;  // eight XCD counters and the pool's
    const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    int mn = INT32_MAX, mx = INT32_MIN, fl = 0;
    if (t < n_all) {
        const int64_t b = t / n_kvt;
        const int tt = (int)(t - b * n_kvt);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = tt * kBk + 4 * sub + e;
            const int x = (r < S) ? seg_kv[b * S + r] : 0;
            mn = (x != 0) ? min(mn, x) : mn;
            mx = (x != 0) ? max(mx, x) : mx;
            fl |= (x == 0) ? 1 : 0;
        }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
        mn = min(mn, __shfl_xor(mn, o));
        mx = max(mx, __shfl_xor(mx, o));
        fl |= __shfl_xor(fl, o);
    }
    if (sub == 0 && t < n_all) tsum[t] = int4{mn, mx, fl, 0};
}

// Active-tile count of every query block, workgroup b * n_qblk + blk: the
// block's rows are summarised as the forward summarises them and every key
// tile is classified from its summary.
constexpr int kCountWaves = kBq / 64;  // one thread per query row of the block
__global__ __launch_bounds__(kBq) void attn_fwd_count_kernel(const int32_t* __restrict__ seg_q,
                                                            const int4* __restrict__ tsum, int S, int n_qblk,
                                                            int n_kvt, int* __restrict__ cnt) {
    __shared__ int meta[4 * kCountWaves];
    const int blk = blockIdx.x % n_qblk, b = blockIdx.x / n_qblk;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int row = blk * kBq + tid;
    const int mine = (row < S) ? seg_q[(int64_t)b * S + row] : 0;
    int omn, omx, ofl;
    block_summary<kCountWaves>(mine, meta, wave, lane, omn, omx, ofl);
    const int4* ts = tsum + (int64_t)b * n_kvt;
    int c = 0;
    for (int t = tid; t < n_kvt; t += kBq) {
        const int4 x = ts[t];
        c += tile_class<true>(omn, omx, ofl, x.x, x.y, x.z) != 0 ? 1 : 0;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
    if (lane == 0) meta[3 * kCountWaves + wave] = c;
    __syncthreads();
    if (tid == 0) {
        int n = 0;
#pragma unroll
        for (int i = 0; i < kCountWaves; ++i) n += meta[3 * kCountWaves + i];
        cnt[(int64_t)b * n_qblk + blk] = n;
    }
}

// Longest-first order of the query blocks of batch b (workgroup b): ord[r]
// is the block with the r-th largest count, ties by block index (a
// permutation of 0 .. n_qblk - 1).
constexpr int kFwdRankThreads = 1024;
__global__ __launch_bounds__(kFwdRankThreads) void attn_fwd_rank_kernel(const int* __restrict__ cnt,
                                                                       int* __restrict__ ord, int n_qblk) {
    extern __shared__ int c[];
    const int64_t base = (int64_t)blockIdx.x * n_qblk;
    for (int i = threadIdx.x; i < n_qblk; i += kFwdRankThreads) c[i] = cnt[base + i];
    __syncthreads();
    for (int i = threadIdx.x; i < n_qblk; i += kFwdRankThreads) {
        const int ci = c[i];
        int r = 0;
        for (int j = 0; j < n_qblk; ++j) r += (c[j] > ci) | ((c[j] == ci) & (j < i));
        ord[base + r] = i;
    }
}

// Persistent masked forward: workgroup p (on XCD x = p % 8) pulls slot k of
// its XCD's counter and runs item k of the XCD's list (sched_coords): when 8
// divides H, its heads x, x + 8, ... one after the other, each head's blocks
// batch by batch, longest first (block ord[b][r]), so that the XCD's
// workgroups stream one head's K/V at a time; otherwise every eighth item of
// the list that walks the batches, then the blocks longest first, then the
// heads.  Either way the XCD takes an eighth of the work, longest first within
// a head, and its workgroups stay busy until its list runs out.  POOL
// (pool_plan): an XCD's counter hands out only its first K W list positions;
// the rest of every XCD's list forms a pool (pool_sched_item) pulled through
// a ninth counter by any workgroup whose own XCD is done, its last R items
// split into parts with records in the workspace.  Every item is pulled
// exactly once (each counter hands out 0, 1, 2, ...), and a workgroup exits
// at the first slot past what is left, so every wave exits.  Requires a grid
// that is a multiple of 8.  ROPE: the queries are rotated in the item
// prologue, as in attn_fwd_kernel.
template <int D, bool ROPE, bool POOL>
__global__ __launch_bounds__(kThreads) void attn_fwd_sched_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_kv,
    __bf16* __restrict__ out, float* __restrict__ lse, int S, int H, float c_log2, int n_qblk,
    int n_kvt, int n_items, FwdWs ws, Rope3DDev rope) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    int* slot = reinterpret_cast<int*>(smem + fwd_lds<D, true>(n_kvt) - sizeof(int));
    bool own = true;  // the XCD's own counter may still hold items
    for (;;) {
        // Recomputed every iteration (see attn_fwd_kernel), so that nothing
        // but the kernel arguments and the flag is carried through an item.
        int xcd = blockIdx.x % kXcds, G = gridDim.x;
        asm volatile("" : "+s"(xcd), "+s"(G));
        const int W = G / kXcds;
        const PoolPlan pp = pool_plan(n_items, G);
        int x = xcd, j = 0;
        TailPart part{nullptr, 0, 1};
        if (own) {
            if (threadIdx.x == 0) *slot = (int)atomicAdd(ws.ctr + xcd, 1u);
            __syncthreads();
            j = __builtin_amdgcn_readfirstlane(*slot);
            __syncthreads();  // every wave has the slot before it is reused
            if (j >= (POOL ? pp.K * W : pp.per + (xcd < pp.rem ? 1 : 0))) {
                if (!POOL) break;
                own = false;
            }
        }
        if (POOL && !own) {
            if (threadIdx.x == 0) *slot = (int)atomicAdd(ws.ctr + kXcds, 1u);
            __syncthreads();
            const int u = __builtin_amdgcn_readfirstlane(*slot);
            __syncthreads();
            if (u >= pp.units()) break;
            const int n_whole = pp.n_pool - pp.R;
            int i = u;
            if (u >= n_whole) {
                const int t = u - n_whole;
                part = TailPart{ws.recs + (size_t)t * tail_record_floats<D>(), t / pp.R, pp.P};
                i = n_whole + t % pp.R;
            }
            pool_sched_item(pp, i, W, x, j);
        }
        int b, h, r;
        sched_coords(x, j, H, n_qblk, n_items, b, h, r);
        const int o = ws.ord[(int64_t)b * n_qblk + r];
        const ItemPos it{b, h, (unsigned)o < (unsigned)n_qblk ? o : 0};  // a permutation; the test keeps it in range
        attn_fwd_item<D, true, ROPE, true, POOL>(smem, q, k, v, seg_q, seg_kv, out, lse, S, H, c_log2, n_kvt, it,
                                                 ws.tsum + (int64_t)b * n_kvt, rope, part);
        __syncthreads();
    }
}

// Workgroups of the persistent grid: one per CU (the kernel's LDS and
// registers allow one), rounded down to a multiple of the XCD count; cached
// per device.
int64_t persistent_workgroups() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < kMaxDev) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < kXcds)
        cus = 256;
    const int g = cus / kXcds * kXcds;
    if (dev < kMaxDev) cache[dev].store(g, std::memory_order_relaxed);
    return g;
}


// Largest split-item count R over the XCDs of a persistent grid (0: no item
// is split, and no combine launch is needed).
int tail_max_r(int n_items, int grid, int long_rounds) {
    int m = 0;
    for (int x = 0; x < kXcds; ++x) m = std::max(m, tail_plan(x, n_items, grid / kXcds, long_rounds).R);
    return m;
}

// Zeroes the eight work counters of an unmasked persistent launch (a
// kernel, not a memset, so that the call can be captured in a graph).
__global__ void attn_fwd_ctr_reset_kernel(uint32_t* __restrict__ ctr) {
    if (threadIdx.x < kXcds) ctr[threadIdx.x] = 0u;
}

template <int D, bool SCHED>
hipError_t launch_combine(const AttnArgs& a, const float* recs, const int* ord, int n_qblk, int n_items, int grid,
                          hipStream_t stream) {
    const int max_r = SCHED ? pool_plan(n_items, grid).R : tail_max_r(n_items, grid, kLongRounds);
    if (max_r == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_fwd_combine_kernel<D, SCHED>), dim3((unsigned)max_r, SCHED ? 1 : kXcds, D / 32),
                       dim3(kBq), 0, stream, recs, ord, reinterpret_cast<__bf16*>(a.out), a.lse, a.S, a.H, n_qblk,
                       n_items, grid);
    return hipGetLastError();
}

// ws: a caller workspace (unmasked calls with more items than the persistent
// grid then take the stealing schedule), or nullptr.
template <int D, bool SEG, bool ROPE>
hipError_t launch_t(const AttnArgs& a, const Rope3DDev& rope, hipStream_t stream, const FwdWs* ws = nullptr) {
    const int n_qblk = (a.S + kBq - 1) / kBq;
    const int n_kvt = (a.S + kBk - 1) / kBk;
    const int64_t n_wg64 = (int64_t)a.B * a.H * n_qblk;
    const int n_wg = (int)n_wg64;
    const size_t lds = fwd_lds<D, SEG>(n_kvt);
    const float c_log2 = a.scale * kLog2e;
    // Unmasked, every item has the same work and the persistent grid keeps
    // the CUs of an XCD in step; with segment IDs items differ (up to 8x on
    // packed clips) and one workgroup per item lets the dispatcher balance them.
    const int64_t pg = persistent_workgroups();
    const int grid = SEG ? n_wg : (int)std::min<int64_t>(n_wg64, pg);
    // Work stealing and split items need the persistent grid (a multiple of
    // 8) with more than one round, at most one record per workgroup, and a
    // long launch or a ragged last round (a short launch of whole rounds runs
    // the plain kernel).
    const bool steal = !SEG && ws != nullptr && n_wg64 > pg && pg <= kTailRecords &&
                       tail_max_r(n_wg, grid, kLongRounds) > 0;
    const auto args = std::make_tuple(reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const __bf16*>(a.k),
                                      reinterpret_cast<const __bf16*>(a.v), a.seg_q, a.seg_kv,
                                      reinterpret_cast<__bf16*>(a.out), a.lse, a.S, a.H, c_log2, n_qblk, n_kvt,
                                      n_wg, rope, steal ? ws->recs : nullptr, steal ? ws->ctr : nullptr);
    if (!steal) {
        std::apply([&](auto... x) {
            hipLaunchKernelGGL((attn_fwd_kernel<D, SEG, ROPE, false>), dim3(grid), dim3(kThreads), lds, stream, x...);
        }, args);
        return hipGetLastError();
    }
    if constexpr (!SEG) {
        hipLaunchKernelGGL(attn_fwd_ctr_reset_kernel, dim3(1), dim3(64), 0, stream, ws->ctr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        std::apply([&](auto... x) {
            hipLaunchKernelGGL((attn_fwd_kernel<D, false, ROPE, true>), dim3(grid), dim3(kThreads), lds, stream, x...);
        }, args);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_combine<D, false>(a, ws->recs, nullptr, n_qblk, n_wg, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

template <int D, bool ROPE>
hipError_t launch_sched_t(const AttnArgs& a, const Rope3DDev& rope, void* workspace, hipStream_t stream) {
    const int n_qblk = (a.S + kBq - 1) / kBq;
    const int n_kvt = (a.S + kBk - 1) / kBk;
    const int64_t n_items64 = (int64_t)a.B * a.H * n_qblk;
    const FwdWs ws = fwd_ws_layout(workspace, a.B, n_kvt, n_qblk);
    const int64_t n_all = (int64_t)a.B * n_kvt;
    hipLaunchKernelGGL(attn_fwd_tilesum_kernel, dim3((unsigned)((n_all + 15) / 16)), dim3(256), 0, stream,
                       a.seg_kv, a.S, n_kvt, n_all, ws.tsum, ws.ctr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_fwd_count_kernel, dim3((unsigned)((int64_t)a.B * n_qblk)), dim3(kBq), 0, stream,
                       a.seg_q, ws.tsum, a.S, n_qblk, n_kvt, ws.cnt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_fwd_rank_kernel, dim3((unsigned)a.B), dim3(kFwdRankThreads),
                       (size_t)n_qblk * sizeof(int), stream, ws.cnt, ws.ord, n_qblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // A multiple of 8 (every XCD counter has workgroups), at most one per CU.
    const int64_t grid = std::min<int64_t>(persistent_workgroups(), (n_items64 + kXcds - 1) / kXcds * kXcds);
    // The pool needs more items than workgroups and at most one part record
    // per workgroup (with exactly whole rounds and a short launch it is empty).
    const bool split = grid <= kTailRecords && n_items64 > grid && pool_plan((int)n_items64, (int)grid).n_pool > 0;
    const auto args = std::make_tuple(reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const __bf16*>(a.k),
                                      reinterpret_cast<const __bf16*>(a.v), a.seg_q, a.seg_kv,
                                      reinterpret_cast<__bf16*>(a.out), a.lse, a.S, a.H, a.scale * kLog2e, n_qblk,
                                      n_kvt, (int)n_items64, ws, rope);
    const size_t lds = fwd_lds<D, true>(n_kvt);
    if (!split) {
        std::apply([&](auto... x) {
            hipLaunchKernelGGL((attn_fwd_sched_kernel<D, ROPE, false>), dim3((unsigned)grid), dim3(kThreads), lds,
                               stream, x...);
        }, args);
        return hipGetLastError();
    }
    std::apply([&](auto... x) {
        hipLaunchKernelGGL((attn_fwd_sched_kernel<D, ROPE, true>), dim3((unsigned)grid), dim3(kThreads), lds,
                           stream, x...);
    }, args);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine<D, true>(a, ws.recs, ws.ord, n_qblk, (int)n_items64, (int)grid, stream);
}

int64_t max_masked_seq() { return (int64_t)kMaxKvTiles * kBk; }

size_t attn_fwd_workspace_bytes(int64_t B, int64_t S) {
    const int64_t n_qblk = (S + kBq - 1) / kBq, n_kvt = (S + kBk - 1) / kBk;
    return 256 + fwd_ws_align((size_t)(B * n_kvt) * sizeof(int4)) + fwd_ws_align((size_t)(B * n_qblk) * sizeof(int)) +
           fwd_ws_align((size_t)(B * n_qblk) * sizeof(int)) + (size_t)kTailRecords * tail_record_floats<128>() * 4;
}

hipError_t launch_attn_fwd_sched(const AttnArgs& a, void* workspace, hipStream_t stream) {
    const Rope3DDev none{};
    if (a.seg_q == nullptr) {
        if (workspace == nullptr) return launch_attn_fwd(a, stream);
        const FwdWs ws = fwd_ws_layout(workspace, a.B, (a.S + kBk - 1) / kBk, (a.S + kBq - 1) / kBq);
        return a.D == 128 ? launch_t<128, false, false>(a, none, stream, &ws)
                          : launch_t<64, false, false>(a, none, stream, &ws);
    }
    return a.D == 128 ? launch_sched_t<128, false>(a, none, workspace, stream)
                      : launch_sched_t<64, false>(a, none, workspace, stream);
}

hipError_t launch_rope3d_attn_fwd_sched(const AttnArgs& a, const Rope3DDev& rope, void* workspace,
                                        hipStream_t stream) {
    if (a.seg_q == nullptr) {
        if (workspace == nullptr) return launch_rope3d_attn_fwd(a, rope, stream);
        const FwdWs ws = fwd_ws_layout(workspace, a.B, (a.S + kBk - 1) / kBk, (a.S + kBq - 1) / kBq);
        return a.D == 128 ? launch_t<128, false, true>(a, rope, stream, &ws)
                          : launch_t<64, false, true>(a, rope, stream, &ws);
    }
    return a.D == 128 ? launch_sched_t<128, true>(a, rope, workspace, stream)
                      : launch_sched_t<64, true>(a, rope, workspace, stream);
}
int64_t queries_per_workgroup() { return kBq; }

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    const bool seg = a.seg_q != nullptr;
    const Rope3DDev none{};
    if (a.D == 128)
        return seg ? launch_t<128, true, false>(a, none, stream) : launch_t<128, false, false>(a, none, stream);
    return seg ? launch_t<64, true, false>(a, none, stream) : launch_t<64, false, false>(a, none, stream);
}

hipError_t launch_rope3d_attn_fwd(const AttnArgs& a, const Rope3DDev& rope, hipStream_t stream) {
    const bool seg = a.seg_q != nullptr;
    if (a.D == 128)
        return seg ? launch_t<128, true, true>(a, rope, stream) : launch_t<128, false, true>(a, rope, stream);
    return seg ? launch_t<64, true, true>(a, rope, stream) : launch_t<64, false, true>(a, rope, stream);
}

}  // namespace vdx
