// natten_fwd_kernel.hip -- gfx950 forward of 3D neighbourhood (windowed)
// self-attention over a t x h x w token grid.
//
// What it computes: for every query token, softmax(scale * q K^T) V over the
// keys of its neighbourhood window, plus the natural-log log-sum-exp (vidax
// paper, arXiv:2609.18077: section 2 "3D RoPE, 3D VAEs, and flash attention"
// for the windowed-attention primitive of the neighbourhood-attention VAE
// decoder; Appendix A, Table 4, group 4, LTX-2.5 VAE decoder rows, for its
// 11 x 11 x 11 window).  Tokens are flattened (t, y, x), x fastest.  Along an
// axis of length n a window of odd size k covers k_eff = min(k, n) positions
// starting at clamp(c - k/2, 0, n - k_eff): it shifts inward at the border.
//
// Design (same machinery as the segment-masked kernel):
//   * one workgroup = 8 wave64s (two per SIMD, two ping-pong groups) and a
//     BT x (8 / BT) x 32 (t, y, x) brick of queries, BT in {1, 2, 4, 8}
//     chosen per call (brick_frames): the shape whose window union holds the
//     fewest key rows per query row -- 4 x 2 for 11^3 windows (14 x 12 key
//     rows against 11 x 18 for 1 x 8), 1 x 8 for single frames or 1-frame t
//     windows; wave w owns the BT x (8 / BT) x 4 patch of the brick at x
//     offset 4w (lane lr the query (lr / (4 BY), (lr / 4) % BY, lr % 4) of it),
//     so a wave's 32 queries span only 4 columns and their x windows at most
//     3 + kw_eff <= 16 keys;
//   * the workgroup walks the key rows (t', y') in the union of its queries'
//     windows -- t' in [start(t0), start(t0 + BT - 1) + kt_eff), y' in
//     [start(y0), start(y0 + BY - 1) + kh_eff) -- two rows per step: a ring slot
//     holds two rows of 48 consecutive x positions from X0 (the brick's first
//     window start, rounded down to 4), which cover the x windows of all 32
//     brick columns;
//   * each wave multiplies one 32-key block per step: the 16 keys of each of
//     the step's two rows that hold its queries' x windows (so kw_eff <= 13),
//     i.e. 8 K Q^T + 8 P V MFMAs per step at D = 128, of which about half
//     the pairs lie in the windows (11 of 16 keys in x); a block of 32 keys
//     of one row for a 16-column patch kept a third;
//   * window tests: key (t', y', x') is valid for a query iff t', y' and x'
//     lie in its windows.  The x test is fixed for the item, so the K Q^T
//     chain starts from a per-lane bias of 0 / -inf instead of zero and
//     out-of-window keys score -inf with no per-step work; the t and y tests
//     are two per step (one per key row), applied to the row maxima and to
//     the exponent's offset, so an out-of-window row gets probability 0;
//     the online softmax is otherwise the segment kernel's;
//   * copies, operand prefetch, ping-pong schedule and epilogue follow the
//     segment-masked kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "attn_common.h"
#include "attn_fwd_launch.h"

namespace vdx {
namespace {

// k-th of n positions counted from the middle outward (a permutation of
// 0 .. n-1): middle first, then alternately one step further down and up.
__device__ __forceinline__ int center_out(int k, int n) {
    if ((n & 1) == 0) return (k & 1) ? n / 2 + k / 2 : n / 2 - 1 - k / 2;
    return (k & 1) ? n / 2 - (k + 1) / 2 : n / 2 + k / 2;
}

// First window position along an axis of length n for coordinate c.
__device__ __forceinline__ int win_start(int c, int k, int n) {
    const int keff = min(k, n);
    return min(max(c - k / 2, 0), n - keff);
}

constexpr int kBrickRows = 8;  // query (t, y) rows per workgroup: BT frames x 8 / BT rows
constexpr int kBrickX = 32;    // query columns per workgroup
constexpr int kPatchX = 4;     // query columns per wave
constexpr int kRowKeys = 48;   // keys of one key row held in LDS
constexpr int kBlockKeys = 16; // keys of one row a wave multiplies
// MFMA operands in flight (the segment kernel keeps 4; here 3 timed about 1%
// faster and 5 or 6 no better).
constexpr int kNatPrefetch = 3;

// Frames per brick, BT in {1, 2, 4, 8} (the brick is BT x 8/BT x 32 queries):
// the shape whose interior window union, min(BT + kt - 1, NT) frames x
// min(8/BT + kh - 1, NH) rows, is smallest per query row of the brick; on a
// tie the one with more frames (its union shrinks more where windows clip at
// the t borders).
int brick_frames(int NT, int NH, int KT, int KH) {
    const int64_t kt = std::min(KT, NT), kh = std::min(KH, NH);
    int best = 1;
    int64_t best_rows = 0, best_q = 1;
    for (int bt = 1; bt <= kBrickRows; bt *= 2) {
        const int64_t by = kBrickRows / bt;
        const int64_t rows = std::min<int64_t>(bt + kt - 1, NT) * std::min<int64_t>(by + kh - 1, NH);
        const int64_t q = std::min<int64_t>(bt, NT) * std::min<int64_t>(by, NH);
        if (bt == 1 || rows * best_q <= best_rows * q) {
            best = bt;
            best_rows = rows;
            best_q = q;
        }
    }
    return best;
}

// LDS ring of the neighbourhood kernel: kSlots slots of K and of V, each two
// key rows of kRowKeys keys (slot rows 0..47 and 48..95), with the K and V
// swizzles of the segment kernel applied to the slot row.
template <int D>
struct NTile {
    static constexpr int kChunks = D / 8;
    static constexpr int kRowBytes = D * 2;
    static constexpr int kSlotRows = 2 * kRowKeys;
    static constexpr int kSlotBytes = kSlotRows * kRowBytes;
    static constexpr int kKRegion = 0;
    static constexpr int kVRegion = kSlots * kSlotBytes;
    static constexpr int kRingBytes = 2 * kSlots * kSlotBytes;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static constexpr int kLoadsPerWave = kSlotBytes / 1024 / kDmaWaves;
    static constexpr int kSteps = D / 16;
    static constexpr int kDBlocks = D / 32;
    // Waves 0-1 of a copying group fill the slot's first row, waves 2-3 its
    // second: no load straddles the two rows.
    static_assert(kLoadsPerWave * 2 * kRowsPerLoad == kRowKeys, "one row per wave pair");
    static_assert(kSlotBytes % 1024 == 0, "slot bases must keep the swizzle bits free");
    static_assert(kRingBytes <= (int)kLdsBytes, "ring exceeds the LDS");
};

template <int D>
struct Nat {
    using T = NTile<D>;
    static constexpr int kQk = T::kSteps;         // K Q^T MFMAs per step (one 32-key block)
    static constexpr int kPv = 2 * T::kDBlocks;   // P V MFMAs per step (its two 16-key rows)
    static constexpr int kRing = kNatPrefetch + 2;

    char* smem;
    const __bf16* kp;  // K of (b, h), token 0
    const __bf16* vp;
    int64_t tok_stride;
    int NH, NW, lane, lr, g, w4;
    float c_log2;
    // workgroup key rows: t' in [ts, ts + nt), y' in [ylo, ylo + ny); n_rows of them
    int ts, nt, ylo, ny, n_rows, x0k, kt, kh, kw;
    int wrap_add;       // token step from the last row of a frame's y range to the first of the next
    int kx, vx;         // operand bases of this wave's block (16 keys of each row of a slot)
    f32x16 xbias;       // 0 where block key 8g + (r & 7) of a row lies in this lane's x window, else -inf
    bool row0, row1;    // the step's two key rows lie in this lane's t and y windows
    int ts_q, ys_q;     // this lane's query t- and y-window starts
    uint32_t dmo[T::kLoadsPerWave];
    bf16x8 qreg[T::kSteps];
    f32x16 oacc[T::kDBlocks];
    f32x16 sacc;
    bf16x8 pb[2];
    bf16x8 ops[kRing];
    uint32_t vb_next, kb_next;
    float m_run, l_run;

    __device__ __forceinline__ static int slot_base(int n) {
        int o = (n % kSlots) * T::kSlotBytes;
        asm volatile("" : "+s"(o));
        return o;
    }
    __device__ __forceinline__ uint32_t vbase(int n) const {
        return lds_addr(smem) + T::kVRegion + slot_base(n) + vx;
    }
    __device__ __forceinline__ uint32_t kbase(int n) const {
        return lds_addr(smem) + T::kKRegion + slot_base(n) + kx;
    }

    // ---- tile copies --------------------------------------------------------
    // Step a holds key rows 2a and 2a+1 of the walk (row r is (ts + r / ny,
    // ylo + r % ny)); a missing last row repeats row 2a and is masked.  Group 0
    // copies K of step n+2 in its MFMA phase of iteration n, group 1 V of step
    // n+1 (the ring discipline of the segment-masked kernel).  tok is the
    // token (in the head) of the first staged key of the row this wave copies.
    struct Copy {
        const __bf16* src;
        char* dst;
        int cnt;
        bool spread;
    };
    template <int G>
    __device__ __forceinline__ void plan(Copy& c, int a, int tok, int n_act) {
        c.cnt = 0;
        c.spread = false;
        if (a < n_act) {
            c.src = (G ? vp : kp) + (int64_t)tok * tok_stride;
            c.dst = smem + (G ? T::kVRegion : T::kKRegion) + slot_base(a) + w4 * T::kLoadsPerWave * 1024;
            c.spread = true;
            c.cnt = T::kLoadsPerWave;
        }
    }
    // Wait for the copies issued before this phase's (c: 0 or kLoadsPerWave).
    __device__ __forceinline__ static void wait_own(int c) {
        if (c != 0)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::kLoadsPerWave) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

    // ---- MFMA phase: K Q^T of step n, then P V of step n-1 --------------------
    // K Q^T MFMA i: k-step i of the block (block key m < 16 from the step's
    // first row, m >= 16 from its second).  P V MFMA j: kst = j / kDBlocks
    // names the row (its 16 keys are one k-step), d-block j % kDBlocks.
    template <bool QK, int I>
    __device__ __forceinline__ bf16x8 operand(uint32_t vb, uint32_t kb) const {
        if constexpr (QK && I < kQk) {
            return *reinterpret_cast<const bf16x8*>(lds_ptr(kb ^ (I << 5)));
        } else {
            constexpr int j = QK ? I - kQk : I;
            constexpr int kst = j / T::kDBlocks, db = j % T::kDBlocks;
            const char* p = lds_ptr((vb ^ (db << 6)) + kst * kRowKeys * T::kRowBytes);
            return tr_read8(p, p + 4 * T::kRowBytes);
        }
    }
    template <bool QK, int I>
    __device__ __forceinline__ void mfma(const bf16x8& a) {
        if constexpr (QK && I < kQk) {
            if constexpr (I == 0)
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[0], xbias, 0, 0, 0);
            else
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[I], sacc, 0, 0, 0);
        } else {
            constexpr int j = QK ? I - kQk : I;
            constexpr int kst = j / T::kDBlocks, db = j % T::kDBlocks;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kst], oacc[db], 0, 0, 0);
        }
    }
    template <bool PV, bool QK>
    __device__ __forceinline__ void prefetch(int vstep, int kstep) {
        constexpr int NM = (QK ? kQk : 0) + (PV ? kPv : 0);
        vb_next = vbase(vstep);
        kb_next = kbase(kstep);
        static_for<0, kNatPrefetch>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i < NM) ops[i % kRing] = operand<QK, i>(vb_next, kb_next);
        });
    }
    template <bool PV, bool QK, bool PRE>
    __device__ __forceinline__ void mfma_phase(int vstep, int kstep, const Copy& cp) {
        constexpr int NM = (QK ? kQk : 0) + (PV ? kPv : 0);
        constexpr int PF = kNatPrefetch;
        __builtin_amdgcn_s_setprio(1);
        if constexpr (!PRE) prefetch<PV, QK>(vstep, kstep);
        const uint32_t vb = vb_next, kb = kb_next;
        static_for<0, NM>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i + PF < NM) ops[(i + PF) % kRing] = operand<QK, i + PF>(vb, kb);
            mfma<QK, i>(ops[i % kRing]);
            copy_step<i, NM>(cp);
            __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_s_setprio(0);
    }

    // ---- VALU phase --------------------------------------------------------------
    // Window tests of the step's key rows (t0k, y0k), (t1k, y1k) (no second
    // row: live1 false).  Accumulator register r holds block key
    // 16 (r >> 3) + 8 g + (r & 7): row r >> 3 of the step, key 8g + (r & 7)
    // of that row's 16.  The x test is in the scores already (the K Q^T chain
    // starts from xbias, so keys outside the lane's x window score -inf); a row
    // outside the lane's t or y window is left out of the maximum and given
    // -inf in the exponent, so its probabilities are exactly 0.
    __device__ __forceinline__ void row_tests(int t0k, int y0k, int t1k, int y1k, bool live1) {
        row0 = (unsigned)(y0k - ys_q) < (unsigned)kh && (unsigned)(t0k - ts_q) < (unsigned)kt;
        row1 = live1 && (unsigned)(y1k - ys_q) < (unsigned)kh && (unsigned)(t1k - ts_q) < (unsigned)kt;
    }
    // Online softmax of the step's 16 scores per lane with the lazily moved
    // reference of the segment-masked kernel (P <= 2^kLazyLog2).
    __device__ __forceinline__ void softmax() {
        float mx0 = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
        float mx1 = fmaxf(fmaxf(sacc[8], sacc[9]), sacc[10]);
#pragma unroll
        for (int r = 3; r < 7; r += 2) {
            mx0 = fmaxf(fmaxf(mx0, sacc[r]), sacc[r + 1]);
            mx1 = fmaxf(fmaxf(mx1, sacc[8 + r]), sacc[8 + r + 1]);
        }
        mx0 = row0 ? fmaxf(mx0, sacc[7]) : -INFINITY;
        mx1 = row1 ? fmaxf(mx1, sacc[15]) : -INFINITY;
        const float mx = pair_max(fmaxf(mx0, mx1)) * c_log2;
        const bool move = mx > m_run + kLazyLog2;
        if (__ballot(move) != 0ull) {
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
        const float a0 = row0 ? -msub : -INFINITY, a1 = row1 ? -msub : -INFINITY;
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c_log2, r < 8 ? a0 : a1));
            ls[r & 3] += p;
            pb[r >> 3][r & 7] = (__bf16)p;
        }
        l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(l_run), "v"(m_run));
    }
};

// A key row of the workgroup's walk: ry = y' - ylo, rt = t' - ts, and tok =
// the token of its first staged key.  step() moves to the next row (y'
// fastest) with integer selects only: stay = -1 while the row stays in its
// frame, 0 when it wraps to the first row of the next frame.
struct Walk {
    int ry, rt, tok;
    __device__ __forceinline__ void step(int ny, int NW, int wrap_add) {
        const int y1 = ry + 1;
        const int stay = (y1 - ny) >> 31;
        ry = y1 & stay;
        rt += 1 + stay;
        tok += (NW & stay) | (wrap_add & ~stay);
    }
};

// The token of the row a wave copies: the step's second row (b) when it has
// one and the wave copies second rows, else its first (a); wave-uniform.
__device__ __forceinline__ int pick_row(bool use_b, int a, int b) {
    return __builtin_amdgcn_readfirstlane(a ^ ((a ^ b) & -(int)use_b));
}

// Ping-pong schedule of group G (see the segment-masked kernel): local
// iteration n = MFMA phase (K Q^T of step n, P V of step n-1) at global phase
// 2n + G, then the VALU phase (masks and softmax of step n) at 2n + 1 + G.
// mrow walks the first row of the step being masked; crow the first row of
// the step being planned, of which waves 0-1 of the group copy the first row
// and waves 2-3 the second (the first again when the step has one row).
template <int G, int D>
__device__ __forceinline__ void natten_loop(Nat<D>& A, int n_act, const Walk& w0) {
    typename Nat<D>::Copy cp;
    const bool second = (A.w4 >> 1) != 0;
    Walk mw = w0, cw = w0;
    // plan the copy of step a (cw at its first row), then move cw two rows on
    auto plan_step = [&](int a) {
        Walk w1 = cw;
        w1.step(A.ny, A.NW, A.wrap_add);
        A.template plan<G>(cp, a, pick_row(second && 2 * a + 1 < A.n_rows, cw.tok, w1.tok), n_act);
        cw = w1;
        cw.step(A.ny, A.NW, A.wrap_add);
    };
    auto valu_phase = [&](int n) {
        Walk m1 = mw;
        m1.step(A.ny, A.NW, A.wrap_add);
        A.row_tests(A.ts + mw.rt, A.ylo + mw.ry, A.ts + m1.rt, A.ylo + m1.ry, 2 * n + 1 < A.n_rows);
        mw = m1;
        mw.step(A.ny, A.NW, A.wrap_add);
        A.softmax();
        plan_step(n + 3 - G);
        A.template prefetch<true, true>(n, n + 1);
        barrier();
    };
    for (int i = 0; i < 2 * (2 - G); ++i) cw.step(A.ny, A.NW, A.wrap_add);  // first planned step: 2 - G
    plan_step(2 - G);
    A.template prefetch<false, true>(0, 0);
    if (G == 1) barrier();  // group 1 idles in global phase 0
    A.template mfma_phase<false, true, true>(0, 0, cp);
    A.wait_own(cp.cnt);
    barrier();
    valu_phase(0);
    for (int n = 1; n < n_act; ++n) {
        const int c = cp.cnt;
        A.template mfma_phase<true, true, true>(n - 1, n, cp);
        A.wait_own(c);
        barrier();
        valu_phase(n);
    }
    {
        const int c = cp.cnt;
        A.template mfma_phase<true, false, false>(n_act - 1, 0, cp);
        A.wait_own(c);
        barrier();
    }
    if (G == 0) barrier();  // group 0 idles in the last global phase
}

template <int D>
__global__ __launch_bounds__(kThreads) void natten_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ out, float* __restrict__ lse, int NT, int NH, int NW, int H, int KT, int KH,
    int KW, float c_log2, int bft, int nbt, int nby, int nbx, int n_wg) {
    using T = NTile<D>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    // XCD-contiguous renumbering: consecutive bricks of one head share an L2.
    // Within a head the bricks go longest first: a brick walks fewer key rows
    // the nearer it lies to a t or y border (windows clipped there, or a
    // partial brick), so the frame-brick index runs from the middle outward
    // (slowest), then the row-brick index from the middle outward, and the
    // CUs of an XCD, dealt the bricks in that order, finish together.
    const int w = blockIdx.x;
    const int per = n_wg / kXcds, rem = n_wg % kXcds;
    const int xcd = w % kXcds;
    const int lid = xcd * per + min(xcd, rem) + w / kXcds;
    const int bx = lid % nbx;
    const int by = center_out((lid / nbx) % nby, nby);
    const int bt = center_out((lid / (nbx * nby)) % nbt, nbt);
    const int bh = lid / (nbx * nby * nbt);
    const int h = bh % H;
    const int b = bh / H;
    const int S = NT * NH * NW;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 31, g = lane >> 5;
    const int grp = wave >> 2;
    // bft frames x bfy rows x 32 columns; wave w takes columns 4w .. 4w + 3 of
    // every (t, y) row of the brick, lane lr the query (lr / (4 bfy),
    // (lr / 4) % bfy, lr % 4) of that patch
    const int bfy = kBrickRows / bft;
    const int t0 = bt * bft, y0 = by * bfy, x0 = bx * kBrickX;
    const int tq = t0 + lr / (kPatchX * bfy);
    const int yq = y0 + (lr / kPatchX) % bfy;
    const int xq = x0 + kPatchX * wave + (lr % kPatchX);
    const bool active = tq < NT && yq < NH && xq < NW;
    const int qi = (min(tq, NT - 1) * NH + min(yq, NH - 1)) * NW + min(xq, NW - 1);

    Nat<D> A;
    A.smem = smem;
    A.tok_stride = (int64_t)H * D;
    A.kp = k + (int64_t)b * S * A.tok_stride + (int64_t)h * D;
    A.vp = v + (int64_t)b * S * A.tok_stride + (int64_t)h * D;
    A.NH = NH;
    A.NW = NW;
    A.lane = lane;
    A.lr = lr;
    A.g = g;
    A.w4 = wave & 3;
    A.c_log2 = c_log2;
    A.kh = min(KH, NH);
    A.kw = min(KW, NW);
    A.kt = min(KT, NT);

    // ---- workgroup key rows and the x range of the rows ------------------------
    A.ts = win_start(t0, KT, NT);
    A.nt = win_start(min(t0 + bft - 1, NT - 1), KT, NT) + A.kt - A.ts;
    A.ylo = win_start(y0, KH, NH);
    A.ny = win_start(min(y0 + bfy - 1, NH - 1), KH, NH) + A.kh - A.ylo;
    A.n_rows = A.nt * A.ny;
    A.x0k = win_start(x0, KW, NW) & ~3;
    const int n_act = (A.n_rows + 1) / 2;  // steps of two key rows
    A.wrap_add = NW * (NH - A.ny + 1);
    const Walk w0{0, 0, (A.ts * NH + A.ylo) * NW + A.x0k};
    // this wave's 16-key block inside a row (from its first column's window
    // start), and the lane's windows
    const int xw = min(x0 + kPatchX * wave, NW - 1);
    const int boff = min(win_start(xw, KW, NW) - A.x0k, kRowKeys - kBlockKeys);
    A.ts_q = win_start(min(tq, NT - 1), KT, NT);
    A.ys_q = win_start(min(yq, NH - 1), KH, NH);
    const int xs_q = win_start(min(xq, NW - 1), KW, NW);
    {
        const int xrel = A.x0k + boff + 8 * g - xs_q;  // block key 8g + e is x offset xrel + e
#pragma unroll
        for (int r = 0; r < 16; ++r) A.xbias[r] = (unsigned)(xrel + (r & 7)) < (unsigned)A.kw ? 0.f : -INFINITY;
    }
    if (!active) A.ys_q = -(1 << 30);  // no key row passes the row test

    // ---- Q slice -> registers ----------------------------------------------------
    {
        const __bf16* qrow = q + ((int64_t)b * S + qi) * A.tok_stride + (int64_t)h * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks)
            A.qreg[ks] = active ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16) : bf16x8{};
    }
    // ---- per-lane LDS offsets (operand rows shifted by the block offset) -------
    {
        // K Q^T: accumulator row lr holds block key m = swap23(lr), i.e. key
        // m & 15 of the block in the step's row m >> 4
        const int m = swap23(lr);
        const int krow = (m >> 4) * kRowKeys + boff + (m & 15);
        A.kx = krow * T::kRowBytes + ((g ^ k_swz<D>(krow)) << 4);
        // v_swz looks at the slot row mod 4 only, and kRowKeys is a multiple
        // of 4: one base serves both rows.
        const int qg = lane >> 4, j = lane & 15;
        const int key = boff + 8 * (qg >> 1) + (j >> 2);
        const int vsw = v_swz<D>(key);
        A.vx = key * T::kRowBytes + 32 * ((qg & 1) ^ vsw) + 16 * ((j & 3) >> 1) + 8 * (j & 1);
        // Tile copies: load jj of this wave covers slot rows kRowsPerLoad*i ..
        // (i = w4 * L + jj); a lane lands at LDS position pos of its slot row
        // and fetches the chunk stored there (K layout for group 0, V layout
        // for group 1) from key r % kRowKeys of its key row.  Keys past the
        // grid row read the row's last key instead (the x masks exclude them);
        // every row of the item starts at x0k, so the clamp is folded in here
        // once and every copy is spread between MFMAs.
#pragma unroll
        for (int jj = 0; jj < T::kLoadsPerWave; ++jj) {
            const int i = A.w4 * T::kLoadsPerWave + jj;
            const int r = T::kRowsPerLoad * i + lane / T::kChunks;  // slot row
            const int pos = lane % T::kChunks;
            const int c = grp ? 2 * ((pos >> 1) ^ v_swz<D>(r)) + (pos & 1) : (pos ^ k_swz<D>(r));
            const int xk = min(A.x0k + r % kRowKeys, NW - 1) - A.x0k;  // key within the row
            A.dmo[jj] = 2u * (uint32_t)(xk * (int)A.tok_stride + c * 8);
        }
    }
#pragma unroll
    for (int i = 0; i < T::kDBlocks; ++i) A.oacc[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < 2; ++i) A.pb[i] = bf16x8{};
    A.m_run = -INFINITY;
    A.l_run = 0.f;

    // ---- prologue: K of steps 0 and 1 (group 0), V of step 0 (group 1) ---------
    {
        typename Nat<D>::Copy c;
        const bool second = (A.w4 >> 1) != 0;
        Walk w = w0;
        for (int a = 0; a < 2 - grp; ++a) {
            Walk w1 = w;
            w1.step(A.ny, A.NW, A.wrap_add);
            const int tok = pick_row(second && 2 * a + 1 < A.n_rows, w.tok, w1.tok);
            if (grp == 0)
                A.template plan<0>(c, a, tok, n_act);
            else
                A.template plan<1>(c, a, tok, n_act);
            if (c.spread) {
#pragma unroll
                for (int j = 0; j < T::kLoadsPerWave; ++j) dma16(c.src, A.dmo[j], c.dst + j * 1024);
            }
            w = w1;
            w.step(A.ny, A.NW, A.wrap_add);
        }
    }
    wait_vm(0);
    barrier();
    asm volatile("" ::"v"(A.qreg[0]), "v"(A.qreg[T::kSteps - 1]));

    if (grp == 0)
        natten_loop<0>(A, n_act, w0);
    else
        natten_loop<1>(A, n_act, w0);

    // ---- epilogue -----------------------------------------------------------------
    const float l_tot = pair_sum(A.l_run);
    if (active) {
        __bf16* orow = out + ((int64_t)b * S + qi) * A.tok_stride + (int64_t)h * D;
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
        if (g == 0) lse[((int64_t)b * H + h) * S + qi] = (A.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

template <int D>
hipError_t launch_t(const NattenArgs& a, hipStream_t stream) {
    using T = NTile<D>;
    const int bft = brick_frames(a.NT, a.NH, a.KT, a.KH), bfy = kBrickRows / bft;
    const int nbt = (a.NT + bft - 1) / bft;
    const int nby = (a.NH + bfy - 1) / bfy;
    const int nbx = (a.NW + kBrickX - 1) / kBrickX;
    const int n_wg = a.B * a.H * nbt * nby * nbx;
    const float c_log2 = a.scale * kLog2e;
    hipLaunchKernelGGL((natten_fwd_kernel<D>), dim3(n_wg), dim3(kThreads), (size_t)T::kRingBytes, stream,
                       reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const __bf16*>(a.k),
                       reinterpret_cast<const __bf16*>(a.v), reinterpret_cast<__bf16*>(a.out), a.lse,
                       a.NT, a.NH, a.NW, a.H, a.KT, a.KH, a.KW, c_log2, bft, nbt, nby, nbx, n_wg);
    return hipGetLastError();
}

}  // namespace

int64_t natten_workgroups(const NattenArgs& a) {
    const int bft = brick_frames(a.NT, a.NH, a.KT, a.KH), bfy = kBrickRows / bft;
    return (int64_t)a.B * a.H * ((a.NT + bft - 1) / bft) * ((a.NH + bfy - 1) / bfy) *
           ((a.NW + kBrickX - 1) / kBrickX);
}

hipError_t launch_natten_fwd(const NattenArgs& a, hipStream_t stream) {
    return a.D == 128 ? launch_t<128>(a, stream) : launch_t<64>(a, stream);
}

}  // namespace vdx
