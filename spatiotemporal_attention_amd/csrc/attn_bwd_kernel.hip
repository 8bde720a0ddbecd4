// attn_bwd_kernel.hip -- gfx950 backward of segment-masked, non-causal
// softmax attention: dq, dk, dv from q, k, v, out, lse and dout.
//
// What it computes (vidax paper, arXiv:2609.18077: section 5 "Conclusions &
// Future Work" names training and fine-tuning, which need this gradient; the
// forward and its segment rule are those of section 2 and Appendix A,
// Table 4, groups 1 and 2).  With P_ij = exp(scale q_i.k_j - lse_i) over the
// valid pairs (equal, nonzero segment IDs; 0 elsewhere):
//   dv_j = sum_i P_ij dout_i
//   dP_ij = dout_i . v_j,  delta_i = sum_j P_ij dP_ij = dout_i . out_i
//   dS_ij = P_ij (dP_ij - delta_i)
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i
// P is recomputed from the forward's log-sum-exp, so nothing of size S x S
// is ever stored.
//
// Three kernels (five with segment IDs), all deterministic (no atomics):
//   * prep: delta_i = dout_i . out_i in fp32 and lse2_i = lse_i log2(e)
//     (+inf for rows without a valid key, and for the padding rows up to the
//     next multiple of 64, so that their P is exactly 0) into a workspace;
//   * dK/dV (key-major): a workgroup holds 128 keys, 32 per wave, whose K and
//     V slices stay in registers as MFMA B operands; it sweeps the 64-query
//     tiles that can hold a valid pair: S = Q K^T and dP = dO V^T (lanes own
//     key columns), P and dS on the VALU, then dV^T += dO^T P and
//     dK^T += Q^T dS with the fp32 P / dS registers reused as bf16 B operands
//     (queries inside a 32-row block are permuted so that the accumulator
//     rows line up with the operand's contraction index);
//   * dQ (query-major): a workgroup holds 128 queries, Q and dO slices in
//     registers; it sweeps the key tiles: S^T = K Q^T, dP^T = V dO^T, dS^T on
//     the VALU, dQ^T += K^T dS^T.
//   * with segment IDs, a count kernel classifies every row block of both
//     sweeps as its sweep will (its active-tile count is its cost) and a rank
//     kernel orders each batch's blocks longest-first, so that the CUs of an
//     XCD, which take a head's blocks in that order, finish together; the
//     order of the blocks changes no result.
// Both sweeps stage their 64-row tiles in LDS by direct global->LDS DMA into
// a ring.  One XOR swizzle of 16-byte chunks serves both operand reads of a
// tile -- row reads (ds_read_b128, A operand of Q K^T-type products) and
// transposed reads (ds_read_b64_tr_b16, A operand of X^T Y products) -- with
// no bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "attn_common.h"
#include "attn_fwd_launch.h"

namespace vdx {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;  // keys (dK/dV) or queries (dQ) per workgroup
// Capacity of the on-chip active-tile list; with the dK/dV sweep's four-stage
// ring at D = 128 it fills 163,232 of the 160 KiB of LDS a workgroup may take
// (checked at compile time with the LDS budgets below).
constexpr int kBwdMaxTiles = 14000;
constexpr int kPad = 64;                  // workspace rows are padded to this multiple
#ifndef VDX_BWD_PREFETCH
#define VDX_BWD_PREFETCH 4
#endif
constexpr int kPf = VDX_BWD_PREFETCH;     // MFMA operands in flight

template <int D>
struct BTile {
    static constexpr int kChunks = D / 8;  // 16-byte chunks per row
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kTileBytes = 64 * kRowBytes;
    static constexpr int kSteps = D / 16;   // MFMA k-steps over D
    static constexpr int kDBlocks = D / 32;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;
    static constexpr int kLoads = kTileBytes / 1024 / kBwdWaves;  // DMAs per wave per tile
    // One ring stage: two 64-row tiles (Q, dO or K, V), then 64 fp32 lse2,
    // 64 fp32 delta and 64 int32 segment IDs.
    static constexpr int kA = 0;
    static constexpr int kB = kTileBytes;
    static constexpr int kVec0 = 2 * kTileBytes;
    static constexpr int kVec1 = kVec0 + 256;
    static constexpr int kSeg = kVec1 + 256;
    static constexpr int kStage = (kSeg + 256 + 1023) & ~1023;
    static_assert(kLoads >= 1, "tile too small for the workgroup");
};

// 16-byte chunk c of tile row r sits at chunk position c ^ u_swz(r).  The
// value depends on r & 15 only; it is a bijection on every 16 rows (row
// reads: 16 lanes fetch 16 different rows' chunk c) and differs in its upper
// bits across rows {4a..4a+3} (D = 128) or {4a, 4a+2} (D = 64), which
// spreads the 4 rows x 64 bytes of a transposed read over all banks.
template <int D>
__device__ __forceinline__ int u_swz(int r) {
    if constexpr (D == 128)
        return ((r & 3) << 2) | ((r >> 2) & 3);
    else
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ void wait_vm_upto(int n) {
    // n is one of the copy counts a wave issues per tile (<= 12).
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    }
}

// Per-lane LDS offsets (within a 64-row tile) of the two operand reads and
// the DMA source offsets of this wave's share of a tile copy.
template <int D>
struct Lanes {
    using T = BTile<D>;
    // Row read, A operand of a 32x32x16 MFMA over rows 32*blk .. +31 and
    // columns 16*ks .. +15: lane (lr, g) takes row swap23(lr), chunk 2ks + g,
    // at (rx ^ (ks << 5)) + 32 * blk * kRowBytes.
    int rx;
    // Transposed read, A operand over columns 32*db .. +31 (m) and rows
    // 16*kst .. +15 (k): two ds_read_b64_tr_b16 at (tx0 / tx1 ^ (db << 6)) +
    // 16 * kst * kRowBytes; lane (q = lane / 16, j = lane % 16) points at row
    // 8(q >> 1) + (j >> 2) (+4) and columns 16(q & 1) + 4(j & 3) .. +3.
    int tx0, tx1;
    uint32_t dmo[T::kLoads];

    __device__ __forceinline__ void init(int wave, int lane, int64_t tok_stride) {
        const int lr = lane & 31, g = lane >> 5;
        const int sr = swap23(lr);
        rx = sr * T::kRowBytes + 16 * (g ^ u_swz<D>(sr));
        const int qg = lane >> 4, j = lane & 15;
        const int r0 = 8 * g + (j >> 2), r1 = r0 + 4;
        const int c0 = 2 * (qg & 1) + ((j & 3) >> 1);
        tx0 = r0 * T::kRowBytes + 16 * (c0 ^ u_swz<D>(r0)) + 8 * (j & 1);
        tx1 = r1 * T::kRowBytes + 16 * (c0 ^ u_swz<D>(r1)) + 8 * (j & 1);
        // DMA instruction i covers rows kRowsPerLoad*i ..; lane l lands at
        // chunk position l % kChunks of its row and fetches the chunk stored
        // there.
#pragma unroll
        for (int jj = 0; jj < T::kLoads; ++jj) {
            const int i = wave * T::kLoads + jj;
            const int r = T::kRowsPerLoad * i + lane / T::kChunks;
            const int c = (lane % T::kChunks) ^ u_swz<D>(r);
            dmo[jj] = 2u * (uint32_t)(r * (int)tok_stride + 8 * c);
        }
    }
    __device__ __forceinline__ static int dma_row(int wave, int jj, int lane) {
        return T::kRowsPerLoad * (wave * T::kLoads + jj) + lane / T::kChunks;
    }
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += a b with acc held in AGPRs (accumulation registers), for
// accumulators that only MFMAs touch until the epilogue: the register
// allocator then never moves them between register files.  The hazard
// recogniser does not look inside inline asm, so the wait states it would
// insert are explicit: a VALU write (including the v_accvgpr_mov the
// allocator may place to relocate acc between code paths) of an operand ->
// MFMA read needs 2, given by the s_nop 1 of every such MFMA (it mostly
// overlaps the wait for the busy matrix pipe), and 4 when NOP (a VALU
// instruction may have written b just before); accumulator_fence() supplies
// the ones between the last MFMA write and a VALU read of the result (an
// 8-pass XDL write needs 11; 20 are given).
template <bool NOP>
__device__ __forceinline__ void mfma32_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    if constexpr (NOP)
        asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void accumulator_fence() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
}

// acc (VGPRs, read by the VALU afterwards) = a b (+ acc unless FIRST), with b
// held in AGPRs: a K or V slice that only MFMAs read (written there once, by
// the VALU, before the sweep: NOP gives the first MFMAs their 4 wait states).
// accumulator_fence() must separate the last such MFMA from the first VALU
// read of acc.
template <bool FIRST, bool NOP>
__device__ __forceinline__ void mfma32_vacc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    if constexpr (FIRST && NOP)
        asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
    else if constexpr (FIRST)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}

// Workgroup id -> (row block, b*H + h), renumbered so that each XCD (own L2)
// runs consecutive row blocks of one head, which share the swept tiles.
__device__ __forceinline__ void wg_coords(int n_blk, int n_wg, int& blk, int& bh) {
    const int w = blockIdx.x;
    const int per = n_wg / kXcds, rem = n_wg % kXcds;
    const int xcd = w % kXcds;
    const int lid = xcd * per + min(xcd, rem) + w / kXcds;
    blk = lid % n_blk;
    bh = lid / n_blk;
}

// ---- prep: delta and lse2 ------------------------------------------------------
// Items walk the workspace order (b, h, i) with i fastest over S_pad rows, so
// the 4-byte results of a block's rows land in one contiguous run per array
// (walking the rows in [B, S, H] memory order instead put neighbouring stores
// S_pad * 4 bytes apart, each in a write burst of its own).  A row's out and
// dout (D bf16 each) are read by D/8 lanes, 16 bytes a lane.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(
    const __bf16* __restrict__ out, const __bf16* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ ws_lse2, float* __restrict__ ws_delta, int S, int H, int S_pad,
    int64_t n_items) {
    constexpr int L = D / 8;
    const int64_t stride = (int64_t)gridDim.x * (256 / L);
    const int part = threadIdx.x % L;
    for (int64_t it = (int64_t)blockIdx.x * (256 / L) + threadIdx.x / L; it < n_items; it += stride) {
        const int64_t i = it % S_pad, bh = it / S_pad;
        if (i < S) {
            const int64_t h = bh % H, b = bh / H;
            const int64_t row = (b * S + i) * H + h;
            const bf16x8 o = *reinterpret_cast<const bf16x8*>(out + row * D + 8 * part);
            const bf16x8 d = *reinterpret_cast<const bf16x8*>(dout + row * D + 8 * part);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)d[e], acc);
#pragma unroll
            for (int m = L / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
            if (part == 0) {
                const float l = lse[bh * S + i];
                ws_delta[it] = acc;
                ws_lse2[it] = (l == -INFINITY) ? INFINITY : l * kLog2e;
            }
        } else if (part == 0) {
            ws_delta[it] = 0.f;
            ws_lse2[it] = INFINITY;
        }
    }
}

// ---- dK / dV ---------------------------------------------------------------------
// Key-major sweep over the active 64-query tiles, each taken as two 32-query
// sub-tiles, software-pipelined inside each wave (one wave per SIMD: the K/V
// slices and the dK/dV accumulators take 192 AGPRs) so that its MFMAs and
// VALU work overlap.  Sub-iteration u:
//   step 1: dV^T += dO^T P and dK^T += Q^T dS of sub-tile u-1 (kNB MFMAs);
//   step 2: S = Q K^T and dP = dO V^T of sub-tile u+1 (kNA MFMAs);
// P and dS of sub-tile u are formed on the VALU between the MFMAs of both
// steps, two elements at a time, half in each step, so that neither step's
// MFMA slots run short of issue time.
// A tile iteration (two sub-iterations) reads tiles t-1, t and t+1 while
// t+2 lands, hence four ring slots and one barrier per tile.  Operands are
// fetched kPf MFMAs ahead through an 8-entry ring, across step and iteration
// boundaries (every tile read across the closing barrier is resident).  S/dP
// and the bf16 P/dS operands alternate between two register buffers (the
// loop is unrolled by a tile).
template <int D, bool SEG>
struct DkDv {
    using T = BTile<D>;
    static constexpr int kSlots = 4;
    static constexpr int kRing = 8;
    static constexpr int kNA = 2 * T::kSteps;    // S and dP MFMAs per sub-tile
    static constexpr int kNB = 4 * T::kDBlocks;  // dV and dK MFMAs per sub-tile
    static constexpr int kPairs = 8;             // softmax element pairs per lane and sub-tile
    static constexpr int kPairAhead = 3;         // lse2 / delta loads in flight
    // The pairs of a sub-tile are spread over two steps (D = 128): kPairsB in
    // the dV/dK step before its S/dP step, from MFMA slot kSlotB0 on (the
    // first slots give the MFMA results they read their wait states), the
    // rest in the S/dP step from slot kSlotA0 on, one every kSlotStep slots.
    // With D = 64 the steps have 8 slots and all pairs go to the S/dP step.
    // A pair's exponentials go one slot before the rest of its arithmetic
    // (kSplit), so that their latency passes behind an MFMA.
    static constexpr int kPairsB = kNB >= 16 ? 4 : 0;
    static constexpr int kSlotB0 = 4, kSlotA0 = kPairsB ? 1 : 0, kSlotStep = kPairsB ? 3 : 1;
    static constexpr int kSplit = kPairsB ? 1 : 0;
    static_assert(kNA % kRing == 0 && kNB % kRing == 0 && kPf <= kRing - 2, "operand ring");
    static_assert(kPairsB == 0 || kSlotB0 + kSlotStep * (kPairsB - 1) < kNB, "pairs of the dV/dK step");
    static_assert(kSlotA0 + kSlotStep * (kPairs - kPairsB - 1) < kNA, "pairs of the S/dP step");

    char* smem;
    Lanes<D> L;
    int g, myseg;
    float c_log2;
    bf16x8 kreg[T::kSteps], vreg[T::kSteps];        // AGPRs (B operands)
    f32x16 dkacc[T::kDBlocks], dvacc[T::kDBlocks];  // AGPRs (accumulators)
    f32x16 sc[2], pc[2];                            // S, dP of a sub-tile, by parity
    bf16x8 pb[2][2], dsb[2][2];                     // P, dS as bf16 B operands [parity][k-step]
    bf16x8 ring[kRing];
    float2 lpair[kPairAhead], dpair[kPairAhead];
    int2 spair[kPairAhead];
    float2 pexp;  // P of the pair between its two halves
    // Lane offsets of the operand reads within a stage: row reads of k-step
    // ks at rxk[ks], the two halves of the transposed reads of d-block db at
    // txk0[db] / txk1[db].
    uint32_t rxk[T::kSteps], txk0[T::kDBlocks], txk1[T::kDBlocks];

    __device__ __forceinline__ static uint32_t slot(int t) {
        int o = (t % kSlots) * T::kStage;
        asm volatile("" : "+s"(o));
        return (uint32_t)o;
    }

    // Per-lane LDS addresses of one ring stage, formed once per tile: every
    // operand read then adds only its region and row offset, as the read's
    // immediate offset.  The sums are pinned in VGPRs; left alone, the
    // compiler keeps the stage address in an SGPR and spends a VALU add on
    // every read.
    struct RowBases {
        uint32_t r[T::kSteps];
    };
    struct TrBases {
        uint32_t t0[T::kDBlocks], t1[T::kDBlocks];
    };
    __device__ __forceinline__ void init_bases() {
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) rxk[ks] = (uint32_t)(L.rx ^ (ks << 5));
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) {
            txk0[db] = (uint32_t)(L.tx0 ^ (db << 6));
            txk1[db] = (uint32_t)(L.tx1 ^ (db << 6));
        }
    }
    __device__ __forceinline__ RowBases rows(uint32_t st) const {
        RowBases b;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) {
            b.r[ks] = st + rxk[ks];
            asm volatile("" : "+v"(b.r[ks]));
        }
        return b;
    }
    __device__ __forceinline__ TrBases trs(uint32_t st) const {
        TrBases b;
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) {
            b.t0[db] = st + txk0[db];
            b.t1[db] = st + txk1[db];
            asm volatile("" : "+v"(b.t0[db]), "+v"(b.t1[db]));
        }
        return b;
    }
    // Address of this lane's first softmax pair rows in a stage (pair j of
    // half h is 4 (32h + 16(j/4) + 2(j%4)) bytes further).
    __device__ __forceinline__ uint32_t pair_base(uint32_t st) const {
        uint32_t b = st + 32u * (uint32_t)g;
        asm volatile("" : "+v"(b));
        return b;
    }

    // MFMA i of the S/dP step of a sub-tile (rows 32*h .. of the tile at st):
    // k-step i / 2, S (even i, Q rows) or dP (odd i, dO rows).
    template <int I>
    __device__ __forceinline__ bf16x8 op_a(const RowBases& rb, int h) const {
        return *reinterpret_cast<const bf16x8*>(
            lds_ptr(rb.r[I / 2] + ((I & 1) ? T::kB : T::kA) + h * 32 * T::kRowBytes));
    }
    // MFMA i of the dV/dK step of a sub-tile: query k-step 2h + i / (2
    // kDBlocks), d-block (i / 2) % kDBlocks, dV (even i, dO) or dK (odd, Q).
    template <int I>
    __device__ __forceinline__ bf16x8 op_b(const TrBases& tb, int h) const {
        constexpr int db = (I / 2) % T::kDBlocks;
        const uint32_t o = ((I & 1) ? T::kA : T::kB) + (2 * h + I / (2 * T::kDBlocks)) * 16 * T::kRowBytes;
        return tr_read8(lds_ptr(tb.t0[db] + o), lds_ptr(tb.t1[db] + o));
    }

    // Softmax pair j of a sub-tile: accumulator registers r = 2j and 2j+1,
    // queries row(j), row(j)+1 of the tile (sub-tile h covers rows 32h..).
    // pb: pair_base() of the stage.
    __device__ __forceinline__ void load_pair(uint32_t pb, int h, int j, bool partial) {
        const uint32_t o = 4 * (32 * h + 16 * (j / 4) + 2 * (j % 4));
        lpair[j % kPairAhead] = *reinterpret_cast<const float2*>(lds_ptr(pb + T::kVec0 + o));
        dpair[j % kPairAhead] = *reinterpret_cast<const float2*>(lds_ptr(pb + T::kVec1 + o));
        // With segment IDs the mask is applied to every tile, full ones
        // included (they pass it unchanged): a branch on the tile kind here
        // would split the register assignment of the pipelined loop.
        if (SEG) spair[j % kPairAhead] = *reinterpret_cast<const int2*>(lds_ptr(pb + T::kSeg + o));
        (void)partial;
    }
    // P = 2^(s c - lse2), dS = P (dP - delta) for pair J of the sub-tile in
    // buffer B, in two halves: the exponentials, then the masks, dS and the
    // bf16 operands.
    template <int B, int J>
    __device__ __forceinline__ void pair_exp() {
        constexpr int r = 2 * J;
        const float2 l = lpair[J % kPairAhead];
        pexp.x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[B][r], c_log2, -l.x));
        pexp.y = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[B][r + 1], c_log2, -l.y));
        asm volatile("" : "+v"(pexp.x), "+v"(pexp.y));
    }
    template <int B, int J>
    __device__ __forceinline__ void pair_form(bool partial) {
        constexpr int r = 2 * J, k = r / 8, e = r % 8;
        const float2 d = dpair[J % kPairAhead];
        float p0 = pexp.x, p1 = pexp.y;
        if (SEG) {
            const int2 s = spair[J % kPairAhead];
            p0 = (s.x == myseg && myseg != 0) ? p0 : 0.f;
            p1 = (s.y == myseg && myseg != 0) ? p1 : 0.f;
        }
        (void)partial;
        pb[B][k][e] = (__bf16)p0;
        pb[B][k][e + 1] = (__bf16)p1;
        dsb[B][k][e] = (__bf16)(p0 * (pc[B][r] - d.x));
        dsb[B][k][e + 1] = (__bf16)(p1 * (pc[B][r + 1] - d.y));
        // Keep the pair here, between the MFMAs it is meant to overlap: the
        // optimiser would otherwise sink it towards its consumer, the next
        // dV/dK step, behind this step's MFMAs.
        asm volatile("" : "+v"(pb[B][k]), "+v"(dsb[B][k]));
    }

    __device__ __forceinline__ void prefetch_a(const RowBases& ra, int h) {
        static_for<0, kPf>([&](auto ic) { ring[ic] = op_a<ic>(ra, h); });
    }
    __device__ __forceinline__ void prefetch_pairs(uint32_t pv, int h, bool partial) {
        static_for<0, kPairAhead>([&](auto jc) { load_pair(pv, h, jc, partial); });
    }

    // Softmax pair of MFMA slot I of a step whose pairs start at slot S0 with
    // pair J0, or -1.
    template <int I, int S0, int J0, int N>
    static constexpr int pair_at() {
        return (I >= S0 && (I - S0) % kSlotStep == 0 && (I - S0) / kSlotStep < N) ? J0 + (I - S0) / kSlotStep : -1;
    }
    // The pair work of MFMA slot I of a step whose pairs start at slot S0
    // with pair J0 (N of them, buffer PB).
    template <int PB, int I, int S0, int J0, int N>
    __device__ __forceinline__ void pairs_at(uint32_t pv, int hv, bool partial) {
        constexpr int je = pair_at<I, S0, J0, N>();
        if constexpr (je >= 0) pair_exp<PB, je>();
        if constexpr (I >= kSplit) {
            constexpr int jf = pair_at<I - kSplit, S0, J0, N>();
            if constexpr (jf >= 0) {
                pair_form<PB, jf>(partial);
                if constexpr (jf + kPairAhead < kPairs) load_pair(pv, hv, jf + kPairAhead, partial);
            }
        }
    }

    // Step 1: dV / dK of the sub-tile (stage bases tb, half h) whose P / dS
    // are in buffer B (operands prefetched).  NEXT_A: the last steps fetch the
    // first operands of the S/dP step of sub-tile (ra, ha).  PB >= 0: the
    // first kPairsB softmax pairs of buffer PB (sub-tile (pv, hv)) go between
    // the MFMAs.
    template <int B, bool NEXT_A, int PB>
    __device__ __forceinline__ void step_b(const TrBases& tb, int h, const RowBases& ra, int ha, uint32_t pv,
                                           int hv, bool partial) {
        static_for<0, kNB>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i + kPf < kNB)
                ring[(i + kPf) % kRing] = op_b<i + kPf>(tb, h);
            else if constexpr (NEXT_A)
                ring[(i + kPf) % kRing] = op_a<i + kPf - kNB>(ra, ha);
            const bf16x8& a = ring[i % kRing];
            constexpr int kst = i / (2 * T::kDBlocks), db = (i / 2) % T::kDBlocks;
            if constexpr (i & 1)
                mfma32_acc<(i < 2)>(dkacc[db], a, dsb[B][kst]);
            else
                mfma32_acc<(i < 2)>(dvacc[db], a, pb[B][kst]);
            if constexpr (PB >= 0) pairs_at<PB, i, kSlotB0, 0, kPairsB>(pv, hv, partial);
            __builtin_amdgcn_sched_barrier(0);
        });
        (void)pv;
        (void)hv;
        (void)partial;
    }
    // Step 2: S / dP of sub-tile (ra, ha) into buffer B ^ 1 (if A) with the
    // remaining softmax pairs of buffer B (sub-tile (tv / pv, hv))
    // interleaved; the last steps fetch the first dV/dK operands of sub-tile
    // (tv, hv).
    template <int B, bool A>
    __device__ __forceinline__ void step_a(const RowBases& ra, int ha, const TrBases& tv, uint32_t pv,
                                           int hv, bool partial) {
        if constexpr (A) {
            static_for<0, kNA>([&](auto ic) {
                constexpr int i = ic;
                if constexpr (i + kPf < kNA)
                    ring[(i + kPf) % kRing] = op_a<i + kPf>(ra, ha);
                else
                    ring[(i + kPf) % kRing] = op_b<i + kPf - kNA>(tv, hv);
                const bf16x8& a = ring[i % kRing];
                constexpr int ks = i / 2;
                if constexpr (i & 1)
                    mfma32_vacc<(ks == 0), false>(pc[B ^ 1], a, vreg[ks]);
                else
                    mfma32_vacc<(ks == 0), false>(sc[B ^ 1], a, kreg[ks]);
                pairs_at<B, i, kSlotA0, kPairsB, kPairs - kPairsB>(pv, hv, partial);
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            static_for<kPairsB, kPairs>([&](auto jc) {
                constexpr int j = jc;
                pair_exp<B, j>();
                pair_form<B, j>(partial);
                if constexpr (j + kPairAhead < kPairs) load_pair(pv, hv, j + kPairAhead, partial);
            });
            static_for<0, kPf>([&](auto ic) { ring[ic] = op_b<ic>(tv, hv); });
        }
    }
    // S / dP of the first sub-tile alone, into buffer 0.
    __device__ __forceinline__ void step_a_only(const RowBases& ra) {
        static_for<0, kNA>([&](auto ic) {
            constexpr int i = ic;
            if constexpr (i + kPf < kNA) ring[(i + kPf) % kRing] = op_a<i + kPf>(ra, 0);
            const bf16x8& a = ring[i % kRing];
            constexpr int ks = i / 2;
            if constexpr (i & 1)
                mfma32_vacc<(ks == 0), (i < 2)>(pc[0], a, vreg[ks]);
            else
                mfma32_vacc<(ks == 0), (i < 2)>(sc[0], a, kreg[ks]);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
};

template <int D, bool SEG>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                          const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                          const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_kv,
                          const float* __restrict__ ws_lse2, const float* __restrict__ ws_delta,
                          __bf16* __restrict__ dk, __bf16* __restrict__ dv, int S, int S_pad,
                          int H, float c_log2, float scale, int n_blk, int n_qt, int n_wg,
                          const int* __restrict__ ord) {
    using T = BTile<D>;
    using K = DkDv<D, SEG>;
    constexpr int kSlots = K::kSlots;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    int blk, bh;
    wg_coords(n_blk, n_wg, blk, bh);
    const int h = bh % H, b = bh / H;
    if (SEG) blk = ord[(int64_t)b * n_blk + blk];  // rank -> key block, longest first
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 31, g = lane >> 5;
    const int kj = blk * kBwdRows + wave * 32 + lr;  // this lane's key
    const int64_t ts = (int64_t)H * D;
    const int64_t head0 = (int64_t)b * S * ts + (int64_t)h * D;
    const __bf16* qp = q + head0;
    const __bf16* dop = dout + head0;
    const float* l2p = ws_lse2 + (int64_t)bh * S_pad;
    const float* dlp = ws_delta + (int64_t)bh * S_pad;
    const int32_t* sqp = SEG ? seg_q + (int64_t)b * S : nullptr;

    K A;
    A.smem = smem;
    A.g = g;
    A.c_log2 = c_log2;
    // K and V slices of this lane's key as B operands (k = d, n = key).
    {
        const int64_t off = head0 + (int64_t)kj * ts + 8 * g;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) {
            A.kreg[ks] = (kj < S) ? *reinterpret_cast<const bf16x8*>(k + off + 16 * ks) : bf16x8{};
            A.vreg[ks] = (kj < S) ? *reinterpret_cast<const bf16x8*>(v + off + 16 * ks) : bf16x8{};
        }
    }
    A.myseg = SEG ? ((kj < S) ? seg_kv[(int64_t)b * S + kj] : 0) : 1;
    A.L.init(wave, lane, ts);
    A.init_bases();

    uint16_t* list = reinterpret_cast<uint16_t*>(smem + kSlots * T::kStage);
    int* meta = reinterpret_cast<int*>(smem + ((kSlots * T::kStage + 2 * (SEG ? n_qt : 0) + 15) & ~15));
    int n_act = n_qt;
    if (SEG)
        n_act = classify_tiles<kBwdWaves>(A.myseg, sqp, S, n_qt, reinterpret_cast<uint8_t*>(smem), list, meta, wave,
                             lane);

    auto tile_of = [&](int n, bool& partial) -> int {
        if (SEG) {
            const int e = __builtin_amdgcn_readfirstlane((int)list[n]);
            partial = (e & 0x8000) != 0;
            return e & 0x7fff;
        }
        partial = false;
        return n;
    };
    // Copies of query tile n of the active list into slot n % 4: this wave's
    // share of Q and dO (rows past S re-read row S-1; their lse2 is +inf), the
    // lse2 and delta rows (wave 0) and the query segment IDs (wave 1).
    auto copy = [&](int n) {
        bool part;
        const int t = tile_of(n, part);
        char* st = smem + (n % kSlots) * T::kStage;
        const int64_t row0 = (int64_t)t * 64;
        const __bf16* sq = qp + row0 * ts;
        const __bf16* sd = dop + row0 * ts;
        const bool tail = row0 + 64 > S;
#pragma unroll
        for (int jj = 0; jj < T::kLoads; ++jj) {
            uint32_t off = A.L.dmo[jj];
            if (tail) {
                const int over = max(0, (int)row0 + Lanes<D>::dma_row(wave, jj, lane) - (S - 1));
                off -= (uint32_t)over * (uint32_t)(2 * ts);
            }
            const int i = wave * T::kLoads + jj;
            dma16(sq, off, st + T::kA + i * 1024);
            dma16(sd, off, st + T::kB + i * 1024);
        }
        if (wave == 0) {
            dma4(l2p + row0, 4u * (uint32_t)lane, st + T::kVec0);
            dma4(dlp + row0, 4u * (uint32_t)lane, st + T::kVec1);
        }
        if (SEG && wave == 1) {
            const int r = min((int)row0 + lane, S - 1);
            dma4(sqp, 4u * (uint32_t)r, st + T::kSeg);
        }
    };

#pragma unroll
    for (int i = 0; i < T::kDBlocks; ++i) A.dkacc[i] = A.dvacc[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < T::kDBlocks; ++i) asm volatile("" : "+a"(A.dkacc[i]), "+a"(A.dvacc[i]));

    if (n_act > 0) {
        copy(0);
        if (n_act > 1) copy(1);
        wait_vm(0);
        barrier();
        // Wait for the K/V slices (and the key's segment ID) here rather than
        // in the loop, where a vmcnt wait would also drain the tile copies,
        // and move the slices into AGPRs now, once: the MFMAs read them from
        // there, and their VALU writes need wait states before the first read.
        asm volatile("" ::"v"(A.kreg[0]), "v"(A.kreg[T::kSteps - 1]), "v"(A.vreg[0]),
                     "v"(A.vreg[T::kSteps - 1]), "v"(A.myseg));
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) asm volatile("" : "+a"(A.kreg[ks]), "+a"(A.vreg[ks]));
        asm volatile("s_nop 3" ::: "memory");

        const uint32_t sm = lds_addr(smem);
        // Tile iteration t = sub-iterations 2t (half 0) and 2t + 1 (half 1):
        //   2t:     dV/dK of (t-1, 1); S/dP of (t, 1) with softmax of (t, 0)
        //   2t + 1: dV/dK of (t, 0); S/dP of (t+1, 0) with softmax of (t, 1)
        // Every iteration has this one shape (and the register allocator one
        // assignment, so it never relocates an accumulator next to an
        // inline-asm MFMA): for t = 0 the dV/dK step of "(t-1, 1)" reads
        // tile 0 with P = dS = 0 and adds exactly 0, and for the last tile
        // the S/dP step of "(t+1, 0)" reads the current slot and its result
        // is never used.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) A.pb[1][kk] = A.dsb[1][kk] = bf16x8{};
        {
            const typename K::RowBases r0 = A.rows(sm + K::slot(0));
            A.prefetch_a(r0, 0);
            A.step_a_only(r0);
        }
        accumulator_fence();
        {
            const typename K::TrBases t0 = A.trs(sm + K::slot(0));
            static_for<0, kPf>([&](auto ic) { A.ring[ic] = A.template op_b<ic>(t0, 1); });
        }
        for (int t = 0; t < n_act; ++t) {
            const bool more = t + 2 < n_act;
            if (more) copy(t + 2);
            bool part;
            tile_of(t, part);
            part = SEG && part;
            const uint32_t s0 = sm + K::slot(t);
            const uint32_t sp = (t > 0) ? sm + K::slot(t - 1) : s0;
            const uint32_t sn = (t + 1 < n_act) ? sm + K::slot(t + 1) : s0;
            const typename K::TrBases tp = A.trs(sp), tc = A.trs(s0);
            const typename K::RowBases rc = A.rows(s0), rn = A.rows(sn);
            const uint32_t pc = A.pair_base(s0);
            A.prefetch_pairs(pc, 0, part);
            A.template step_b<1, true, 0>(tp, 1, rc, 1, pc, 0, part);
            A.template step_a<0, true>(rc, 1, tc, pc, 0, part);
            A.prefetch_pairs(pc, 1, part);
            A.template step_b<0, true, 1>(tc, 0, rn, 0, pc, 1, part);
            A.template step_a<1, true>(rn, 0, tc, pc, 1, part);
            if (more) wait_vm(0);
            barrier();
        }
        // dV/dK of the last sub-tile (tile n_act - 1, half 1).
        {
            const typename K::TrBases tl = A.trs(sm + K::slot(n_act - 1));
            A.template step_b<1, false, -1>(tl, 1, typename K::RowBases{}, 0, 0, 0, false);
        }
    }

    // ---- epilogue: dk = scale dK^T, dv = dV^T (bf16) ----------------------------
    accumulator_fence();
    if (kj < S) {
        const int64_t o = head0 + (int64_t)kj * ts;
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * g;
                __bf16 k4[4], v4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    k4[e] = (__bf16)(A.dkacc[db][4 * r4 + e] * scale);
                    v4[e] = (__bf16)A.dvacc[db][4 * r4 + e];
                }
                *reinterpret_cast<uint2*>(dk + o + d) = *reinterpret_cast<const uint2*>(k4);
                *reinterpret_cast<uint2*>(dv + o + d) = *reinterpret_cast<const uint2*>(v4);
            }
        }
    }
}

// ---- dQ --------------------------------------------------------------------------
template <int D, bool SEG>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void attn_bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                        const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                        const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_kv,
                        const float* __restrict__ ws_lse2, const float* __restrict__ ws_delta,
                        __bf16* __restrict__ dq, int S, int S_pad, int H, float c_log2, float scale,
                        int n_blk, int n_kt, int n_wg, const int* __restrict__ ord) {
    using T = BTile<D>;
    constexpr int kSlots = 2;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    int blk, bh;
    wg_coords(n_blk, n_wg, blk, bh);
    const int h = bh % H, b = bh / H;
    if (SEG) blk = ord[(int64_t)b * n_blk + blk];  // rank -> query block, longest first
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 31, g = lane >> 5;
    const int qi = blk * kBwdRows + wave * 32 + lr;  // this lane's query
    const int64_t ts = (int64_t)H * D;
    const int64_t head0 = (int64_t)b * S * ts + (int64_t)h * D;
    const __bf16* kp = k + head0;
    const __bf16* vp = v + head0;
    const int32_t* skp = SEG ? seg_kv + (int64_t)b * S : nullptr;

    // Q and dO slices of this lane's query as B operands (k = d, n = query).
    bf16x8 qreg[T::kSteps], doreg[T::kSteps];
    {
        const int64_t off = head0 + (int64_t)qi * ts + 8 * g;
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) {
            qreg[ks] = (qi < S) ? *reinterpret_cast<const bf16x8*>(q + off + 16 * ks) : bf16x8{};
            doreg[ks] = (qi < S) ? *reinterpret_cast<const bf16x8*>(dout + off + 16 * ks) : bf16x8{};
        }
    }
    const int myseg = SEG ? ((qi < S) ? seg_q[(int64_t)b * S + qi] : 0) : 1;
    const float lse2 = (qi < S) ? ws_lse2[(int64_t)bh * S_pad + qi] : INFINITY;
    const float delta = (qi < S) ? ws_delta[(int64_t)bh * S_pad + qi] : 0.f;

    Lanes<D> L;
    L.init(wave, lane, ts);
    // Lane offsets of the operand reads within a stage (row reads per k-step,
    // the two halves of the transposed reads per d-block).
    uint32_t rxk[T::kSteps], txk0[T::kDBlocks], txk1[T::kDBlocks];
#pragma unroll
    for (int ks = 0; ks < T::kSteps; ++ks) rxk[ks] = (uint32_t)(L.rx ^ (ks << 5));
#pragma unroll
    for (int db = 0; db < T::kDBlocks; ++db) {
        txk0[db] = (uint32_t)(L.tx0 ^ (db << 6));
        txk1[db] = (uint32_t)(L.tx1 ^ (db << 6));
    }

    uint16_t* list = reinterpret_cast<uint16_t*>(smem + kSlots * T::kStage);
    int* meta = reinterpret_cast<int*>(smem + ((kSlots * T::kStage + 2 * (SEG ? n_kt : 0) + 15) & ~15));
    int n_act = n_kt;
    if (SEG)
        n_act = classify_tiles<kBwdWaves>(myseg, skp, S, n_kt, reinterpret_cast<uint8_t*>(smem), list, meta, wave,
                             lane);

    auto tile_of = [&](int n, bool& partial) -> int {
        if (SEG) {
            const int e = __builtin_amdgcn_readfirstlane((int)list[n]);
            partial = (e & 0x8000) != 0;
            return e & 0x7fff;
        }
        partial = (n == n_kt - 1) && (S % 64 != 0);
        return n;
    };
    // Copies of key tile n into slot n % 2: this wave's share of K and V (rows
    // past S re-read row S-1; the masks exclude them) and, from wave 1, the key
    // segment IDs.  Issued one iteration before the tile is read.
    auto copy = [&](int n) {
        bool part;
        const int t = tile_of(n, part);
        char* st = smem + (n % kSlots) * T::kStage;
        const int64_t row0 = (int64_t)t * 64;
        const __bf16* sk = kp + row0 * ts;
        const __bf16* sv = vp + row0 * ts;
        const bool tail = row0 + 64 > S;
#pragma unroll
        for (int jj = 0; jj < T::kLoads; ++jj) {
            uint32_t off = L.dmo[jj];
            if (tail) {
                const int over = max(0, (int)row0 + Lanes<D>::dma_row(wave, jj, lane) - (S - 1));
                off -= (uint32_t)over * (uint32_t)(2 * ts);
            }
            const int i = wave * T::kLoads + jj;
            dma16(sk, off, st + T::kA + i * 1024);
            dma16(sv, off, st + T::kB + i * 1024);
        }
        if (SEG && wave == 1) {
            const int r = min((int)row0 + lane, S - 1);
            dma4(skp, 4u * (uint32_t)r, st + T::kSeg);
        }
    };

    // dQ^T accumulators in AGPRs; the Q and dO slices move there too (B
    // operands of the inline-asm MFMAs, see mfma32_vacc / mfma32_acc).
    f32x16 dqacc[T::kDBlocks];
#pragma unroll
    for (int i = 0; i < T::kDBlocks; ++i) dqacc[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < T::kDBlocks; ++i) asm volatile("" : "+a"(dqacc[i]));

    if (n_act > 0) copy(0);
    wait_vm(0);
    barrier();
    asm volatile("" ::"v"(qreg[0]), "v"(qreg[T::kSteps - 1]), "v"(doreg[0]), "v"(doreg[T::kSteps - 1]),
                 "v"(myseg), "v"(lse2), "v"(delta));
#pragma unroll
    for (int ks = 0; ks < T::kSteps; ++ks) asm volatile("" : "+a"(qreg[ks]), "+a"(doreg[ks]));
    asm volatile("s_nop 3" ::: "memory");
    const bool live = myseg != 0;

    // Operands are fetched kPf MFMAs ahead through a ring two entries longer.
    constexpr int kRing = kPf + 2;
    constexpr int kNA = 4 * T::kSteps;    // S^T and dP^T MFMAs per 64-key tile
    constexpr int kNB = 4 * T::kDBlocks;  // dQ^T MFMAs per tile
    bf16x8 ring[kRing];
    for (int n = 0; n < n_act; ++n) {
        const bool more = n + 1 < n_act;
        if (more) copy(n + 1);
        bool partial;
        const int t = tile_of(n, partial);
        const uint32_t st = lds_addr(smem) + (n % kSlots) * T::kStage;
        // Per-lane addresses of this stage, formed once per tile and pinned in
        // VGPRs, so that each operand read adds its region and row offset as
        // the instruction's immediate (left alone, the compiler keeps the
        // stage address in an SGPR and spends a VALU add on every read).
        uint32_t rb[T::kSteps], tb0[T::kDBlocks], tb1[T::kDBlocks];
#pragma unroll
        for (int ks = 0; ks < T::kSteps; ++ks) {
            rb[ks] = st + rxk[ks];
            asm volatile("" : "+v"(rb[ks]));
        }

        // S^T = K Q^T and dP^T = V dO^T over 64 keys: MFMA i takes k-step
        // i / 4, 32-key block (i / 2) % 2, S^T (even i) or dP^T (odd i).
        f32x16 sacc[2], pacc[2];
        {
            auto op = [&](auto ic) -> bf16x8 {
                constexpr int i = ic;
                return *reinterpret_cast<const bf16x8*>(
                    lds_ptr(rb[i / 4] + ((i & 1) ? T::kB : T::kA) + ((i / 2) % 2) * 32 * T::kRowBytes));
            };
            static_for<0, kPf>([&](auto ic) { ring[ic] = op(ic); });
            static_for<0, kNA>([&](auto ic) {
                constexpr int i = ic, ks = i / 4, bb = (i / 2) % 2;
                if constexpr (i + kPf < kNA) ring[(i + kPf) % kRing] = op(std::integral_constant<int, i + kPf>{});
                const bf16x8& a = ring[i % kRing];
                if constexpr (i & 1)
                    mfma32_vacc<(ks == 0), (i < 2)>(pacc[bb], a, doreg[ks]);
                else
                    mfma32_vacc<(ks == 0), (i < 2)>(sacc[bb], a, qreg[ks]);
                __builtin_amdgcn_sched_barrier(0);
            });
            // The wait states between the last MFMA write of S^T / dP^T and
            // their first VALU read, tied to the registers so that no read is
            // scheduled above them.
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                         : "+v"(sacc[0]), "+v"(sacc[1]), "+v"(pacc[0]), "+v"(pacc[1]));
        }

        // dS^T = P^T (dP^T - delta); register r of block bb holds key
        // t*64 + bb*32 + 16(r >> 3) + 8g + (r & 7).  Partial tiles (the ragged
        // last tile; with segment IDs, tiles with some pair of differing IDs)
        // mask keys past S and keys whose ID differs with selects (the slot
        // always holds 64 IDs); on full tiles every pair is valid.
        bf16x8 dsb[4];
        auto form_ds = [&](auto maskc) {
            constexpr bool kMask = decltype(maskc)::value;
            const int lim = S - t * 64 - 8 * g;
            const int* sgs = reinterpret_cast<const int*>(lds_ptr(st + T::kSeg)) + 8 * g;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jc = bb * 32 + 16 * (r >> 3) + (r & 7);
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[bb][r], c_log2, -lse2));
                    if constexpr (kMask) {
                        bool ok = jc < lim;
                        if (SEG) ok = ok & (sgs[jc] == myseg) & live;
                        p = ok ? p : 0.f;
                    }
                    dsb[2 * bb + (r >> 3)][r & 7] = (__bf16)(p * (pacc[bb][r] - delta));
                }
            }
        };
        if (partial)
            form_ds(std::true_type{});
        else
            form_ds(std::false_type{});
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) {
            tb0[db] = st + txk0[db];
            tb1[db] = st + txk1[db];
            asm volatile("" : "+v"(tb0[db]), "+v"(tb1[db]));
        }

        // dQ^T += K^T dS^T: MFMA i takes key k-step i / kDBlocks, d-block
        // i % kDBlocks.
        {
            auto op = [&](auto ic) -> bf16x8 {
                constexpr int i = ic;
                constexpr int db = i % T::kDBlocks;
                const uint32_t o = T::kA + (i / T::kDBlocks) * 16 * T::kRowBytes;
                return tr_read8(lds_ptr(tb0[db] + o), lds_ptr(tb1[db] + o));
            };
            static_for<0, kPf>([&](auto ic) { ring[ic] = op(ic); });
            static_for<0, kNB>([&](auto ic) {
                constexpr int i = ic;
                if constexpr (i + kPf < kNB) ring[(i + kPf) % kRing] = op(std::integral_constant<int, i + kPf>{});
                mfma32_acc<(i < 2)>(dqacc[i % T::kDBlocks], ring[i % kRing], dsb[i / T::kDBlocks]);
                __builtin_amdgcn_sched_barrier(0);
            });
        }

        // The copy of tile n+1 must have landed in every wave before the
        // barrier that opens iteration n+1.
        wait_vm(0);
        barrier();
    }
    accumulator_fence();

    // ---- epilogue: dq = scale dQ^T (bf16) ------------------------------------------
    if (qi < S) {
        const int64_t o = head0 + (int64_t)qi * ts;
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * g;
                __bf16 q4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) q4[e] = (__bf16)(dqacc[db][4 * r4 + e] * scale);
                *reinterpret_cast<uint2*>(dq + o + d) = *reinterpret_cast<const uint2*>(q4);
            }
        }
    }
}

// ---- block order (segment IDs only) ----------------------------------------------
// Active-tile count of every row block of both sweeps: workgroup
// (b * n_blk + blk) * 2 + side classifies block blk of batch b -- key rows
// against query tiles for side 0 (dK/dV), query rows against key tiles for
// side 1 (dQ) -- exactly as that sweep does, and stores the count at
// cnt[(side * B + b) * n_blk + blk].
constexpr size_t count_lds(int n_tiles) {
    return (((size_t)n_tiles + 15) & ~(size_t)15) + (((size_t)2 * n_tiles + 15) & ~(size_t)15) +
           16 * sizeof(int);
}
__global__ __launch_bounds__(kBwdThreads) void attn_bwd_count_kernel(
    const int32_t* __restrict__ seg_q, const int32_t* __restrict__ seg_kv, int S, int B, int n_blk,
    int n_tiles, int* __restrict__ cnt) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int side = blockIdx.x & 1;
    const int blk = (blockIdx.x >> 1) % n_blk, b = (blockIdx.x >> 1) / n_blk;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int row = blk * kBwdRows + wave * 32 + (lane & 31);  // the sweeps' row of this lane
    const int32_t* mine_ids = (side ? seg_q : seg_kv) + (int64_t)b * S;
    const int32_t* other = (side ? seg_kv : seg_q) + (int64_t)b * S;
    const int mine = (row < S) ? mine_ids[row] : 0;
    const size_t o1 = ((size_t)n_tiles + 15) & ~(size_t)15;
    const size_t o2 = o1 + (((size_t)2 * n_tiles + 15) & ~(size_t)15);
    const int n = classify_tiles<kBwdWaves>(mine, other, S, n_tiles, reinterpret_cast<uint8_t*>(smem),
                                            reinterpret_cast<uint16_t*>(smem + o1),
                                            reinterpret_cast<int*>(smem + o2), wave, lane);
    if (tid == 0) cnt[((int64_t)side * B + b) * n_blk + blk] = n;
}

// Longest-first order of the row blocks of one (side, batch), workgroup
// side * B + b: ord[r] is the block with the r-th largest count, ties by
// block index (a permutation of 0 .. n_blk - 1).
constexpr int kRankThreads = 1024;
__global__ __launch_bounds__(kRankThreads) void attn_bwd_rank_kernel(const int* __restrict__ cnt,
                                                                    int* __restrict__ ord, int n_blk) {
    extern __shared__ int c[];
    const int64_t base = (int64_t)blockIdx.x * n_blk;
    for (int i = threadIdx.x; i < n_blk; i += kRankThreads) c[i] = cnt[base + i];
    __syncthreads();
    for (int i = threadIdx.x; i < n_blk; i += kRankThreads) {
        const int ci = c[i];
        int r = 0;
        for (int j = 0; j < n_blk; ++j) r += (c[j] > ci) | ((c[j] == ci) & (j < i));
        ord[base + r] = i;
    }
}
static_assert(count_lds(kBwdMaxTiles) <= kLdsBytes && (size_t)(kBwdMaxTiles * 64 / kBwdRows) * sizeof(int) <= kLdsBytes,
              "block-order scratch must fit in the LDS");

template <int D>
constexpr size_t dkdv_lds(bool seg, int n_tiles) {
    const size_t b = DkDv<D, false>::kSlots * (size_t)BTile<D>::kStage + (seg ? 2 * (size_t)n_tiles : 0);
    return ((b + 15) & ~(size_t)15) + 16 * sizeof(int);
}
template <int D>
constexpr size_t dq_lds(bool seg, int n_tiles) {
    const size_t b = 2 * (size_t)BTile<D>::kStage + (seg ? 2 * (size_t)n_tiles : 0);
    return ((b + 15) & ~(size_t)15) + 16 * sizeof(int);
}
static_assert(dkdv_lds<128>(true, kBwdMaxTiles) <= kLdsBytes && dkdv_lds<64>(true, kBwdMaxTiles) <= kLdsBytes &&
                  dq_lds<128>(true, kBwdMaxTiles) <= kLdsBytes && dq_lds<64>(true, kBwdMaxTiles) <= kLdsBytes,
              "a full active-tile list must fit in the LDS beside the ring");

template <int D, bool SEG>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
    const int S_pad = (int)(((int64_t)a.S + kPad - 1) / kPad * kPad);
    float* ws_lse2 = reinterpret_cast<float*>(a.workspace);
    float* ws_delta = ws_lse2 + (int64_t)a.B * a.H * S_pad;
    const float c_log2 = a.scale * kLog2e;
    const auto* q = reinterpret_cast<const __bf16*>(a.q);
    const auto* k = reinterpret_cast<const __bf16*>(a.k);
    const auto* v = reinterpret_cast<const __bf16*>(a.v);
    const auto* dout = reinterpret_cast<const __bf16*>(a.dout);
    {
        const int64_t n_items = (int64_t)a.B * a.H * S_pad;
        const int64_t per_block = 256 / (D / 8);
        const int64_t blocks = std::min<int64_t>((n_items + per_block - 1) / per_block, 1 << 20);
        hipLaunchKernelGGL((attn_bwd_prep_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const __bf16*>(a.out), dout, a.lse, ws_lse2, ws_delta,
                           a.S, a.H, S_pad, n_items);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int n_blk = (a.S + kBwdRows - 1) / kBwdRows;
    const int n_tiles = (a.S + 63) / 64;
    const int n_wg = (int)((int64_t)a.B * a.H * n_blk);
    // Block orders: counts [side][b][blk], then orders [side][b][rank]
    // (side 0: key blocks of dK/dV, side 1: query blocks of dQ).
    int* ws_cnt = reinterpret_cast<int*>(ws_delta + (int64_t)a.B * a.H * S_pad);
    int* ws_ord = ws_cnt + 2 * (int64_t)a.B * n_blk;
    if (SEG) {
        hipLaunchKernelGGL(attn_bwd_count_kernel, dim3((unsigned)(2 * (int64_t)a.B * n_blk)), dim3(kBwdThreads),
                           count_lds(n_tiles), stream, a.seg_q, a.seg_kv, a.S, a.B, n_blk, n_tiles, ws_cnt);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_bwd_rank_kernel, dim3((unsigned)(2 * a.B)), dim3(kRankThreads),
                           (size_t)n_blk * sizeof(int), stream, ws_cnt, ws_ord, n_blk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, SEG>), dim3(n_wg), dim3(kBwdThreads),
                       dkdv_lds<D>(SEG, n_tiles), stream, q, k, v, dout, a.seg_q, a.seg_kv, ws_lse2,
                       ws_delta, reinterpret_cast<__bf16*>(a.dk), reinterpret_cast<__bf16*>(a.dv), a.S,
                       S_pad, a.H, c_log2, a.scale, n_blk, n_tiles, n_wg, ws_ord);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, SEG>), dim3(n_wg), dim3(kBwdThreads),
                       dq_lds<D>(SEG, n_tiles), stream, q, k, v, dout, a.seg_q, a.seg_kv, ws_lse2,
                       ws_delta, reinterpret_cast<__bf16*>(a.dq), a.S, S_pad, a.H, c_log2, a.scale,
                       n_blk, n_tiles, n_wg, ws_ord + (int64_t)a.B * n_blk);
    return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t B, int64_t S, int64_t H) {
    const int64_t S_pad = (S + kPad - 1) / kPad * kPad;
    const int64_t n_blk = (S + kBwdRows - 1) / kBwdRows;
    return (size_t)(2 * B * H * S_pad) * sizeof(float) + (size_t)(4 * B * n_blk) * sizeof(int);
}

int64_t bwd_max_masked_seq() { return (int64_t)kBwdMaxTiles * 64; }
int64_t bwd_rows_per_workgroup() { return kBwdRows; }

hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t stream) {
    const bool seg = a.seg_q != nullptr;
    if (a.D == 128) return seg ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
    return seg ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
}

}  // namespace vdx
