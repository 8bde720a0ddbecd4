// attn_common.h -- device building blocks shared by the gfx950 attention
// kernels: tile geometry and LDS swizzles, MFMA-layout helpers, wave
// reductions, barriers, counted waits and the direct global->LDS copies.
//
// Included by each kernel source inside its own translation unit (the
// definitions live in an anonymous namespace).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace vdx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBq = 32 * kWaves;  // queries per workgroup
constexpr int kBk = 64;           // keys per tile
constexpr int kDmaWaves = kWaves / 2;  // one ping-pong group issues each tile copy
constexpr int kSlots = 3;         // ring depth of the K, V and segment-ID stages
#ifndef VDX_OPERAND_PREFETCH
#define VDX_OPERAND_PREFETCH 4
#endif
constexpr int kOperandPrefetch = VDX_OPERAND_PREFETCH;  // MFMA operands in flight
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr size_t kLdsBytes = 160 * 1024;  // gfx950: LDS one workgroup may allocate
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
#ifndef VDX_LAZY_LOG2
#define VDX_LAZY_LOG2 8.0f
#endif
// A row's P may grow to 2^kLazyLog2 before its reference maximum is moved.
constexpr float kLazyLog2 = VDX_LAZY_LOG2;

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
    static constexpr int kLoadsPerWave = kTileBytes / 1024 / kDmaWaves;
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
// Wait until at most n of this wave's vector-memory loads are outstanding.
// Wait until at most n loads are outstanding, for the counts a phase's
// copies take (n in {0, 1, L, L+1} with L loads per tile share); the common
// count is tested first.
template <int L>
__device__ __forceinline__ void wait_copies(int n) {
    static_assert(L >= 2 && L + 1 <= 6, "unsupported copy count");
    if (n == L) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    } else if (n == L + 1) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L + 1) : "memory");
    } else if (n == 1) {
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    }
}

// Direct global->LDS copies: lane l's bytes land at LDS address M0 + size*l.
// Issued as inline asm so that the compiler does not treat every later LDS read
// as a possible alias of the in-flight copy (it would insert vmcnt(0) waits and
// serialise the prefetch); completion is tracked by hand with wait_vm() and the
// workgroup barrier that follows it.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ const char* lds_ptr(uint32_t a) {
    return (const char*)((const __attribute__((address_space(3))) char*)(uintptr_t)a);
}
// The global address is a wave-uniform base (SGPR pair) plus a per-lane
// 32-bit byte offset.  The s_nop 4 supplies the wait states GFX9 requires
// before a vector-memory instruction that reads an SGPR (the base pair, M0)
// written by a VALU instruction (five; the compiler may reload a spilled SGPR
// with v_readlane right before the asm) or M0 written by SALU (one): the
// hazard recogniser does not look inside inline asm.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, char* lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                 "{m0}"(lds_addr(lds))
                 : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, char* lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base),
                 "{m0}"(lds_addr(lds))
                 : "memory");
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

// Class of a tile pair from the two sides' summaries (min / max of the
// nonzero IDs, INT32_MAX / INT32_MIN when there are none, and a flag for an
// ID 0 or a row past S): 0 skip (no valid pair), 1 full (every pair valid:
// one nonzero ID on both sides, no padding, no rows past S), 2 partial.
// kOwnPadFree: the caller overwrites the results of its own padding rows (ID
// 0 or past S), so their pairs need no mask and only the other side's
// padding keeps a tile from being full.
template <bool kOwnPadFree = false>
__device__ __forceinline__ uint8_t tile_class(int omn, int omx, int ofl, int mn, int mx, int fl) {
    if (omn > omx || mn > mx || max(omn, mn) > min(omx, mx)) return 0;
    if ((kOwnPadFree || !ofl) && !fl && omn == omx && mn == mx && omn == mn) return 1;
    return 2;
}

// Compacts the active tiles of cls[0, n_tiles), in order, into list (bit 15
// set: partial); every wave of the workgroup (NW of them) must call it, and
// all of cls must be written before.  meta[3 NW] holds the count, which is
// returned to every wave.
template <int NW>
__device__ int compact_tiles(const uint8_t* cls, int n_tiles, uint16_t* list, int* meta, int wave, int lane) {
    __syncthreads();
    if (wave == 0) {
        int base = 0;
        for (int t0 = 0; t0 < n_tiles; t0 += 64) {
            const int t = t0 + lane;
            const int c = (t < n_tiles) ? cls[t] : 0;
            const uint64_t m = __ballot(c != 0);
            const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
            if (c != 0) list[pos] = (uint16_t)(t | ((c == 2) ? 0x8000 : 0));
            base += __popcll(m);
        }
        if (lane == 0) meta[3 * NW] = base;
    }
    __syncthreads();
    return meta[3 * NW];
}

// Summary of the workgroup's rows (ID `mine` per lane of every wave; 0 for
// padding and rows past S): min and max of the nonzero IDs (INT32_MAX /
// INT32_MIN when there are none) and a flag for an ID 0.  Every wave of the
// workgroup (NW of them) must call it; meta[3 NW] is scratch.
template <int NW>
__device__ __forceinline__ void block_summary(int mine, int* meta, int wave, int lane, int& omn, int& omx,
                                              int& ofl) {
    {
        int mn = (mine != 0) ? mine : INT32_MAX;
        int mx = (mine != 0) ? mine : INT32_MIN;
        int fl = (mine == 0) ? 1 : 0;
        mn = wave_min(mn);
        mx = wave_max(mx);
        fl = wave_max(fl);
        if (lane == 0) {
            meta[wave] = mn;
            meta[NW + wave] = mx;
            meta[2 * NW + wave] = fl;
        }
    }
    __syncthreads();
    omn = INT32_MAX;
    omx = INT32_MIN;
    ofl = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        omn = min(omn, meta[i]);
        omx = max(omx, meta[NW + i]);
        ofl |= meta[2 * NW + i];
    }
}

// Classifies every 64-row tile of the opposite side (segment IDs `other`, S
// entries) against this workgroup's rows (ID `mine` per lane; 0 for padding
// and rows past S) with tile_class() and compacts the active tiles, in
// order, into `list`.  `cls` is scratch of n_tiles bytes, `meta` of 3 NW + 1
// ints; every wave of the workgroup (NW of them) must call it.  Returns the
// number of active tiles.  A wave covers four tiles per step (16 lanes a
// tile, 4 IDs a lane) and issues kU steps' loads before reducing any of
// them, so the loads' latency overlaps instead of adding up tile by tile.
template <int NW, bool kOwnPadFree = false>
__device__ int classify_tiles(int mine, const int32_t* other, int S, int n_tiles, uint8_t* cls,
                              uint16_t* list, int* meta, int wave, int lane) {
    constexpr int kU = 4;
    int omn, omx, ofl;
    block_summary<NW>(mine, meta, wave, lane, omn, omx, ofl);
    const int gq = lane >> 4, sub = lane & 15;
    const int n_groups = (n_tiles + 3) / 4;
    for (int g0 = wave; g0 < n_groups; g0 += NW * kU) {
        int id[kU][4];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int t = (g0 + u * NW) * 4 + gq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = t * 64 + 4 * sub + e;
                id[u][e] = (t < n_tiles && r < S) ? other[r] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int t = (g0 + u * NW) * 4 + gq;
            int mn = INT32_MAX, mx = INT32_MIN, fl = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = id[u][e];
                mn = (x != 0) ? min(mn, x) : mn;
                mx = (x != 0) ? max(mx, x) : mx;
                fl |= (x == 0) ? 1 : 0;
            }
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                mn = min(mn, __shfl_xor(mn, o));
                mx = max(mx, __shfl_xor(mx, o));
                fl |= __shfl_xor(fl, o);
            }
            if (sub == 0 && t < n_tiles) cls[t] = tile_class<kOwnPadFree>(omn, omx, ofl, mn, mx, fl);
        }
    }
    return compact_tiles<NW>(cls, n_tiles, list, meta, wave, lane);
}

// classify_tiles from the opposite side's per-tile summaries instead of its
// IDs: sum[t] = {min nonzero ID, max nonzero ID, flag, 0} of tile t, as the
// loop above reduces them.  One lane per tile, four tiles' loads in flight
// per lane.
template <int NW, bool kOwnPadFree = false>
__device__ int classify_tiles_sum(int mine, const int4* sum, int n_tiles, uint8_t* cls, uint16_t* list,
                                  int* meta, int wave, int lane) {
    constexpr int kU = 4;
    int omn, omx, ofl;
    block_summary<NW>(mine, meta, wave, lane, omn, omx, ofl);
    const int tid = wave * 64 + lane;
    for (int t0 = 0; t0 < n_tiles; t0 += NW * 64 * kU) {
        int4 s[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int t = t0 + u * NW * 64 + tid;
            s[u] = (t < n_tiles) ? sum[t] : int4{INT32_MAX, INT32_MIN, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int t = t0 + u * NW * 64 + tid;
            if (t < n_tiles) cls[t] = tile_class<kOwnPadFree>(omn, omx, ofl, s[u].x, s[u].y, s[u].z);
        }
    }
    return compact_tiles<NW>(cls, n_tiles, list, meta, wave, lane);
}

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

}  // namespace
}  // namespace vdx
