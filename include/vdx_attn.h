/*
 * vdx_attn.h -- C ABI of the segment-masked, non-causal flash-attention
 * forward for video-DiT token volumes on gfx950 (MI355X).
 *
 * The operation (vidax paper, arXiv:2609.18077):
 *   - section 1, "Spatiotemporal constraints in video generation": full
 *     self-attention over the patchified frames x h x w token volume, tens of
 *     thousands of tokens per sequence;
 *   - section 2, "3D RoPE, 3D VAEs, and flash attention": attention runs as a
 *     flash-attention kernel (reference [2], exact attention computed tile by
 *     tile, the S x S score matrix never stored);
 *   - Appendix A, Table 4, group 2 (HunyuanVideo-1.5 row): per-token segment
 *     IDs replace a dense (B, H, Sq, Sk) mask and let invalid key blocks be
 *     skipped; Table 4, group 1 (CogVideoX row): padding must be masked.
 *
 * For every batch b, head h and query i:
 *     J    = { j : seg_q[b,i] == seg_kv[b,j] and seg_q[b,i] != 0 }
 *            (all j when both segment pointers are NULL)
 *     s_j  = scale * sum_d q[b,i,h,d] * k[b,j,h,d]
 *     out[b,i,h,:] = sum_{j in J} softmax(s)_j * v[b,j,h,:]       (bf16, RNE)
 *     lse[b,h,i]   = log(sum_{j in J} exp(s_j))                  (fp32, natural log)
 *   A row with empty J gets out = +0.0 (all bits zero) and lse = -inf.
 *   Segment ID 0 marks padding: it matches nothing, itself included.
 *
 * Every pointer argument is a DEVICE pointer owned by the caller.  The library
 * allocates nothing, keeps no pointer after returning and holds no state
 * beyond a per-device, once-cached architecture check.  Calls are
 * asynchronous on `stream` (0 = null stream); buffers must stay alive until
 * the stream work completes.  Results are deterministic: the same inputs give
 * bit-identical outputs (fixed reduction order, no atomics).
 */
#ifndef VDX_ATTN_H
#define VDX_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

#define VDX_ABI_VERSION 1

/* Status codes.  Argument validation runs before any HIP call, in the order
 * below (NULL -> segment pair -> shape -> head dim -> scale -> alignment),
 * and reports the first failure without touching device memory. */
enum vdx_status {
    VDX_OK = 0,
    VDX_ERR_NULL_PTR = 1, /* q, k, v, out or lse is NULL                        */
    VDX_ERR_SEG_PAIR = 2, /* exactly one of seg_q / seg_kv is NULL              */
    VDX_ERR_SHAPE = 3,    /* B, S or H < 1, element count overflows int64, the
                             grid would exceed 2^31-1 workgroups, 64*H*D
                             exceeds 2^31-1, or a masked call has
                             S > 1,966,080 (the on-chip key-tile table holds
                             30,720 tiles of 64 keys)                          */
    VDX_ERR_HEAD_DIM = 4, /* D is not 64 or 128                                 */
    VDX_ERR_SCALE = 5,    /* scale is not finite or is <= 0                     */
    VDX_ERR_ALIGN = 6,    /* q, k, v, out not 16-byte aligned; seg_q, seg_kv or
                             lse not 4-byte aligned                              */
    VDX_ERR_DEVICE = 7,   /* the current HIP device is not gfx950, or the
                             device query failed                                */
    VDX_ERR_LAUNCH = 8    /* the kernel launch reported an error                */
};

/*
 * vdx_attn_fwd -- one forward pass of segment-masked self-attention.
 *
 *   q, k, v   bf16 [B, S, H, D], contiguous (token stride H*D elements),
 *             read-only; they may alias each other.
 *   seg_q     int32 [B, S] segment ID per query token, or NULL.
 *   seg_kv    int32 [B, S] segment ID per key/value token, or NULL.
 *             Both NULL = unmasked (every pair valid); exactly one NULL is
 *             VDX_ERR_SEG_PAIR.
 *   out       bf16 [B, S, H, D], written in full (no pre-zeroing needed).
 *   lse       fp32 [B, H, S], natural-log log-sum-exp of the scaled scores
 *             over each row's valid keys, written in full.
 *             out and lse must not overlap any input or each other.
 *   B, S, H   batch, tokens per sequence (queries = keys = S), heads; >= 1.
 *   D         head dim, 64 or 128.
 *   scale     finite, > 0; multiplies q . k (typically 1/sqrt(D)).
 *   stream    HIP stream the kernel is enqueued on; no host synchronisation.
 *
 * Returns VDX_OK or a vdx_status code.  Faults during kernel execution
 * surface at the caller's next synchronisation, as usual for HIP.
 */
int vdx_attn_fwd(const void* q, const void* k, const void* v,
                 const int32_t* seg_q, const int32_t* seg_kv,
                 void* out, float* lse,
                 int B, int S, int H, int D, float scale, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* vdx_status_str(int status);

/* VDX_ABI_VERSION of the built library. */
int vdx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VDX_ATTN_H */
