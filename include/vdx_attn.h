/*
 * vdx_attn.h -- C ABI of the segment-masked, non-causal flash-attention
 * forward for video-DiT token volumes on gfx950 (MI355X), of the 3D
 * neighbourhood (windowed) attention forward (vdx_natten3d_fwd, below), of
 * the attention gradient (vdx_attn_bwd, below), and of the 3D rotary
 * position embedding of queries and keys, alone (vdx_rope3d_apply) and fused
 * into the attention forward (vdx_rope3d_attn_fwd).
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
 * the stream work completes.  Results are deterministic: the same inputs on
 * the same device give bit-identical outputs (fixed reduction order, no
 * atomics in the arithmetic; the *_ws entry points hand out work items with
 * atomic counters in their workspace, which decides only which workgroup
 * computes an item, and split some items along their keys by a rule fixed
 * by the shape and the device's CU count).
 */
#ifndef VDX_ATTN_H
#define VDX_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

#define VDX_ABI_VERSION 7

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
    VDX_ERR_LAUNCH = 8,   /* the kernel launch reported an error                */
    VDX_ERR_WINDOW = 9,   /* vdx_natten3d_fwd: a window size is even or < 1, or
                             the effective x window min(KW, NW) exceeds 13      */
    VDX_ERR_WORKSPACE = 10, /* vdx_attn_bwd, or a *_ws forward with segment
                             IDs: workspace NULL, smaller than the call's
                             vdx_attn_*_workspace_size(B, S, H), or not
                             16-byte aligned                                    */
    VDX_ERR_ROPE = 11,    /* vdx_rope3d_*: the embedding description is NULL,
                             its pos is NULL, a section width is odd or < 0,
                             the widths add up to more than D, a row count is
                             < 0, a table of a section of nonzero width is
                             NULL, or pos / a table is not 4-byte aligned      */
    VDX_ERR_SCRATCH = 12  /* vdx_attn_bwd_noalloc: vdx_attn_bwd_workspace_size
                             (B, S, H) exceeds VDX_BWD_NOALLOC_SCRATCH_BYTES   */
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

/*
 * vdx_attn_fwd_ws -- vdx_attn_fwd with a caller workspace, which the call
 * uses to balance uneven work and to split the last items of a persistent
 * launch; the same operation.
 *
 * The pages motivate it (vidax paper, arXiv:2609.18077, Appendix A, Table 4,
 * group 2): with SegmentIds a query block skips every key block of other
 * segments, so blocks of short and long clips packed into one sequence do
 * very different amounts of work.  With segment IDs this call enqueues a
 * summary of every 64-key tile's IDs, the active-tile count of every
 * 256-query block, each batch's blocks ordered longest first, then a
 * persistent forward whose workgroups pull (block, head) items in that order
 * from per-XCD work counters and classify tiles from the summaries.  The
 * counters change only which workgroup computes an item, never its result.
 *
 * A persistent launch has G workgroups (the CU count rounded down to a
 * multiple of 8; W = G / 8 per XCD); an item is one (batch, head, 256-query
 * block).  Split items: an item is split along its active key tiles into P
 * parts run side by side, and a last kernel merges each item's parts (their
 * running maxima, sums and unnormalised outputs, added in part order).
 * Every other query block gives vdx_attn_fwd's bits; a split block equals
 * them up to rounding (each part rounds its probabilities to bf16 against
 * its own running maximum), within the same accuracy bound.  Which items
 * are split: none when there are no more items n than G.  Otherwise XCD x
 * holds n_x = per + (x < rem) items (per = n / 8, rem = n mod 8).
 *   - Without segment IDs XCD x's items are a contiguous run starting at
 *     item x per + min(x, rem) (items numbered (b H + h) ceil(S / 256) +
 *     block); its last R are split into P = min(8, W / R) parts when that is
 *     >= 2, R = W / 4 when n_x / W >= 4, else R = n_x mod W.  The XCD's
 *     workgroups claim its units from its own counter, then from the other
 *     XCDs'.
 *   - With segment IDs XCD x's items are its longest-first list; its counter
 *     hands out its first K W (K = per / W - 2 when per / W >= 4, else
 *     per / W), the rest of every XCD's list forms a pool of n - K G items
 *     (XCD x's after those of XCDs below x) that every workgroup pulls from
 *     once its own items are done, and the pool's last R items (G / 4 when
 *     per / W >= 4, else all of them) are split into P = min(8, 256 / R,
 *     G / R) parts when that is >= 2.
 * The XCDs run at different speeds under this load; both schedules let the
 * faster ones take over the slower ones' last items.
 *
 *   q ... scale, stream   exactly as for vdx_attn_fwd.
 *   workspace  device scratch of at least vdx_attn_fwd_workspace_size(B, S,
 *              H) bytes, 16-byte aligned, owned by the caller; its contents
 *              on entry do not matter and are overwritten (two calls in
 *              flight at once need two workspaces).  Required with segment
 *              IDs.  Without them it may be NULL, and the call is then
 *              vdx_attn_fwd (no pool, no split).
 * Validation: as vdx_attn_fwd, then the workspace (with segment IDs, or
 * whenever it is not NULL) -> VDX_ERR_WORKSPACE; the first failure is
 * reported before any HIP call.  Results are deterministic.
 */
int vdx_attn_fwd_ws(const void* q, const void* k, const void* v,
                    const int32_t* seg_q, const int32_t* seg_kv,
                    void* out, float* lse, void* workspace, size_t workspace_bytes,
                    int B, int S, int H, int D, float scale, hipStream_t stream);

/* Bytes of workspace vdx_attn_fwd_ws needs for (B, S, H): 256 (work
 * counters) + R(16 * B * ceil(S / 64)) (tile summaries) + R(4 * B *
 * ceil(S / 256)) (block counts) + R(4 * B * ceil(S / 256)) (block orders) +
 * 256 * 256 * 130 * 4 (part records of the split items: per part the
 * fp32 unnormalised output, maximum and sum of 256 rows at D <= 128), R()
 * rounding up to a multiple of 256.  H does not enter.  0 if B, S or H < 1. */
size_t vdx_attn_fwd_workspace_size(int B, int S, int H);

/*
 * vdx_natten3d_fwd -- one forward pass of 3D neighbourhood (windowed)
 * self-attention over a t x h x w token grid.
 *
 * The operation (vidax paper, arXiv:2609.18077):
 *   - section 2, "3D RoPE, 3D VAEs, and flash attention": models without a
 *     native kernel for it, such as LTX-2.5's neighbourhood-attention VAE
 *     decoder, use a windowed-attention primitive;
 *   - Appendix A, Table 4, group 4 (LTX-2.5 VAE decoder rows): the window
 *     spans 11 x 11 x 11 grid positions for that model's stage-5 kernel.
 *
 * Tokens are the grid flattened (t, y, x), x fastest: S = NT*NH*NW and token
 * s = (t*NH + y)*NW + x.  Along an axis of length n, a window of odd size k
 * covers k_eff = min(k, n) positions starting at clamp(c - k/2, 0, n - k_eff)
 * (it shifts inward at the grid border, so every query sees exactly
 * k_eff,t * k_eff,h * k_eff,w keys).  For every batch b, head h, query i:
 *     J    = the keys in the window of i
 *     out[b,i,h,:] = sum_{j in J} softmax(scale * q_i . k_j)_j * v[b,j,h,:]  (bf16, RNE)
 *     lse[b,h,i]   = log(sum_{j in J} exp(scale * q_i . k_j))               (fp32)
 *
 *   q, k, v   bf16 [B, S, H, D], contiguous, read-only (may alias).
 *   out, lse  bf16 [B, S, H, D] and fp32 [B, H, S], written in full; they must
 *             not overlap the inputs or each other.
 *   NT,NH,NW  grid extents (>= 1), S = NT*NH*NW <= 2^31-1.
 *   H, D      heads >= 1; D is 64 or 128.
 *   KT,KH,KW  odd window sizes >= 1; min(KW, NW) <= 13.
 *   scale     finite, > 0.
 *   stream    HIP stream; asynchronous, no host synchronisation.
 * Every pointer is a DEVICE pointer owned by the caller; the library
 * allocates nothing.  Validation runs before any HIP call, in the order
 * NULL -> shape -> head dim -> window -> scale -> alignment (q, k, v, out
 * 16-byte, lse 4-byte), and reports the first failure without touching
 * device memory.  Results are deterministic.
 */
int vdx_natten3d_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int NT, int NH, int NW, int H, int D, int KT, int KH, int KW,
                     float scale, hipStream_t stream);

/*
 * vdx_attn_bwd -- gradient of vdx_attn_fwd: dq, dk, dv for a given dout.
 *
 * The operation (vidax paper, arXiv:2609.18077): section 5, "Conclusions &
 * Future Work", lists training and fine-tuning (LoRA and full-parameter) of
 * the video models as future work; training needs this gradient of the
 * attention of section 2 / Appendix A, Table 4, groups 1 and 2.  With J_i
 * and s_ij as for vdx_attn_fwd and P_ij = exp(s_ij - lse[b,h,i]) for j in J_i
 * (0 otherwise), for every batch b and head h:
 *     dv_j    = sum_i P_ij dout_i
 *     dP_ij   = dout_i . v_j,     delta_i = dout_i . out_i  (= sum_j P_ij dP_ij)
 *     dS_ij   = P_ij (dP_ij - delta_i)
 *     dq_i    = scale * sum_j dS_ij k_j
 *     dk_j    = scale * sum_i dS_ij q_i
 *   (vectors over the head dim; all written as bf16, RNE, accumulated in
 *   fp32).  Rows with empty J_i (lse = -inf) get dq_i = 0 and contribute
 *   nothing to dk and dv; keys that no query attends get dk_j = dv_j = 0.
 *
 *   q, k, v, seg_q, seg_kv, B, S, H, D, scale
 *             exactly as passed to vdx_attn_fwd.
 *   out, lse  that call's outputs (bf16 [B, S, H, D], fp32 [B, H, S]).
 *   dout      bf16 [B, S, H, D], gradient of the loss with respect to out.
 *   dq,dk,dv  bf16 [B, S, H, D], written in full; they must not overlap any
 *             input, the workspace or each other.
 *   workspace device scratch of at least vdx_attn_bwd_workspace_size(B, S, H)
 *             bytes, 16-byte aligned, owned by the caller; its contents on
 *             entry do not matter and are overwritten (it holds per-row
 *             fp32 terms and, with segment IDs, per-block work counts and
 *             orders between the kernels of one call, so two calls in
 *             flight at once need two workspaces).
 *   stream    HIP stream; the kernels (three, five with segment IDs) are
 *             enqueued on it in order, asynchronous, no host
 *             synchronisation.
 * Every pointer is a DEVICE pointer owned by the caller; the library
 * allocates nothing.  Validation runs before any HIP call, in the order
 * NULL (q, k, v, out, lse, dout, dq, dk, dv) -> segment pair -> shape (as for
 * vdx_attn_fwd, and S <= 2^31 - 65; a masked call needs S <= 896,000: the
 * on-chip query-tile table of the dK/dV sweep holds 14,000 tiles of 64)
 * -> head dim -> scale -> alignment (bf16
 * tensors 16-byte, lse and segment IDs 4-byte) -> workspace, and reports the
 * first failure without touching device memory.  Results are deterministic
 * (no atomics).
 */
int vdx_attn_bwd(const void* q, const void* k, const void* v,
                 const int32_t* seg_q, const int32_t* seg_kv,
                 const void* out, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int S, int H, int D, float scale, hipStream_t stream);

/*
 * vdx_attn_bwd_noalloc -- vdx_attn_bwd with no workspace argument and no
 * allocation of any kind, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, semantics and results as vdx_attn_bwd (bit for
 * bit) without workspace / workspace_bytes.
 *
 * The scratch vdx_attn_bwd would take from its workspace lives in one static
 * device array of VDX_BWD_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held by the
 * library until the process ends; a call needs
 * vdx_attn_bwd_workspace_size(B, S, H) bytes of it (the 720p layer, B=1,
 * S=75,600, H=40, needs 24.2 MB) and returns VDX_ERR_SCRATCH, before any HIP
 * call, if that is more.  Every call on a GPU shares that GPU's array, which
 * keeps the last call's contents (nothing in it needs clearing: each call
 * writes what it reads): calls that overlap in time on one GPU -- on
 * different streams, or from different threads -- race and give wrong
 * results; serialise them.  The first call on a device looks up the array's
 * address there (the call's current device).
 * Validation order: as vdx_attn_bwd up to alignment, then the scratch size.
 */
#define VDX_BWD_NOALLOC_SCRATCH_BYTES (32u << 20)
int vdx_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                         const int32_t* seg_q, const int32_t* seg_kv,
                         const void* out, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv,
                         int B, int S, int H, int D, float scale, hipStream_t stream);

/* Bytes of workspace vdx_attn_bwd needs for (B, S, H): 8 * B * H * S_pad with
 * S_pad = S rounded up to a multiple of 64 (two fp32 terms per row), plus
 * 16 * B * ceil(S / 128) (per batch, the active-tile count and the
 * longest-first rank of every 128-row block of both sweeps, used with
 * segment IDs).  0 if B, S or H < 1 or the size overflows. */
size_t vdx_attn_bwd_workspace_size(int B, int S, int H);

/*
 * 3D rotary position embedding of queries and keys.
 *
 * The operation (vidax paper, arXiv:2609.18077): section 2, "3D RoPE, 3D VAEs,
 * and flash attention", places a rotary position embedding over time, height
 * and width on the queries and keys right before attention and notes that
 * the families' conventions differ and are kept exactly; section 3.1 names
 * Wan and CogVideoX1.5 as 3D-RoPE DiTs.  No formula is printed, so every
 * family-specific choice is an argument:
 *   - features [0, dims[0]), [dims[0], dims[0] + dims[1]) and
 *     [dims[0] + dims[1], dims[0] + dims[1] + dims[2]) of the head dim belong
 *     to the t, y and x axes; later features are not rotated;
 *   - pair p of an axis section at offset o and width w is the features
 *     (o + 2p, o + 2p + 1) if interleaved, else (o + p, o + p + w / 2);
 *   - its angle is c = cos_tab[a][pos_a * (w / 2) + p],
 *     s = sin_tab[a][pos_a * (w / 2) + p] at the token's coordinate pos_a;
 *   - (x0, x1) becomes (x0 c - x1 s, x0 s + x1 c), formed exactly up to one
 *     rounding in fp64 and rounded once to bf16 (to nearest, ties to even);
 *   - a token with a coordinate outside its axis's table (< 0 or >= n[a]:
 *     text tokens, padding) is not rotated.
 */
typedef struct vdx_rope3d {
    const int32_t* pos;        /* DEVICE int32 [B, S, 3]: (t, y, x) per token     */
    const float* cos_tab[3];   /* DEVICE fp32 [n[a], dims[a] / 2] per axis (t, y,
                                  x); may be NULL where dims[a] == 0              */
    const float* sin_tab[3];   /* DEVICE fp32, same shapes                       */
    int n[3];                  /* table rows per axis, >= 0                      */
    int dims[3];               /* even section widths, sum <= D                  */
    int interleaved;           /* nonzero: pairs (2p, 2p + 1), else (p, p + w/2) */
} vdx_rope3d;

/*
 * vdx_rope3d_apply -- y = the 3D rotary embedding of x.
 *
 *   x, y      bf16 [B, S, H, D], contiguous, 16-byte aligned; y may be x (in
 *             place), otherwise they must not overlap.
 *   rope      host pointer to the description above (read during the call
 *             only); the tensors it points to must stay alive until the
 *             stream work completes.
 *   B, S, H   >= 1; D is 64 or 128.
 * Validation runs before any HIP call, in the order NULL (x, y) -> shape ->
 * head dim -> alignment -> rope, and reports the first failure without
 * touching device memory.  Asynchronous on `stream`; deterministic.
 */
int vdx_rope3d_apply(const void* x, void* y, const vdx_rope3d* rope,
                     int B, int S, int H, int D, hipStream_t stream);

/*
 * vdx_rope3d_attn_fwd -- vdx_attn_fwd on the 3D-rotary-embedded queries and
 * keys (v is used as given): out and lse are bit for bit those of
 * vdx_attn_fwd called on vdx_rope3d_apply(q) and vdx_rope3d_apply(k).  The
 * keys are rotated once into k_rot by a pre-pass on `stream`; the queries are
 * rotated in registers as each workgroup loads them.
 *
 *   q, k, v, seg_q, seg_kv, out, lse, B, S, H, D, scale, stream
 *             as for vdx_attn_fwd.
 *   rope      as for vdx_rope3d_apply.
 *   k_rot     DEVICE bf16 [B, S, H, D], 16-byte aligned, owned by the caller:
 *             receives the rotated keys.  It may be k itself (the keys are
 *             then rotated in place); otherwise it must not overlap q, k, v,
 *             out or lse.
 * Validation: NULL (q, k, v, out, lse, k_rot) -> segment pair -> shape -> head
 * dim -> scale -> alignment (k_rot 16-byte as well) -> rope, before any HIP
 * call and without touching device memory.
 */
int vdx_rope3d_attn_fwd(const void* q, const void* k, const void* v,
                        const int32_t* seg_q, const int32_t* seg_kv,
                        const vdx_rope3d* rope, void* k_rot,
                        void* out, float* lse,
                        int B, int S, int H, int D, float scale, hipStream_t stream);

/*
 * vdx_rope3d_attn_fwd_ws -- vdx_rope3d_attn_fwd on the schedule of
 * vdx_attn_fwd_ws (same workspace layout and size,
 * vdx_attn_fwd_workspace_size(B, S, H)): with segment IDs the persistent,
 * longest-first launch, and with or without them the split items (and,
 * without them, the pool).  Without segment IDs the workspace may be NULL
 * (then neither).  Results
 * relate to vdx_rope3d_attn_fwd's as vdx_attn_fwd_ws's to vdx_attn_fwd's.
 * Validation: as vdx_rope3d_attn_fwd, then the workspace (with segment IDs,
 * or whenever it is not NULL) -> VDX_ERR_WORKSPACE.
 */
int vdx_rope3d_attn_fwd_ws(const void* q, const void* k, const void* v,
                           const int32_t* seg_q, const int32_t* seg_kv,
                           const vdx_rope3d* rope, void* k_rot,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           int B, int S, int H, int D, float scale, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* vdx_status_str(int status);

/* VDX_ABI_VERSION of the built library. */
int vdx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VDX_ATTN_H */
