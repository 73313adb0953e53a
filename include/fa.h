/*
 * fa.h -- C ABI of the MI355X (gfx950) attention-forward library.
 *
 * Computes Attention(Q,K,V) = softmax(scale * Q K^T) V tile by tile with an
 * online softmax, so the Q_S x KV_S score matrix never exists in memory
 * (FlashAttn operator guide, function description).  Three paths:
 *   - prefill (Q_S >= 1) with an optional causal or boolean mask;
 *   - incremental decode (Q_S == 1) against a padded KV cache with per-batch
 *     actual lengths and grouped-query heads (aclnnIncreFlashAttention guide,
 *     sections 1.1 and 4);
 *   - FlashDecoding split-KV: stage 1 writes an unnormalised partial output
 *     with its row maximum and exponential sum per KV chunk, stage 2 merges
 *     them (FlashDecoding tutorial, sections 2 and 3; FlashAttn developer
 *     guide, section 10).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers (HBM).  The caller allocates and
 *     owns all memory, workspace included; the library never allocates, never
 *     synchronises the host and keeps no state between calls, so calls are
 *     reentrant.  Buffers must stay valid until the stream has run the work.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; device faults surface at the caller's
 *     next synchronisation.
 *   - Validation is synchronous and complete before anything is enqueued: a
 *     call that returns an error has launched nothing.  The message of the
 *     last error on the calling thread is available from fa_last_error().
 *   - q, k, v and out share one layout and one 16-bit storage type.
 *       FA_BNSD: [B][N][S][D]    FA_BSND: [B][S][N][D]   (both contiguous)
 *       FA_TND:  [T][N][D], the B sequences packed end to end (developer
 *                guide 1.3); q_seq / kv_seq are then the totals Q_T / KV_T
 *                and cu_seqlens_q / cu_seqlens_kv give the boundaries.
 *     BSH is BSND with H = N*D.  Base pointers must be 16-byte aligned.
 *   - k and v are either contiguous in that layout (FA_KV_CONTIGUOUS) or a
 *     paged cache (FA_KV_PAGED_*, decode only; see fa_params.kv_layout).
 *   - Query head n1 reads KV head n1 / g with g = num_heads / num_kv_heads:
 *     g consecutive query heads share one KV head (FlashAttn developer guide,
 *     1.1 MHA and GQA).
 *   - lse is float32 [B][num_heads][q_seq] in BNSD and BSND and [Q_T][num_heads]
 *     in TND (developer guide 1.6 gives both shapes), natural log:
 *     lse = log(sum_j exp(s_j - m)) + m.
 *   - A row with no valid key (length 0, or every key masked) writes out = 0
 *     and lse = +inf (developer guide, 1.7 RowInvalid).
 *   - Output stores round to nearest even from fp32.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status classes after the aclnnIncreFlashAttention guide, section 4
 * (null-pointer, invalid-parameter and runtime error codes). */
typedef enum {
    FA_OK = 0,
    FA_ERR_NULLPTR = 1,        /* a required pointer is NULL */
    FA_ERR_PARAM_INVALID = 2,  /* shapes, sizes, options or alignment out of range */
    FA_ERR_UNSUPPORTED = 3,    /* valid on the pages but not built here (e.g. head_dim 192) */
    FA_ERR_RUNTIME = 4         /* the HIP runtime refused a launch */
} fa_status;

typedef enum { FA_BNSD = 0, FA_BSND = 1, FA_TND = 2 } fa_layout;
typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/* Mask modes (developer guide 1.5: 0 = none, 3 = causal, 4 = window; IFA
 * guide 4 and 8.1: a boolean attenMask whose true entries are excluded). */
typedef enum {
    FA_MASK_NONE = 0,
    FA_MASK_CAUSAL = 1,  /* key j > query i excluded (top-left aligned, absolute indices) */
    FA_MASK_BOOL = 2,    /* uint8 tensor, nonzero = excluded */
    FA_MASK_WINDOW = 3   /* band: key j kept iff i - win_left <= j <= i + win_right */
} fa_mask_mode;

/* KV cache storage (FlashAttn developer guide 1.2, PagedAttention, and its
 * layout_kv table): contiguous [B][KV_S][KV_N][D] / [B][KV_N][KV_S][D] as
 * set by `layout`, or fixed-size physical blocks indexed by a block table.
 *   FA_KV_PAGED_BBND: k, v are [num_blocks][block_size][KV_N][D] (BSND inside a block)
 *   FA_KV_PAGED_BNBD: k, v are [num_blocks][KV_N][block_size][D] (BNSD inside a block)
 * Token j of batch b lives in row j % block_size of physical block
 * block_table[b * max_blocks_per_seq + j / block_size].  q, out and lse keep
 * `layout`.  The NZ fractal block format of the pages is not provided. */
typedef enum {
    FA_KV_CONTIGUOUS = 0,
    FA_KV_PAGED_BBND = 1,
    FA_KV_PAGED_BNBD = 2
} fa_kv_layout;

typedef struct {
    int64_t batch;            /* B >= 1 */
    int64_t num_heads;        /* Q_N >= 1 */
    int64_t num_kv_heads;     /* KV_N; 0 means num_heads (IFA guide 4); must divide Q_N */
    int64_t q_seq;            /* Q_S >= 1 */
    int64_t kv_seq;           /* KV_S >= 1: the padded cache length */
    int64_t head_dim;         /* D: 64, 128 and 256 built */
    fa_layout layout;
    fa_dtype dtype;
    double scale;             /* softmax scale, finite (the pages default it to 1.0) */
    /* Device int64 [batch] actual KV lengths, or NULL (= kv_seq).  Each value
     * is clamped to [0, kv_seq] on the device; positions at or beyond it are
     * never read into the result, whatever they hold (IFA guide 1.1; developer
     * guide 1.4, the shorter length takes effect). */
    const int64_t *actual_seq_lengths;
    fa_mask_mode mask_mode;
    /* FA_MASK_BOOL only (must be NULL otherwise): device uint8 mask addressed as
     * mask[b*s0 + n1*s1 + i*s2 + j*s3] with mask_stride = {s0,s1,s2,s3} in
     * elements; a stride of 0 broadcasts that axis (e.g. (B,1,1,S) or (1,1,S,S)). */
    const uint8_t *mask;
    int64_t mask_stride[4];
    /* Paged KV cache (all zero / NULL for FA_KV_CONTIGUOUS, where a non-NULL
     * block_table is an error).  A paged cache needs actual_seq_lengths
     * (developer guide 1.2 makes the per-batch lengths mandatory with paging)
     * and a split-KV shape: q_seq == 1 without a mask or seqused_q (any
     * head_dim), or head_dim 64 / 128 with g * q_seq <= 512 (g = num_heads /
     * num_kv_heads, any mask); other paged calls return FA_ERR_UNSUPPORTED.
     *   block_table: device int32 [batch][max_blocks_per_seq], row-major.
     *     Entries of blocks a batch's length reaches must lie in
     *     [0, num_blocks); the kernels clamp them into that range so a bad
     *     entry reads a wrong block rather than out-of-bounds memory.
     *   block_size: tokens per block, a multiple of 16 in [16, 1024].
     *   max_blocks_per_seq >= 1, with kv_seq <= max_blocks_per_seq * block_size.
     *   num_blocks >= 1: physical blocks held by k and by v. */
    fa_kv_layout kv_layout;
    const int32_t *block_table;
    int64_t block_size;
    int64_t max_blocks_per_seq;
    int64_t num_blocks;
    /* FA_MASK_WINDOW: tokens kept before and after the query's own index
     * (developer guide 1.5, win_left / win_right); -1 leaves that side
     * unbounded, so (-1, 0) is the causal mask and (-1, -1) no mask.  Values
     * below -1 are invalid.  Tiles wholly outside the band are skipped.  In
     * every other mask mode both must be -1 (the guide requires it without a
     * window), else FA_ERR_PARAM_INVALID. */
    int64_t win_left;
    int64_t win_right;
    /* Device int32 (developer guide 1.4).  cu_seqlens_q and cu_seqlens_kv are
     * for FA_TND only (must be NULL otherwise); seqused_q applies to every
     * layout.
     *   cu_seqlens_q, cu_seqlens_kv: [batch + 1], starting at 0 and
     *     non-decreasing; sequence b owns q rows [cu_q[b], cu_q[b+1]) and kv
     *     rows [cu_kv[b], cu_kv[b+1]); cu_q[batch] <= q_seq, cu_kv[batch] <= kv_seq.
     *     The kernels clamp every offset into its tensor, so malformed values
     *     give wrong rows, never out-of-bounds accesses.
     *   seqused_q: [batch] or NULL: query rows of batch / sequence b
     *     actually used; the shorter of it and q_seq (the sequence length in
     *     TND) takes effect.  Rows at or past it are written as 0 with
     *     lse = +inf, in every layout.
     * actual_seq_lengths (int64) truncates each sequence's keys the same way.
     * Query rows not used by any sequence (past seqused_q, or past
     * cu_seqlens_q[batch]) are written as 0 with lse = +inf, the output
     * initialisation the developer guide describes.  TND always runs the
     * prefill kernel, needs batch <= 16383 and a workspace of
     * fa_workspace_size bytes for its work list, and no paged cache. */
    const int32_t *cu_seqlens_q;
    const int32_t *cu_seqlens_kv;
    const int32_t *seqused_q;
} fa_params;

/* fa_workspace_size -- phase 1 of fa_fwd (the two-phase shape of the IFA guide,
 * section 3): bytes of device workspace fa_fwd needs for *p (0 when none).
 * Also picks the split plan fa_fwd will use for q_seq == 1, for the device
 * that is current on the calling thread: fa_splitkv_plan's fixed chunks, or,
 * for 4 to 32 query heads per KV head (head_dim 64 or 128) with
 * actual_seq_lengths, pieces balanced over the actual lengths (derived on the
 * device). */
fa_status fa_workspace_size(const fa_params *p, size_t *bytes);

/* fa_fwd -- phase 2: the attention forward.  q: [B,Q_N,Q_S,D] or [B,Q_S,Q_N,D];
 * k, v: the same layout with KV_N heads and KV_S rows; out: shape of q;
 * lse: float32 [B,Q_N,Q_S] or NULL (not written).  The split-KV path
 * (FlashAttn developer guide 1.9: FlashDecode cuts the KV axis when the
 * query rows alone cannot occupy the cores, e.g. S1 = 1) runs
 *   - q_seq == 1 without a mask or seqused_q (any head_dim), and q_seq == 1
 *     with a boolean mask of unit key stride on a contiguous cache (any
 *     head_dim);
 *   - with head_dim 64 or 128 and g * q_seq <= 512: q_seq == 1 with any
 *     mask or seqused_q (the decode of the IFA guide with its attenMask),
 *     a paged cache, and a few query positions against a long cache when
 *     the prefill's query tiles would occupy fewer workgroups than there
 *     are CUs and a row can see at least 640 keys (1024 at head_dim 64; the causal mask is
 *     top-left, so a causal row sees at most q_seq of them);
 * with a split plan the library chooses (see fa_splitkv_plan): one split is
 * a single stage-1 launch that writes the output; more run stage 1 and then
 * fa_combine's kernel (measured faster on MI355X than the fused single
 * launch of fa_decode_fused).  The workspace must then be at least
 * fa_workspace_size bytes, 256-byte aligned; its contents need no
 * initialisation.  Every other case runs the prefill kernels.  The packed layout FA_TND needs
 * fa_workspace_size bytes (256-byte aligned) for the cost-ordered list of its
 * query tiles.  A boolean mask whose rows are contiguous, 16-byte aligned key
 * runs (mask_stride[3] == 1; the pointer, the other strides and kv_seq
 * multiples of 16) takes an optional workspace of fa_workspace_size bytes:
 * given one (256-byte aligned, else FA_ERR_PARAM_INVALID, as for one too
 * small), a first kernel summarises the mask per tile of 128 query rows x 64
 * keys (any key visible, any key masked) and the prefill then skips the tiles
 * the mask hides entirely, as the developer guide (1.5) does for the window
 * mode; with workspace NULL it visits every tile.  The results are the same
 * either way.  Other prefill cases take no workspace (it is ignored). */
fa_status fa_fwd(const fa_params *p, const void *q, const void *k, const void *v,
                 void *out, float *lse, void *workspace, size_t workspace_bytes,
                 void *stream);

/* fa_splitkv_plan -- the split-count heuristic (IFA guide 8.2: split the KV
 * axis when B*KV_N is below 0.4 x the core count; FlashDecoding tutorial,
 * preface: cut the cache so every core has a piece).  Host-side work: the
 * target is as many stage-1 workgroups as the CUs hold at once, from the HIP
 * occupancy calculator for the instantiation that will run (4 per CU when no
 * device answers), so the stage-1 grid is one round.
 *   num_cus: compute units to fill (<= 0: query the current device).
 *   chunk_hint: tokens per split, a positive multiple of 64, or 0 = automatic.
 * Returns num_splits >= 1 and chunk (a multiple of 64) with
 * num_splits * chunk >= kv_seq, and the workspace bytes of the partials
 * (o_part, m_part, l_part below) for that plan. */
fa_status fa_splitkv_plan(const fa_params *p, int num_cus, int64_t chunk_hint,
                          int64_t *num_splits, int64_t *chunk, size_t *workspace_bytes);

/* fa_decode_splitkv -- FlashDecoding stage 1 (FlashDecoding tutorial 3.2;
 * FlashAttn developer guide 10).  Takes q_seq == 1 without a mask or
 * seqused_q (any head_dim), q_seq == 1 with a boolean mask of unit key
 * stride on a contiguous cache (any head_dim), or, with head_dim 64 / 128
 * and g * q_seq <= 512, any q_seq, mask and seqused_q (else
 * FA_ERR_UNSUPPORTED).  Chunk c covers keys [c*chunk, (c+1)*chunk) cut at
 * the batch's length.  For every row (b, n1, i) and chunk c it writes, over
 * the keys of the chunk the row sees (mask, length, seqused_q),
 *   m_part = max_j s_j,  l_part = sum_j exp(s_j - m_part),
 *   o_part[d] = sum_j exp(s_j - m_part) v_j[d]    (NOT divided by l_part)
 * with s_j = scale * q.k_j, natural units.  A chunk the row sees no key of
 * writes m = -inf, l = 0 and o = 0.  Layouts (float32, contiguous; row
 * (b, n1, i) = (b * Q_N + n1) * q_seq + i):
 *   o_part [B][Q_N][q_seq][num_splits][D] (16-byte aligned),
 *   m_part and l_part [B][Q_N][q_seq][num_splits] (4-byte aligned).
 * num_splits * chunk must cover kv_seq; chunk a positive multiple of 64
 * and at most a cap (a paged cache: 1016 * block_size, the block ids of one
 * chunk being staged on chip; a contiguous one: (chunk + 256) rows of one
 * head within 2^31 bytes, the K/V offsets being 32-bit); fa_splitkv_plan
 * respects both.  With 4 to 32 query heads per KV head and head_dim 64 or
 * 128 (contiguous or paged cache), the chunk runs on the matrix cores (the
 * query heads of a KV head are the rows of one tile; P is rounded to the input
 * type before the PV product, as in the prefill; chunks of at most 512 tokens
 * run on one-wave workgroups, longer ones on two-wave workgroups), and so
 * does every call with several query positions, a mask or seqused_q; other
 * shapes use the vector units. */
fa_status fa_decode_splitkv(const fa_params *p, int64_t num_splits, int64_t chunk,
                            const void *q, const void *k, const void *v,
                            float *o_part, float *m_part, float *l_part, void *stream);

/* fa_decode_fused -- FlashDecoding in ONE launch (FlashAttn developer guide:
 * the FD block and the FA/FD overlap, whose SyncAll this replaces).  Stage 1
 * as in fa_decode_splitkv, writing its partials into `workspace`; the last
 * workgroup to finish a (batch, KV head, head group) unit merges that unit's
 * rows (fa_combine's reduction) into out / lse and resets the unit's counter.
 *   num_splits: 1..256 (1 = one chunk, no merge and no workspace needed);
 *   chunk as for fa_decode_splitkv.
 * Takes q_seq == 1 without a mask or seqused_q (else FA_ERR_UNSUPPORTED).
 *   workspace: at least the bytes fa_decode_fused_plan reports, 256-byte aligned:
 *     o_part, m_part, l_part (fa_decode_splitkv's layouts, each region
 *     256-byte aligned) followed by one uint32 counter per unit.  CONTRACT:
 *     the counters must be zero before the first call -- zero-fill the
 *     workspace once after allocating it; every completed call leaves them
 *     zero, so the same workspace can be reused (also from a captured graph)
 *     without clearing.  Calls that share a workspace must not overlap.
 * On MI355X this is slower than stage 1 + fa_combine (the merging workgroup's
 * device-coherent reads cost more than the second launch), so fa_fwd does not
 * use it. */
fa_status fa_decode_fused(const fa_params *p, int64_t num_splits, int64_t chunk,
                          const void *q, const void *k, const void *v, void *workspace,
                          size_t workspace_bytes, void *out, float *lse, void *stream);

/* fa_decode_fused_plan -- the split plan for fa_decode_fused: as
 * fa_splitkv_plan, but sized for the vector stage 1 that the fused launch
 * runs (its residency and its units of batch, KV head and head group) and
 * capped at the fused merge's 256 splits (the chunk grows instead).
 * num_cus <= 0 queries the current device.  Returns FA_ERR_UNSUPPORTED for
 * shapes fa_decode_fused does not take, or when 256 chunks of the largest
 * chunk cannot cover kv_seq. */
fa_status fa_decode_fused_plan(const fa_params *p, int num_cus, int64_t *num_splits, int64_t *chunk,
                               size_t *workspace_bytes);

/* fa_combine -- FlashDecoding stage 2, the LSE merge (FlashAttn developer
 * guide 10: m = max_i m_i, l = sum_i l_i exp(m_i - m),
 * o = sum_i o_i exp(m_i - m) / l; FlashDecoding tutorial section 2).  Reads the
 * stage-1 layouts above (any q_seq; o_part 16-byte aligned) and writes out
 * (shape of q, in p's layout and dtype) and lse (nullable, [B][Q_N][Q_S])
 * = log l + m.  Splits with m_i = -inf are skipped; a row whose splits are
 * all empty writes 0 and +inf. */
fa_status fa_combine(const fa_params *p, int64_t num_splits, const float *o_part,
                     const float *m_part, const float *l_part, void *out, float *lse,
                     void *stream);

/* fa_fwd_noalloc -- fa_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments and results as fa_fwd without the workspace:
 * the paths that need one (split-KV partials, the packed-layout work list,
 * the boolean-mask summary) use a scratch array of 16 MiB that the library
 * holds on each GPU from the time the library is loaded until the process
 * ends.  The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); on its first call on a device it looks up
 * that device's scratch address (hipGetSymbolAddress, with the device
 * current) and keeps it.  A call whose fa_workspace_size exceeds 16 MiB
 * returns FA_ERR_PARAM_INVALID and launches nothing.  The scratch needs no
 * initialisation, but every call on one GPU shares it: calls that may
 * overlap on one device (several streams or threads) race and must be
 * serialised by the caller. */
fa_status fa_fwd_noalloc(const fa_params *p, const void *q, const void *k, const void *v,
                         void *out, float *lse, void *stream);

/* fa_describe -- one line of text naming what fa_fwd would launch for p: the
 * path (prefill, decode, general split), each kernel with its instantiation
 * <dtype, head dim, mask kind> and grid, the split plan, and the workspace
 * bytes (as fa_workspace_size).  The FlashAttn page's Quick Start finds the
 * kernel variant a case launched (its tiling key) in the run logs; this is
 * the same information for this library.  With the environment variable
 * FA_LOG set (and not "0"), fa_fwd prints this line to stderr before it
 * launches.  buf receives at most buf_bytes bytes, NUL-terminated (longer
 * text is cut).  Validates p like fa_fwd; reads no device memory and
 * launches nothing (on a host without a GPU the plan assumes 256 CUs). */
fa_status fa_describe(const fa_params *p, char *buf, size_t buf_bytes);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char *fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
