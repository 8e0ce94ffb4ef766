/*
 * fa_fwd.h -- exact tiled-softmax attention forward pass on MI355X (gfx950).
 *
 * The operation: for every batch b, head h and query row i,
 *     s_ij   = scale * (q_i . k_j)                 over the allowed keys j
 *     o_i    = sum_j softmax_j(s_i) v_j
 *     lse_i  = ln sum_j exp(s_ij)                  (the per-row log-sum-exp)
 * i.e. O = softmax(Q K^T * scale) V, as defined on "FlashAttention tiles exact
 * softmax without materializing the score matrix" (nalar.dev, opening
 * definition) and, per query, on "transformer math: flash attention math"
 * (aicassindra.com, section "What we must compute, and why storage is the
 * problem"). The library evaluates it tile by tile with the online-softmax
 * recurrence (running max, running denominator, unnormalised accumulator,
 * rescale factor exp(m_old - m_new)) so the N x N score and probability
 * matrices never reach device memory (same aicassindra.com page, "The
 * block-wise update, and the full algorithm"). lse is the compact per-row
 * statistic a backward pass recomputes from ("Decoding flash attention",
 * bibekananda.in, section "The backward pass").
 *
 * Allowed keys: every j in [0, N), or only j <= i when causal != 0 (square,
 * top-left aligned; nalar.dev, "Causal masking fits inside the tiled
 * computation"). Every row keeps at least key 0, so no row is empty.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "fa_types.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Tuning options for fa_fwd_ex. They change how the result is reached, never
 * what it is (the same exact softmax attention, up to rounding).
 *
 * rescale_threshold_log2 (f16 only): the online recurrence keeps every partial
 *   sum relative to a reference maximum m and rescales them by
 *   alpha = exp(m_old - m_new) when m moves ("transformer math: flash
 *   attention math", aicassindra.com, "The rescaling identity, derived").
 *   With 0 the reference is the running maximum at every step, the loop
 *   exactly as that page writes it ("The block-wise update, and the full
 *   algorithm"). With t > 0 it moves only when needed to keep every
 *   unnormalised probability <= 2^t, and then to t/2 above the running
 *   maximum, so most tiles skip the rescale ("fewer rescaling operations",
 *   "Decoding flash attention", bibekananda.in, "Later versions"). The
 *   kernel tests this on the sums of each tile's probabilities that the
 *   recurrence forms anyway: when a sum exceeds 2^t (which any score more
 *   than t above the reference makes happen) the wave moves the reference
 *   and recomputes that tile. Range [0, 15]; fa_fwd uses 8. bf16 ignores
 *   it and always keeps the exact running maximum: a probability rounded to
 *   bf16 (8 significant bits) is off by up to 2^-8 of itself, and only
 *   against the exact maximum is a row's largest weight exactly 1.
 * variant: which kernel evaluates it; 0 = the default, 1 = the same kernel
 *   named explicitly (32 query rows per wave, two waves per SIMD). Range
 *   [0, 1].
 */
typedef struct fa_fwd_options {
    float rescale_threshold_log2;
    int variant;
} fa_fwd_options;

/*
 * fa_fwd -- enqueue the attention forward pass on `stream`.
 *
 * q, k, v : device pointers, contiguous row-major [B, H, N, d] of `dtype`.
 * o       : device pointer, contiguous [B, H, N, d] of `dtype`; receives the
 *           output rounded to nearest-even from fp32.
 * lse     : device pointer, contiguous [B, H, N] fp32, or NULL to skip it;
 *           receives ln sum_j exp(s_ij) in natural-log units.
 * B, H, N : batch, heads, sequence length (queries = keys = N). Each >= 1,
 *           B*H*ceil(N/256) <= 2^31 - 1 and N*d*2 < 2^31 (one head of one
 *           tensor under 2 GiB; N <= 8388607 at d = 128).
 * d       : head dimension, 64 or 128.
 * scale   : logit multiplier (1/sqrt(d) is the usual choice); finite, > 0.
 * causal  : non-zero excludes key j from query i when j > i.
 * stream  : HIP stream (0 = the null stream). The call only enqueues work and
 *           returns; the caller synchronises.
 * dtype   : an fa_dtype value (the element type cannot be read off a void*).
 *
 * Ownership: the caller allocates and frees every buffer; the library
 * allocates nothing, keeps no state between calls and uses no workspace, so
 * calls are re-entrant and thread-safe. o and lse must not overlap q, k, v
 * or each other. Numerics: products accumulate in fp32 on the matrix cores;
 * the probabilities are rounded to `dtype` as the second product's operand;
 * the running statistics are fp32. The denominator (O's normaliser and the
 * argument of lse's logarithm) sums the rounded probabilities in f16 and the
 * unrounded fp32 ones in bf16.
 * Errors: see fa_status. Device faults surface at the caller's next
 * synchronisation.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t N, int64_t d,
           float scale, int causal, hipStream_t stream, fa_dtype dtype);

/*
 * fa_fwd_ex -- fa_fwd with tuning options (see fa_fwd_options). opts == NULL
 * gives exactly fa_fwd. Same arguments, layouts, ownership, synchronisation
 * and errors as fa_fwd, plus FA_ERR_OPTION for an out-of-range option.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int64_t B, int64_t H, int64_t N, int64_t d,
              float scale, int causal, hipStream_t stream, fa_dtype dtype,
              const fa_fwd_options* opts);

/*
 * A general mask for fa_fwd_masked. Key j is allowed for query i (of batch b) when
 *   window_left  < 0  or  j >= i - window_left,
 *   window_right < 0  or  j <= i + window_right,     and
 *   seqlens_k == NULL or  j <  seqlens_k[b].
 * window_left = -1, window_right = 0 is the causal mask; a window of w keys back and none ahead
 * is sliding-window (local) attention; seqlens_k is key padding (per-batch key lengths). The pages
 * admit any mask applied to every score tile before the max ("FlashAttention tiles exact
 * softmax without materializing the score matrix", nalar.dev, "Causal masking fits inside the
 * tiled computation", last paragraph; "transformer math: flash attention math",
 * aicassindra.com, "Pitfalls in implementing the recurrence": masked scores are -inf before the
 * block max). A row with no allowed key has no softmax: its output is 0 and its lse -inf.
 */
typedef struct fa_mask {
    int64_t window_left;       /* -1 (no limit) or 0 .. 2^31 - 1 */
    int64_t window_right;      /* -1 (no limit) or 0 .. 2^31 - 1 */
    const int32_t* seqlens_k;  /* NULL, or device pointer to B int32 key lengths (4-byte aligned);
                                  values are clamped to [0, N] on the device */
} fa_mask;

/*
 * fa_fwd_masked -- fa_fwd under a general mask (see fa_mask). Key tiles outside a query tile's
 * window are neither loaded nor computed, so a window of w keys costs O(N w), not O(N^2).
 * Arguments as for fa_fwd, with `causal` replaced by `mask` (not NULL). A window of N - 1 or more
 * keys excludes nothing and is taken as -1; the masks -1/-1 and -1/0 without seqlens_k then run
 * fa_fwd's own kernels. The masked kernel runs with 128-row workgroups at d = 64 and for windows
 * of at most 2048 keys (window_left + window_right + 1), else with 256-row ones (the same
 * results). Errors: those of fa_fwd; FA_ERR_NULL for a NULL mask, FA_ERR_OPTION for a window out
 * of range, FA_ERR_ALIGN for a misaligned seqlens_k.
 */
int fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t H, int64_t N, int64_t d,
                  float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask);

/*
 * A mask over blocks of the score matrix (block-sparse attention) for fa_fwd_blocksparse. Query i
 * lies in query block i / block_q, key j in key block j / block_k; the pair is allowed only when
 *   mask[b * stride_b + h * stride_h + (i / block_q) * n_kb + j / block_k] != 0,
 * n_kb = ceil(N / block_k), n_qb = ceil(N / block_q). Any mask applied to the scores before the
 * max keeps the method exact ("Causal masking fits inside the tiled computation", nalar.dev, last
 * paragraph); one given per block lets whole tiles be skipped.
 */
typedef struct fa_block_mask {
    const uint8_t* mask;  /* device pointer; the caller's buffer holds every byte addressed:
                             (B-1)*stride_b + (H-1)*stride_h + n_qb*n_kb bytes at least */
    int64_t block_q;      /* query rows per block: a positive multiple of 64 */
    int64_t block_k;      /* keys per block: a positive multiple of 64 */
    int64_t stride_b;     /* bytes between the masks of consecutive batches (0: shared) */
    int64_t stride_h;     /* bytes between the masks of consecutive heads (0: shared) */
} fa_block_mask;

/*
 * fa_fwd_blocksparse -- fa_fwd under a block mask (see fa_block_mask), optionally combined with
 * the window and key lengths of fa_mask (`mask` may be NULL: no further restriction; causal is
 * window_left = -1, window_right = 0). Each 256-row query tile loads and computes only the 64-key
 * tiles that one of its 32-row groups needs; a row with no allowed key gets o = 0, lse = -inf.
 * Arguments as for fa_fwd_masked, plus `blocks` (not NULL). Errors: those of fa_fwd_masked;
 * FA_ERR_NULL for a NULL `blocks` or blocks->mask, FA_ERR_OPTION for a block size that is not a
 * positive multiple of 64 or a negative stride. Any N that fa_fwd takes: the list of a query
 * tile's key tiles is built 1024 candidates at a time.
 */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t N, int64_t d,
                       float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask,
                       const fa_block_mask* blocks);

/*
 * fa_fwd_splitkv -- fa_fwd with the keys of every query tile cut into num_splits runs that run
 * as separate workgroups (split-KV), for shapes whose B*H*ceil(N/256) query tiles leave compute
 * units idle. Each split writes a partial result -- its output normalised over its own keys, in
 * fp32, and the log-sum-exp of its logits -- to `workspace`; a second kernel merges them with the
 * rescaling identity ("transformer math: flash attention math", aicassindra.com, "The rescaling
 * identity, derived"): lse = ln sum_s exp(L_s), o = sum_s exp(L_s - lse) o_s. By that page's
 * "Proof of exactness" the grouping of the keys does not change the result, which is that of
 * fa_fwd up to rounding.
 *
 * Arguments as for fa_fwd, plus:
 * num_splits      : 1 .. 64 (1 is exactly fa_fwd and needs no workspace);
 *                   fa_fwd_splitkv_heuristic suggests a value.
 * workspace       : device memory of at least fa_fwd_splitkv_workspace_size(B, H, N, d,
 *                   num_splits) bytes, 16-byte aligned, not overlapping q, k, v, o or lse. The
 *                   caller owns it; its contents before and after the call are unspecified, and
 *                   two calls in flight at once need two workspaces.
 * Errors: those of fa_fwd, FA_ERR_OPTION for num_splits out of range, FA_ERR_WORKSPACE.
 * Uses the default kernel and rescale threshold of fa_fwd.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d,
                   float scale, int causal, hipStream_t stream, fa_dtype dtype,
                   int num_splits, void* workspace, size_t workspace_bytes);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same kernels, with
 * the partial results kept in a fixed scratch array of the library instead of a caller workspace.
 * It calls no hipMalloc, hipFree or other allocating routine.
 *
 * Arguments, layouts and results as for fa_fwd_splitkv without the workspace arguments; num_splits
 * 1 .. 64 (1 is exactly fa_fwd). The partials must fit the scratch:
 * fa_fwd_splitkv_workspace_size(B, H, N, d, num_splits) <= 64 MiB, i.e. B*H*N*(d+2)*num_splits
 * <= 2^24 (at 2 splits: 64 527 rows B*H*N of d = 128, 127 100 of d = 64); larger problems return
 * FA_ERR_SCRATCH before any device work. Each GPU holds its own 64 MiB array from the library's
 * first use there until the process ends (its address is looked up once per device, on the first
 * call with that device current). All calls on one GPU share that array: calls that overlap on
 * one GPU (two streams, two threads) race and give wrong results; serialise them. Its contents
 * between calls are unspecified.
 * Errors: those of fa_fwd_splitkv except FA_ERR_WORKSPACE, plus FA_ERR_SCRATCH.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d,
                           float scale, int causal, hipStream_t stream, fa_dtype dtype,
                           int num_splits);

/*
 * fa_fwd_splitkv_masked -- fa_fwd_masked with split-KV: the key tiles a query tile's window
 * reaches (fa_mask: sliding window and per-batch key lengths) are cut into num_splits runs, each
 * reduced by its own workgroup and merged as in fa_fwd_splitkv. A run may hold no allowed key of
 * some row (or none at all): its partial result has weight 0 in the merge, and a row no split
 * holds a key of gets o = 0 and lse = -inf, as in fa_fwd_masked.
 * Arguments as for fa_fwd_masked plus num_splits, workspace and workspace_bytes as for
 * fa_fwd_splitkv (the same workspace size). The masks -1/-1 and -1/0 without seqlens_k run
 * fa_fwd_splitkv, and num_splits = 1 runs fa_fwd_masked. Errors: those of fa_fwd_masked and
 * fa_fwd_splitkv.
 */
int fa_fwd_splitkv_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask,
                          int num_splits, void* workspace, size_t workspace_bytes);

/*
 * fa_fwd_splitkv_blocksparse -- fa_fwd_blocksparse with split-KV: the key tiles a query tile's
 * window reaches are cut into num_splits equal runs, as in fa_fwd_splitkv_masked; each run's
 * workgroup lists and computes only the tiles of its run that the block mask (and window and key
 * lengths) leave to one of its 32-row groups, and the runs are merged by the rescaling identity as
 * in fa_fwd_splitkv. Splitting the keys before applying the mask, not the list of needed tiles,
 * keeps the split of every query tile the same for one call; a run whose tiles the mask removes
 * costs one empty workgroup and adds weight 0 in the merge. Rows with no allowed key get o = 0,
 * lse = -inf.
 * Arguments as for fa_fwd_blocksparse plus num_splits, workspace and workspace_bytes as for
 * fa_fwd_splitkv (the same workspace size); num_splits = 1 runs fa_fwd_blocksparse. Errors: those
 * of fa_fwd_blocksparse and fa_fwd_splitkv.
 */
int fa_fwd_splitkv_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t B, int64_t H, int64_t N, int64_t d,
                               float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask,
                               const fa_block_mask* blocks, int num_splits, void* workspace,
                               size_t workspace_bytes);

/* Bytes of workspace fa_fwd_splitkv (and fa_fwd_splitkv_masked, fa_fwd_splitkv_blocksparse) needs:
 * num_splits * B*H*N * (d + 2) * 4, or 0 when num_splits <= 1 or an argument is out of range. */
size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int num_splits);

/* A split count for fa_fwd_splitkv from a cost model: one workgroup of 256 query rows runs per
 * compute unit at a time, so G = B*H*ceil(N/256) tiles cut in S splits take ceil(G*S/256) rounds
 * of 1/S of the key tiles (plus a fixed start-up cost per workgroup), and the merge reads S
 * partial results per row. At least four key tiles of 64 per split (half as many keys counted
 * when causal), at most 64; 1 when splitting cannot help. */
int fa_fwd_splitkv_heuristic(int64_t B, int64_t H, int64_t N, int64_t d, int causal);

/* Static, NUL-terminated description of a return code (never NULL). */
const char* fa_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
