/*
 * fa_bwd.h -- backward pass of exact attention on MI355X (gfx950).
 *
 * Given the forward inputs q, k, v, its output o and per-row log-sum-exp lse
 * (from fa_fwd), and the gradient dout = dL/do of some loss L, fa_bwd returns
 * dq, dk, dv = dL/dq, dL/dk, dL/dv. With p_ij = exp(s_ij - lse_i) the softmax
 * weights of the forward pass (s_ij = scale * q_i . k_j over the allowed keys):
 *     dP_ij = dout_i . v_j
 *     D_i   = dout_i . o_i                   (= sum_j p_ij dP_ij)
 *     dS_ij = p_ij (dP_ij - D_i)
 *     dv_j  = sum_i p_ij dout_i
 *     dk_j  = scale * sum_i dS_ij q_i
 *     dq_i  = scale * sum_j dS_ij k_j
 * (the chain rule through the definition of fa_fwd.h). As the pages describe
 * for the backward pass, only the compact per-row statistic is kept from the
 * forward pass and the score tiles are recomputed from q, k and lse, so no
 * N x N matrix reaches device memory ("Decoding flash attention",
 * bibekananda.in, section "The backward pass"; "FlashAttention tiles exact
 * softmax without materializing the score matrix", nalar.dev, section
 * "Backward computation can trade recomputation for stored intermediates").
 * Allowed keys and the causal convention are those of fa_fwd.h.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include "fa_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_bwd -- enqueue the attention backward pass on `stream`.
 *
 * q, k, v, o, dout : device pointers, contiguous row-major [B, H, N, d] of
 *                    `dtype`, 16-byte aligned; o is fa_fwd's output for the
 *                    same q, k, v, scale and causal.
 * lse              : device pointer, contiguous [B, H, N] fp32, fa_fwd's
 *                    per-row log-sum-exp (natural log); 4-byte aligned.
 * dq, dk, dv       : device pointers, contiguous [B, H, N, d] of `dtype`,
 *                    16-byte aligned; receive the gradients, rounded to
 *                    nearest-even from fp32.
 * delta            : device pointer, contiguous [B, H, N] fp32, 4-byte
 *                    aligned; receives D_i = dout_i . o_i (the backward pass
 *                    computes it first and reads it back; the caller may
 *                    reuse the buffer after the call completes).
 * B, H, N, d, scale, causal, stream, dtype : as for fa_fwd, with the same
 *                    limits (d = 64 or 128; B*H*ceil(N/256) <= 2^31 - 1;
 *                    N*d*2 < 2^31).
 *
 * Ownership: the caller allocates and frees every buffer; the library
 * allocates nothing and keeps no state between calls. dq, dk, dv and delta
 * must not overlap each other or any input. Every output element is written
 * by exactly one thread with a fixed order of summation, so repeated calls
 * give bit-identical results.
 * Numerics: products accumulate in fp32 on the matrix cores; p and dS are
 * rounded to `dtype` as operands of the products that consume them.
 * Errors: the fa_status codes of fa_fwd.h (FA_ERR_NULL for any NULL pointer,
 * FA_ERR_ALIGN, FA_ERR_ALIAS for an overlapping output, ...), all returned
 * before any device work except FA_ERR_LAUNCH. Device faults surface at the
 * caller's next synchronisation.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse,
           void* dq, void* dk, void* dv, float* delta,
           int64_t B, int64_t H, int64_t N, int64_t d,
           float scale, int causal, hipStream_t stream, fa_dtype dtype);

/*
 * fa_bwd_masked -- fa_bwd under the general mask of fa_fwd_masked (fa_mask in fa_fwd.h: a
 * sliding window and per-batch key lengths). The chain rule is unchanged; every sum runs over
 * the allowed pairs only, since a masked score carries no probability ("Causal masking fits
 * inside the tiled computation", nalar.dev: the mask applies before the max, so masked entries
 * have p = 0 and add nothing). `o` and `lse` are those fa_fwd_masked returned under the same
 * mask; a row with no allowed key (lse = -inf) gets dq = 0 and delta = 0, and a key no row
 * allows gets dk = dv = 0. Only the tiles inside each workgroup's window are loaded.
 * Arguments as for fa_bwd, with `causal` replaced by `mask` (not NULL); the masks -1/-1 and
 * -1/0 without seqlens_k run fa_bwd's own kernels. Errors: those of fa_bwd; FA_ERR_NULL for a
 * NULL mask, FA_ERR_OPTION for a window out of range, FA_ERR_ALIGN for a misaligned seqlens_k.
 */
int fa_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, float* delta,
                  int64_t B, int64_t H, int64_t N, int64_t d,
                  float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask);

/*
 * fa_bwd_blocksparse -- fa_bwd under the block mask of fa_fwd_blocksparse (fa_block_mask in
 * fa_fwd.h), optionally combined with a window and key lengths (`mask` may be NULL). The sums of
 * the chain rule run over the allowed pairs only: a block the mask drops holds no probability,
 * so it adds nothing to any gradient (the same reading of "Causal masking fits inside the tiled
 * computation", nalar.dev, as for fa_bwd_masked). `o` and `lse` are those fa_fwd_blocksparse
 * returned under the same masks. Each dQ workgroup (256 rows) loads only the 64-key tiles one of
 * its 32-row groups needs, and each dK/dV workgroup (128 keys) only the 64-row query tiles one of
 * its 32 x 32 pairs of rows and keys needs. A row with no allowed key gets dq = 0 and delta = 0,
 * a key no row allows dk = dv = 0.
 * Arguments as for fa_bwd_masked, plus `blocks` (not NULL); `mask` may be NULL.
 * Errors: those of fa_bwd_masked; FA_ERR_NULL for a NULL `blocks` or blocks->mask,
 * FA_ERR_OPTION for a block size that is not a positive multiple of 64 or a negative stride.
 * Any N that fa_bwd takes: the work lists are built 1024 tiles at a time.
 */
int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse,
                       void* dq, void* dk, void* dv, float* delta,
                       int64_t B, int64_t H, int64_t N, int64_t d,
                       float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask,
                       const fa_block_mask* blocks);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
