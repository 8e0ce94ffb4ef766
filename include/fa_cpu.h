/*
 * fa_cpu.h -- the attention forward pass of fa_fwd.h on the host CPU, tiled the same way.
 *
 * "transformer math: flash attention math" (aicassindra.com, section "Why the same math matters
 * on a CPU") makes the point that the recurrence pays on a CPU for the same reason as on a GPU:
 * a small fast cache in front of slow memory. Tiling keeps the active score block (32 query rows
 * x 64 keys) and the running state (m, l and the unnormalised output o~ of each row) in cache
 * while keys and values stream through once per query tile, and the update is a max and two
 * scaled sums that run in SIMD lanes. This is that CPU variant: the same exact attention as
 * fa_fwd (the definition and causal convention of fa_fwd.h), computed in fp32 from f16/bf16
 * inputs, on host memory. It is a separate entry point for host data; the GPU entry points
 * never call it.
 */
#ifndef FA_CPU_H
#define FA_CPU_H

#include <stdint.h>

#include "fa_types.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_fwd_cpu -- attention forward on host memory.
 *
 * q, k, v     : host pointers, contiguous row-major [B, H, N, d] of `dtype`.
 * o           : host pointer [B, H, N, d] of `dtype`; receives the output rounded to nearest-even.
 * lse         : host pointer [B, H, N] fp32, or NULL; receives ln sum_j exp(s_ij).
 * B, H, N, d  : as for fa_fwd (d = 64 or 128; B*H*N*d*2 bytes must fit in memory).
 * scale       : logit multiplier, finite and > 0.
 * causal      : non-zero excludes key j from query i when j > i.
 * dtype       : FA_F16 or FA_BF16.
 * num_threads : worker threads; <= 0 uses every hardware thread. Each (head, query tile) is
 *               computed by one thread in a fixed order, so the result does not depend on it.
 *
 * Blocking: returns when o and lse are written. Ownership: the caller owns every buffer; o and
 * lse must not overlap the inputs or each other. Numerics: scores, probabilities and sums in
 * fp32 (no intermediate rounding to dtype); exp2 by range reduction and a polynomial (relative
 * error below 2e-7). Errors: fa_status codes (no alignment requirement on the host).
 */
int fa_fwd_cpu(const void* q, const void* k, const void* v, void* o, float* lse,
               int64_t B, int64_t H, int64_t N, int64_t d,
               float scale, int causal, fa_dtype dtype, int num_threads);

#ifdef __cplusplus
}
#endif

#endif /* FA_CPU_H */
