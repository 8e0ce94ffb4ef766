/*
 * fa_types.h -- element types and return codes shared by every entry point of the library
 * (fa_fwd.h, fa_bwd.h, fa_cpu.h). No HIP dependency.
 */
#ifndef FA_TYPES_H
#define FA_TYPES_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum fa_dtype {
    FA_F16 = 0,  /* IEEE binary16 */
    FA_BF16 = 1  /* bfloat16 */
} fa_dtype;

/* Return codes. Every code except FA_ERR_LAUNCH is returned before any work
 * starts, and nothing is written. */
typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* q, k, v or o is NULL */
    FA_ERR_SHAPE = 2,     /* B, H or N < 1, or a size beyond the entry point's limits */
    FA_ERR_HEAD_DIM = 3,  /* d is not 64 or 128 */
    FA_ERR_DTYPE = 4,     /* dtype is not FA_F16 or FA_BF16 */
    FA_ERR_ALIGN = 5,     /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
    FA_ERR_SCALE = 6,     /* scale is not finite and > 0 */
    FA_ERR_LAUNCH = 7,    /* a kernel launch (hipGetLastError) or a host thread failed */
    FA_ERR_ALIAS = 8,     /* o or lse overlaps an input, or o overlaps lse */
    FA_ERR_OPTION = 9,    /* an fa_fwd_options field or num_splits is out of range */
    FA_ERR_WORKSPACE = 10, /* fa_fwd_splitkv: workspace NULL, not 16-byte aligned, smaller than
                              fa_fwd_splitkv_workspace_size, or overlapping an argument */
    FA_ERR_SCRATCH = 11    /* fa_fwd_splitkv_noalloc: the partials exceed the fixed 64 MiB scratch */
} fa_status;

#ifdef __cplusplus
}
#endif

#endif /* FA_TYPES_H */
