/*
 * block_sum.h -- C ABI of the block all-reduce sum in librmsnorm.so: the sum
 * of every element of a device tensor, on MI355X (gfx950).
 *
 * The operation follows page "Block All Reduce CUDA代码学习" (leetCUDA
 * reduce): one scalar, the sum of all n elements; narrow storage is widened
 * before it is accumulated (its "acc dtype" discussion: store narrow,
 * accumulate wide), fp8 is decoded first, and int8 is accumulated in int32.
 * Here floating inputs (f32, f16, bf16, OCP fp8 E4M3 and E5M2) accumulate in
 * fp32 and int8 in int32 (wrapping modulo 2^32 as int32 addition does).
 *
 * Result and reproducibility: each workgroup sums a fixed set of elements in
 * a fixed order, and the last workgroup to finish adds the per-workgroup
 * partial sums in index order, so the fp32 result is identical from run to
 * run for the same n and the same base address (the split into head, 16-byte
 * chunks and tail depends on the address).  The fp32 result differs from the
 * exact sum by at most (m + 64) * 2^-24 * sum|x| with m = max(33, n*S/2^21 + 1)
 * * (16/S) elements added by one thread in sequence (S = element bytes): the
 * depth of its summation tree.  The int8 result is exact modulo 2^32.
 *
 * Conventions (shared with rmsnorm.h, whose RMSN_* codes and
 * rmsnorm_strerror / rmsnorm_last_error apply):
 *   - x and out are DEVICE pointers; x holds n contiguous elements and must
 *     be aligned to its element size; out receives one float (floating
 *     dtypes) or one int32_t (BRS_I8).
 *   - workspace: a DEVICE buffer of at least BRS_WORKSPACE_BYTES bytes,
 *     16-byte aligned, owned by the caller.  Its first BRS_WORKSPACE_HEADER
 *     bytes (completion counters) must be zero before its first use:
 *     allocate it zeroed; every call leaves them zero again.  Calls that
 *     share a workspace must be ordered on one stream.
 *   - The call enqueues one kernel on `stream` (NULL: the default stream),
 *     allocates nothing and does not synchronise.  Arguments are validated
 *     before the launch; on error nothing is launched.
 *   - n == 0 writes 0 to out.
 */
#ifndef BLOCK_SUM_H
#define BLOCK_SUM_H

#include <stdint.h>

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BRS_F32 = 0,
  BRS_F16 = 1,
  BRS_BF16 = 2,
  BRS_FP8_E4M3 = 3, /* OCP E4M3: bias 7, no infinities, S.1111.111 is NaN */
  BRS_FP8_E5M2 = 4, /* OCP E5M2: bias 15, IEEE-style infinities and NaNs  */
  BRS_I8 = 5
} brs_dtype;

/* Workgroups per launch never exceed BRS_MAX_GROUPS; the workspace holds a
 * header of completion counters and one 4-byte partial per workgroup. */
#define BRS_MAX_GROUPS 2048
#define BRS_WORKSPACE_HEADER 4608
#define BRS_WORKSPACE_BYTES (BRS_WORKSPACE_HEADER + 4 * BRS_MAX_GROUPS)

/*
 * block_all_reduce_sum -- *out = sum of x[0..n).  Returns RMSN_OK or
 * RMSN_ERR_NULL, RMSN_ERR_SHAPE (n < 0, x not aligned to its element size,
 * workspace too small or not 16-byte aligned), RMSN_ERR_DTYPE,
 * RMSN_ERR_ALIAS (out or workspace overlapping x or each other), or
 * RMSN_ERR_HIP.
 */
int block_all_reduce_sum(void* out, const void* x, int64_t n, int dtype, void* workspace,
                         int64_t workspace_bytes, void* stream);

/*
 * block_all_reduce_sum_noalloc -- block_all_reduce_sum with no workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The counters and per-workgroup partials live in a device array of
 * BRS_WORKSPACE_BYTES bytes inside the library, one copy per GPU (each GPU
 * the library runs on holds its copy until the process ends); the call
 * allocates and frees nothing.  Limit: none on n beyond the workspace
 * form's -- a launch uses at most BRS_MAX_GROUPS partials, which the array
 * holds.  The first call on a GPU also enqueues, ahead of the sum, a small
 * kernel that zeroes the array's counters; every sum leaves them zero again.
 * All calls on one GPU share that GPU's array: calls that may run at the
 * same time on one GPU (on different streams, or from threads without
 * ordering between them) race and give wrong sums; order them on one
 * stream.  out, x, n, dtype, stream and the return codes are as for
 * block_all_reduce_sum (RMSN_ERR_HIP also when the array's address cannot
 * be obtained).
 */
int block_all_reduce_sum_noalloc(void* out, const void* x, int64_t n, int dtype, void* stream);

/*
 * block_sum_tune -- for tuning and testing only: every later sum of this
 * process launches exactly `groups` workgroups (1..BRS_MAX_GROUPS); 0
 * restores the size rule.  Returns RMSN_OK or RMSN_ERR_SHAPE.
 */
int block_sum_tune(int groups);

#ifdef __cplusplus
}
#endif

#endif /* BLOCK_SUM_H */
