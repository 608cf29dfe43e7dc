/*
 * rmsnorm.h -- C ABI of librmsnorm.so: row-wise RMSNorm and the fused
 * "K partials + residual -> residual in place -> RMSNorm" form on MI355X
 * (gfx950) with hand-written HIP kernels.
 *
 * The operation (per row i of a contiguous row-major [rows, hidden] tensor):
 *   RMSNorm (page "RMSNorm kernel", section 1 Background: the PyTorch RMSNorm
 *   definition over the last dimension; section 2 "Abstraction": per-row sum
 *   of squares, mean, + eps, square root, then x_j * gamma_j / RMS):
 *       y_j = x_j * rsqrt(mean_j(x_j^2) + eps) * gamma_j
 *   Fused form (page "Tokenweave fused-RMSNorm-AR kernel", section "Code
 *   walkthrough": the reduced rank partials plus the residual are written
 *   back to the residual in place, and the stored row is normalised):
 *       acc_j = p0_j + p1_j + ... + p(K-1)_j + r_j   (binary32, this order)
 *       r_j  <- round_to_dtype(acc_j)                 (in place)
 *       y_j   = r_j * rsqrt(mean_j(r_j^2) + eps) * gamma_j
 *
 * Numerics: values are widened to fp32; the residual sum is a sequence of
 * binary32 adds seeded with p0, rounded once to the storage dtype (round to
 * nearest even), so the stored residual is exactly reproducible.  The sum of
 * squares is accumulated in fp32; y is computed in fp32 as (r * inv) * gamma
 * and rounded once to the output dtype.  fp32 denormals are preserved.
 *
 * Conventions for every entry point (the *_ex forms below relax the first):
 *   - All data pointers are DEVICE pointers to contiguous row-major tensors;
 *     row i occupies elements [i*hidden, (i+1)*hidden).  gamma is [hidden].
 *     All tensors share one dtype (RMSN_F32, RMSN_F16, RMSN_BF16).
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; work is enqueued on `stream` (a hipStream_t; NULL means
 *     the default stream) and the call returns.  A fault inside a kernel
 *     surfaces at the caller's next synchronisation.
 *   - Arguments are validated before anything is launched; on any error
 *     nothing is launched and a negative RMSN_ERR_* code is returned.
 *     rmsnorm_last_error() describes the most recent failure of the calling
 *     thread.  rows == 0 is a no-op that returns RMSN_OK.
 *   - Any base alignment is accepted.  Kernels move 16-byte chunks when every
 *     base is 16-byte aligned and hidden*sizeof(dtype) is a multiple of 16,
 *     else the widest of 8 or 4 bytes that both allow, else single elements;
 *     the numerics are the same for every width.
 *   - Limits: 1 <= hidden <= RMSN_MAX_HIDDEN, rows >= 0, eps finite and >= 0.
 */
#ifndef RMSNORM_H
#define RMSNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RMSN_F32 = 0, RMSN_F16 = 1, RMSN_BF16 = 2 } rmsn_dtype;

enum {
  RMSN_OK = 0,
  RMSN_ERR_NULL = -1,   /* a required pointer is NULL (rows > 0)               */
  RMSN_ERR_SHAPE = -2,  /* rows < 0, hidden < 1 or hidden > RMSN_MAX_HIDDEN    */
  RMSN_ERR_DTYPE = -3,  /* unknown dtype code                                  */
  RMSN_ERR_K = -4,      /* k outside [1, RMSN_KMAX]                            */
  RMSN_ERR_ALIAS = -5,  /* forbidden overlap between buffers (see below)       */
  RMSN_ERR_EPS = -6,    /* eps negative, NaN or infinite                       */
  RMSN_ERR_HIP = -7     /* the HIP runtime reported an error at launch         */
};

#define RMSN_KMAX 16
#define RMSN_GATHER_MAX 16
#define RMSN_MAX_HIDDEN (1 << 24)

/*
 * rmsnorm_fwd -- plain RMSNorm (page "RMSNorm kernel", sections 1 and 2).
 *   out    [rows, hidden] written.  May be exactly x (in-place); any other
 *          overlap with x, and any overlap with gamma, is RMSN_ERR_ALIAS.
 *   x      [rows, hidden] read.
 *   gamma  [hidden] read.
 *   eps    added to the mean of squares inside the square root.
 */
int rmsnorm_fwd(void* out, const void* x, const void* gamma, int64_t rows, int64_t hidden,
                float eps, int dtype, void* stream);

/*
 * add_rmsnorm_fwd -- fused K-partial sum + residual + RMSNorm (page
 * "Tokenweave fused-RMSNorm-AR kernel", "Code walkthrough"; with every
 * partial already in local device memory).
 *   out       [rows, hidden] written.  May be exactly one of the partials.
 *   residual  [rows, hidden] read, then overwritten with the rounded sum.
 *   partials  HOST array of k device pointers, each [rows, hidden] read; the
 *             array is copied at the call and may be freed on return.
 *             Partials may alias one another.
 *   k         1..RMSN_KMAX.
 *   Forbidden overlaps (RMSN_ERR_ALIAS): out with residual or gamma; out
 *   partially overlapping a partial; residual with any partial or gamma.
 */
int add_rmsnorm_fwd(void* out, void* residual, const void* const* partials, int k,
                    const void* gamma, int64_t rows, int64_t hidden, float eps, int dtype,
                    void* stream);

/*
 * add_rmsnorm_ag_fwd -- add_rmsnorm_fwd with an all-gather epilogue: every
 * normalised row is stored into each of the nout gather buffers, in one pass
 * (page "Tokenweave fused-RMSNorm-AR kernel", "Code walkthrough": one rank
 * reduces its share of the tokens over the ranks' partials, adds its
 * residual, normalises, and broadcasts the normalised rows to every rank by
 * stores; here every buffer is local device memory -- with several GPUs,
 * outs[j] would be rank j's gather buffer at this rank's rows, and partials
 * the ranks' partial buffers at the same rows).
 *   outs      HOST array of nout device pointers, each [rows, hidden]
 *             written with the same values (add_rmsnorm_fwd's out); the
 *             array is copied at the call.
 *   nout      1..RMSN_GATHER_MAX (RMSN_ERR_SHAPE otherwise).
 *   residual, partials, k, gamma: as for add_rmsnorm_fwd.
 *   Forbidden overlaps (RMSN_ERR_ALIAS): as for add_rmsnorm_fwd, and any
 *   output buffer with another one, with residual, gamma or any partial
 *   (exact aliasing included).  Returns RMSN_ERR_NULL for a NULL outs,
 *   outs[j], residual, partials or gamma (rows > 0).
 */
int add_rmsnorm_ag_fwd(void* const* outs, int nout, void* residual, const void* const* partials,
                       int k, const void* gamma, int64_t rows, int64_t hidden, float eps,
                       int dtype, void* stream);

/*
 * The general interface -- page "RMSNorm kernel", section 2, which states the
 * input as [..., hidden_dim]: any number of leading dimensions flattened into
 * rows, the hidden dimension contiguous.  Beyond rmsnorm_fwd /
 * add_rmsnorm_fwd it allows:
 *   - a row stride per tensor, in ELEMENTS of that tensor's dtype (row i of
 *     a tensor starts i * stride elements after its base).  A stride must be
 *     >= hidden when rows > 1 (RMSN_ERR_SHAPE otherwise); views that skip
 *     rows or columns of a larger buffer are accepted as they are;
 *   - gamma in fp32 (gamma_dtype RMSN_F32) with fp16 / bf16 data, or in the
 *     data dtype (any other gamma dtype is RMSN_ERR_DTYPE);
 *   - an output dtype of its own (any of the three).  y is computed in fp32
 *     exactly as above and rounded once to the output dtype.
 * The data (x, partials, residual) share `dtype`; the residual is stored in
 * it, bit-exact as above.  Everything else is as for the plain entry points:
 * device pointers, nothing allocated, asynchronous on `stream`, validation
 * before launch.  Aliasing: out may be exactly an input (same base, same
 * stride) only when out_dtype == dtype; any other shared byte between out
 * and an input, the residual or gamma, or between the residual and a
 * partial or gamma, is RMSN_ERR_ALIAS (rows of equal stride that interleave
 * without sharing bytes do not overlap).  With 16-byte chunks of data, each
 * tensor's base and row pitch must be aligned to its own access width (16
 * bytes, or E elements of its dtype when narrower); otherwise narrower
 * chunks are used, with the same numerics.
 */

/* rmsnorm_fwd_ex -- plain RMSNorm, general layout and dtypes. */
int rmsnorm_fwd_ex(void* out, int64_t out_stride, int out_dtype, const void* x, int64_t x_stride,
                   int dtype, const void* gamma, int gamma_dtype, int64_t rows, int64_t hidden,
                   float eps, void* stream);

/*
 * add_rmsnorm_fwd_ex -- fused form, general layout and dtypes.
 * partial_strides is a HOST array of k strides (copied at the call), or NULL
 * for partials of stride hidden.
 */
int add_rmsnorm_fwd_ex(void* out, int64_t out_stride, int out_dtype, void* residual,
                       int64_t residual_stride, const void* const* partials,
                       const int64_t* partial_strides, int k, int dtype, const void* gamma,
                       int gamma_dtype, int64_t rows, int64_t hidden, float eps, void* stream);

/* Static description of an error code (never NULL). */
const char* rmsnorm_strerror(int code);

/* Description of the calling thread's most recent failed call ("" if none). */
const char* rmsnorm_last_error(void);

/*
 * rmsnorm_plan -- which kernel the dispatcher picks for a call with these
 * sizes (k = 0 means plain RMSNorm; align is the alignment in bytes that
 * every base pointer shares, 16 or more meaning 16-byte aligned).  Writes a
 * NUL-terminated name such as "vgpr<bf16,tpr=512,npt=1,wg=512,k=1,nt>" into
 * buf and returns RMSN_OK, or an error code for sizes that a call would
 * reject.  Launches nothing.
 */
int rmsnorm_plan(int64_t rows, int64_t hidden, int k, int dtype, int align, char* buf,
                 int buflen);

/*
 * rmsnorm_variants -- names of every compiled kernel variant for dtype,
 * newline-separated, into buf.  Returns the number of variants (>= 0) or an
 * error code.  Any name can be forced with rmsnorm_tune.
 */
int rmsnorm_variants(int dtype, char* buf, int buflen);

/*
 * rmsnorm_tune -- for tuning and testing only.  From now on every call of
 * this process (every entry point of this header, and the plan queries)
 * uses the kernel variant named `variant` (a name from rmsnorm_variants,
 * rmsnorm_variants_ag or rmsnorm_variants_ex; a call the variant cannot run
 * then fails with RMSN_ERR_SHAPE), and launches at most grid_cap workgroups
 * (rows beyond are processed in a grid-stride loop).  variant NULL or ""
 * restores the dispatcher's choice; grid_cap <= 0 restores the default
 * grid.  Nothing else (no environment variable) changes the choice.  Set it
 * before the calls it should affect: it is not synchronised with calls
 * running on other threads.  Returns RMSN_OK, or RMSN_ERR_SHAPE for a name
 * longer than 127 bytes (nothing is changed then).
 */
int rmsnorm_tune(const char* variant, int64_t grid_cap);

/* rmsnorm_plan_ag / rmsnorm_variants_ag -- the same for add_rmsnorm_ag_fwd
 * (k >= 1; names end in ",ag>"; rmsnorm_tune forces them the same way). */
int rmsnorm_plan_ag(int64_t rows, int64_t hidden, int k, int dtype, int align, char* buf,
                    int buflen);
int rmsnorm_variants_ag(int dtype, char* buf, int buflen);

/* rmsnorm_plan_ex / rmsnorm_variants_ex -- the same for the general
 * interface's dtype combinations (contiguous rows for the plan). */
int rmsnorm_plan_ex(int64_t rows, int64_t hidden, int k, int dtype, int gamma_dtype,
                    int out_dtype, int align, char* buf, int buflen);
int rmsnorm_variants_ex(int dtype, int gamma_dtype, int out_dtype, char* buf, int buflen);

/*
 * rmsnorm_plan_call -- validate one call of the general interface exactly
 * as add_rmsnorm_fwd_ex (residual != NULL) or rmsnorm_fwd_ex (residual ==
 * NULL: then k == 1 and partials[0] is x) would, with these very pointers,
 * strides and dtypes, and write the name of the kernel that call would
 * launch into buf ("none" when rows == 0).  Launches nothing and touches no
 * device memory: callers can check a call before recording it in a graph.
 * Returns RMSN_OK or the error code the call would return.
 */
int rmsnorm_plan_call(void* out, int64_t out_stride, int out_dtype, void* residual,
                      int64_t residual_stride, const void* const* partials,
                      const int64_t* partial_strides, int k, int dtype, const void* gamma,
                      int gamma_dtype, int64_t rows, int64_t hidden, float eps, char* buf,
                      int buflen);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_H */
