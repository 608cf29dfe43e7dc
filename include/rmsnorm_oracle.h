/*
 * rmsnorm_oracle.h -- C ABI of the CPU oracle for row-wise RMSNorm and its
 * fused "K partials + residual, update residual in place, normalise" form.
 *
 * TEST INFRASTRUCTURE.  The oracle is a plain, slow, single-threaded C
 * implementation that lives in its own shared library (oracle/, built with
 * gcc).  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg load it.  The GPU library (include/rmsnorm.h) neither includes this
 * header nor links the oracle, and the two share no code.
 *
 * What is computed (per row i, independently):
 *   - Definition of RMSNorm over the last (hidden) dimension: page "RMSNorm
 *     kernel", section 1 Background (the linked PyTorch RMSNorm definition)
 *     and section 2 Analytics & Implementation, "Abstraction" (per-row sum of
 *     squares, mean, + eps, square root; then x_i * gamma_i / RMS(x)).
 *   - Fused form: page "Tokenweave fused-RMSNorm-AR kernel", section "Code
 *     walkthrough" (the per-token body of fused_rs_ln_ag_cta_kernel: reduced
 *     partials plus residual, residual written back in place, sum of squares
 *     of the stored values, rsqrt(variance / hidden + eps), then residual *
 *     scale * weight).
 *
 * All pointers are HOST pointers.  Tensors are contiguous row-major
 * [rows, hidden]; row i occupies elements [i*hidden, (i+1)*hidden).
 * gamma is [hidden] in the same dtype as the data.
 */
#ifndef RMSNORM_ORACLE_H
#define RMSNORM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes (same numbering as the GPU library's, defined independently) */
#define RMSNORM_ORACLE_F32  0
#define RMSNORM_ORACLE_F16  1
#define RMSNORM_ORACLE_BF16 2

/* return codes */
#define RMSNORM_ORACLE_OK          0
#define RMSNORM_ORACLE_ERR_NULL   -1  /* a required pointer is NULL          */
#define RMSNORM_ORACLE_ERR_SHAPE  -2  /* hidden < 1 or rows < 0              */
#define RMSNORM_ORACLE_ERR_DTYPE  -3  /* unknown dtype code                  */
#define RMSNORM_ORACLE_ERR_K      -4  /* k outside [1, RMSNORM_ORACLE_KMAX]  */
#define RMSNORM_ORACLE_ERR_EPS    -6  /* eps negative or not finite          */
#define RMSNORM_ORACLE_ERR_NOMEM  -8  /* scratch row could not be allocated  */

#define RMSNORM_ORACLE_KMAX 16

/*
 * rmsnorm_oracle -- reference result of both forms.
 *
 *  out       [rows, hidden] dtype, written: y rounded once (round to nearest,
 *            ties to even) from the double-precision value.  May be NULL when
 *            only y_f64 / rstd_out are wanted.  May alias partials[j] or the
 *            plain-mode input exactly: every row is read fully before any of
 *            it is written.
 *  residual  [rows, hidden] dtype, read and overwritten with r' (fused mode),
 *            or NULL for plain RMSNorm (then k must be 1 and partials[0] is x).
 *  partials  host array of k host pointers, each [rows, hidden] dtype.
 *  k         number of partials, 1..RMSNORM_ORACLE_KMAX.
 *  gamma     [hidden] dtype.
 *  eps       added to the mean of squares inside the square root; widened
 *            exactly to double.  Must be finite and >= 0.
 *  rstd_out  optional [rows] doubles: 1/sqrt(mean(v^2) + eps) per row.
 *
 * Fused mode, per element j of row i:
 *   acc = float(p_0); acc = fl32(acc + float(p_1)); ... ; acc = fl32(acc + float(r))
 *   (IEEE binary32 adds in exactly this order, accumulator seeded with p_0),
 *   r' = rne_dtype(acc) is stored into residual, and v_j = r'.
 * Plain mode: v_j = x_j.
 * Then, in double: ms = (sum_j v_j^2) / hidden; inv = 1/sqrt(ms + eps);
 *   y_j = (v_j * inv) * gamma_j; out_j = rne_dtype(y_j).
 * NaN in gives NaN out; values beyond the dtype's range round to +-inf.
 * rows == 0 is a no-op returning RMSNORM_ORACLE_OK.
 */
int rmsnorm_oracle(void* out, void* residual, const void* const* partials, int k,
                   const void* gamma, int64_t rows, int64_t hidden, float eps,
                   int dtype, double* rstd_out);

/*
 * rmsnorm_oracle_f64 -- the same computation, additionally returning the
 * unrounded double y (y_f64, [rows, hidden], may be NULL).  Used by the
 * oracle's own pins, which check the double result against closed forms and
 * the rounding step separately.
 */
int rmsnorm_oracle_f64(void* out, double* y_f64, void* residual,
                       const void* const* partials, int k, const void* gamma,
                       int64_t rows, int64_t hidden, float eps, int dtype,
                       double* rstd_out);

/*
 * rmsnorm_oracle_ex -- the general form: the same computation with gamma in
 * gamma_dtype and out in out_dtype (each one of the three dtype codes; the
 * data -- partials, residual -- stay in dtype).  gamma is read exactly in
 * its own dtype; y is rounded once, from double, to out_dtype.  The residual
 * is computed and stored exactly as above, in dtype.  out may be NULL; it
 * may alias an input exactly only when out_dtype == dtype.
 */
int rmsnorm_oracle_ex(void* out, int out_dtype, double* y_f64, void* residual,
                      const void* const* partials, int k, int dtype,
                      const void* gamma, int gamma_dtype, int64_t rows, int64_t hidden,
                      float eps, double* rstd_out);

/*
 * rmsnorm_oracle_round -- round n doubles to dtype (nearest, ties to even,
 * overflow to +-inf, NaN to quiet NaN) and store them; exposes the oracle's
 * converter so that it can be pinned against independent converters.
 */
int rmsnorm_oracle_round(void* dst, const double* src, int64_t n, int dtype);

/* rmsnorm_oracle_decode -- widen n dtype values to double (exact). */
int rmsnorm_oracle_decode(double* dst, const void* src, int64_t n, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_ORACLE_H */
