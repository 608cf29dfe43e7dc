/*
 * block_sum_oracle.h -- C ABI of the CPU oracle for the block all-reduce sum
 * family (page "Block All Reduce CUDA代码学习": the sum of every element of a
 * tensor, for f32 / f16 / bf16 / fp8 e4m3 / fp8 e5m2 inputs accumulated in
 * floating point and int8 inputs accumulated in int32).
 *
 * TEST INFRASTRUCTURE, built into the same oracle library as
 * rmsnorm_oracle.h; the GPU library never includes or links it.
 */
#ifndef BLOCK_SUM_ORACLE_H
#define BLOCK_SUM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes (same numbering as the GPU library's block_sum.h) */
#define BLOCK_SUM_ORACLE_F32 0
#define BLOCK_SUM_ORACLE_F16 1
#define BLOCK_SUM_ORACLE_BF16 2
#define BLOCK_SUM_ORACLE_FP8_E4M3 3 /* OCP E4M3 ("fn": no inf, NaN = S.1111.111) */
#define BLOCK_SUM_ORACLE_FP8_E5M2 4 /* OCP E5M2 (IEEE-like, with inf)            */
#define BLOCK_SUM_ORACLE_I8 5

/*
 * block_sum_oracle -- sum of the n elements of x (HOST memory).
 *   Floating dtypes: *sum_f64 = the sum of the exact element values,
 *     accumulated in double in index order (error <= n * 2^-53 * sum|x|);
 *     *abs_f64 (nullable) = sum of |x| (for error bounds).  NaN in gives NaN;
 *     +inf and -inf together give NaN.
 *   I8: *sum_i32 = the exact sum reduced modulo 2^32 to int32 (what int32
 *     accumulation gives); *sum_f64 (nullable) = the exact sum.
 * Returns 0, -1 (NULL pointer with n > 0), -2 (n < 0) or -3 (dtype).
 */
int block_sum_oracle(double* sum_f64, double* abs_f64, int32_t* sum_i32, const void* x, int64_t n,
                     int dtype);

/* block_sum_oracle_decode -- exact value of n elements of dtype as doubles. */
int block_sum_oracle_decode(double* dst, const void* x, int64_t n, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* BLOCK_SUM_ORACLE_H */
