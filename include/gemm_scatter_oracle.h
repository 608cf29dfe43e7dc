/*
 * gemm_scatter_oracle.h -- C ABI of the CPU oracle for the GEMM whose
 * epilogue writes its result straight into reduce-scatter buffers (page
 * "LLM System: 通信计算融合算子实现 01 - sm80GEMM + ReduceScatter": section
 * "flux实现：sm80 gemm+rs" for the idea, section "cutlass自定义epilogue–sm80"
 * for the epilogue's arithmetic and its scatter store).
 *
 * TEST INFRASTRUCTURE, built into the same oracle library as
 * rmsnorm_oracle.h; the GPU library never includes or links it.
 */
#ifndef GEMM_SCATTER_ORACLE_H
#define GEMM_SCATTER_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_SCATTER_ORACLE_WORLD_MAX 16

/*
 * gemm_scatter_oracle -- rows [row0, row1) of
 *
 *     D[i][j] = alpha * sum_{p < k} A[i][p] * B[j][p]  +  beta * C[i][j]
 *
 * with A [m][k] (row stride lda), B [n][k] (row stride ldb: the weight
 * layout, k contiguous), C [m][n] (row stride ldc; NULL: the beta term is
 * absent).  All values are decoded exactly; products and sums are in double,
 * in index order p = 0, 1, ...; alpha and beta are the float arguments
 * widened exactly.  IEEE rules apply throughout (0 * inf is NaN, a NaN
 * anywhere in a row of A or a column of B gives NaN).
 *
 * The m rows form `world` chunks of m / world rows each; row i belongs to
 * chunk q = i / (m / world) and is stored, rounded once to dtype with
 * round-to-nearest-even, at dst[q] + (i - q * m / world) * ldd.  dst may be
 * NULL (nothing is stored).
 *
 * y_f64 (nullable): [row1 - row0][n] unrounded values.  mag_f64 (nullable):
 * the same shape, |alpha| * sum_p |A[i][p] * B[j][p]| + |beta * C[i][j]|,
 * the scale against which a floating-point implementation's rounding error
 * is bounded.
 *
 * HOST pointers.  dtype: 1 (IEEE binary16) or 2 (bfloat16) -- the codes of
 * rmsnorm_oracle.h.  Returns 0, -1 (NULL pointer), -2 (bad shape, stride,
 * world or row range), -3 (dtype) or -8 (out of memory).
 */
int gemm_scatter_oracle(void* const* dst, int64_t ldd, int world, const void* a, int64_t lda,
                        const void* b, int64_t ldb, const void* c, int64_t ldc, float alpha,
                        float beta, int64_t m, int64_t n, int64_t k, int dtype, int64_t row0,
                        int64_t row1, double* y_f64, double* mag_f64);

/*
 * gemm_scatter_oracle_chunk_order -- the order in which the chunks of one
 * rank's product are produced: every other rank's chunk first, in ring order
 * starting after `rank`, and the rank's own chunk last (page "LLM System:
 * 通信计算融合算子实现 01", section "gemmrs版本的swizzle如何编排").
 * order[s] = (rank + 1 + s) mod world for s < world.  Returns 0 or -2.
 */
int gemm_scatter_oracle_chunk_order(int world, int rank, int* order);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_SCATTER_ORACLE_H */
