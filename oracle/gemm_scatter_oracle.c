/*
 * gemm_scatter_oracle.c -- plain CPU oracle for the GEMM whose epilogue
 * stores into reduce-scatter buffers.
 *
 * TEST INFRASTRUCTURE, not product code (see rmsnorm_oracle.c).
 *
 * What is computed: page "LLM System: 通信计算融合算子实现 01 - sm80GEMM +
 * ReduceScatter".  Its section "flux实现：sm80 gemm+rs" describes the second
 * GEMM of a tensor-parallel FFN whose epilogue, instead of writing the
 * product to ordinary memory, writes it into the reduce-scatter buffers;
 * section "cutlass自定义epilogue–sm80" gives the epilogue's arithmetic (the
 * accumulator scaled by alpha, plus beta times a loaded C) and its store (a
 * scatter: each part of the output goes to the buffer of the rank that
 * holds it).  Its section "gemmrs版本的swizzle如何编排" says the output is
 * cut into one chunk per rank, only one of which stays local.
 *
 * Readings taken where the page is silent (each also listed with the
 * design notes):
 *   - B is given in the weight layout [n][k] (k contiguous), so the product
 *     is A * B^T: the layout of a linear layer's weight.
 *   - The chunks split the rows (the token dimension): chunk q holds rows
 *     [q * m / world, (q + 1) * m / world), as a reduce-scatter over tokens
 *     leaves each rank a contiguous block of rows.  m must divide evenly.
 *   - The result is rounded once, round-to-nearest-even, from the exact
 *     value to the 16-bit storage type.
 *   - The chunk production order: the other ranks' chunks in ring order
 *     starting after the local rank, the local chunk last.  The page's own
 *     eight-GPU schedule table is tied to its machine's topology and is not
 *     reproduced.
 *
 * The arithmetic is the definition: each element is the dot product of a row
 * of A and a row of B, summed in double in index order (products of two
 * 16-bit values are exact in double; the sum's error is at most
 * k * 2^-53 * sum |products|), scaled and shifted as the epilogue states.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "gemm_scatter_oracle.h"
#include "rmsnorm_oracle.h"

int gemm_scatter_oracle(void* const* dst, int64_t ldd, int world, const void* a, int64_t lda,
                        const void* b, int64_t ldb, const void* c, int64_t ldc, float alpha,
                        float beta, int64_t m, int64_t n, int64_t k, int dtype, int64_t row0,
                        int64_t row1, double* y_f64, double* mag_f64) {
  if (dtype != RMSNORM_ORACLE_F16 && dtype != RMSNORM_ORACLE_BF16) return -3;
  if (m < 0 || n < 0 || k < 0) return -2;
  if (world < 1 || world > GEMM_SCATTER_ORACLE_WORLD_MAX || m % world != 0) return -2;
  if (row0 < 0 || row1 < row0 || row1 > m) return -2;
  if (lda < k || ldb < k || (c && ldc < n) || (dst && ldd < n)) return -2;
  if (row1 == row0 || n == 0) return 0;
  if ((k > 0 && (!a || !b))) return -1;
  if (dst) {
    for (int q = 0; q < world; ++q)
      if (!dst[q]) return -1;
  }

  /* every 16-bit code decoded exactly once */
  double* value = (double*)malloc(65536 * sizeof(double));
  double* row = (double*)malloc((size_t)n * sizeof(double));
  uint16_t* codes = (uint16_t*)malloc(65536 * sizeof(uint16_t));
  if (!value || !row || !codes) {
    free(value);
    free(row);
    free(codes);
    return -8;
  }
  for (int u = 0; u < 65536; ++u) codes[u] = (uint16_t)u;
  rmsnorm_oracle_decode(value, codes, 65536, dtype);
  free(codes);

  const uint16_t* A = (const uint16_t*)a;
  const uint16_t* B = (const uint16_t*)b;
  const uint16_t* C = (const uint16_t*)c;
  const int64_t chunk = m / world;
  for (int64_t i = row0; i < row1; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0, dot_abs = 0.0;
      for (int64_t p = 0; p < k; ++p) {
        const double prod = value[A[i * lda + p]] * value[B[j * ldb + p]];
        dot += prod;
        dot_abs += fabs(prod);
      }
      double y = (double)alpha * dot;
      double mag = fabs((double)alpha) * dot_abs;
      if (C) {
        const double cv = value[C[i * ldc + j]];
        y += (double)beta * cv;
        mag += fabs((double)beta * cv);
      }
      row[j] = y;
      if (y_f64) y_f64[(i - row0) * n + j] = y;
      if (mag_f64) mag_f64[(i - row0) * n + j] = mag;
    }
    if (dst) {
      const int64_t q = i / chunk;
      uint16_t* out = (uint16_t*)dst[q] + (i - q * chunk) * ldd;
      rmsnorm_oracle_round(out, row, n, dtype);
    }
  }
  free(value);
  free(row);
  return 0;
}

int gemm_scatter_oracle_chunk_order(int world, int rank, int* order) {
  if (world < 1 || world > GEMM_SCATTER_ORACLE_WORLD_MAX || rank < 0 || rank >= world || !order)
    return -2;
  for (int s = 0; s < world; ++s) order[s] = (rank + 1 + s) % world;
  return 0;
}
