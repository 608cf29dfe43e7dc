/*
 * block_sum_oracle.c -- plain CPU oracle for the block all-reduce sum family.
 *
 * TEST INFRASTRUCTURE, not product code (see rmsnorm_oracle.c).
 *
 * What is computed: page "Block All Reduce CUDA代码学习" -- the sum of all
 * elements of a tensor, with low-precision storage widened before it is
 * accumulated (its "acc dtype" discussion: store narrow, accumulate wide),
 * fp8 formats decoded before they are added, and int8 widened to int32.
 * The oracle takes the plainest reading: decode every element exactly, add
 * them in index order in double (floating inputs) or in int64 (int8, then
 * reduced modulo 2^32 as int32 accumulation would).
 *
 * Formats (written from their published definitions):
 *   bf16: the upper half of an IEEE binary32;  f16: IEEE binary16;
 *   fp8 E4M3 (OCP): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 *     exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities;
 *   fp8 E5M2 (OCP): sign, 5 exponent bits (bias 15), 2 mantissa bits, with
 *     IEEE subnormals, infinities and NaNs.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "block_sum_oracle.h"

static double decode(const void* x, int64_t i, int dtype) {
  const unsigned char* b = (const unsigned char*)x;
  switch (dtype) {
    case BLOCK_SUM_ORACLE_F32: {
      float f;
      memcpy(&f, b + 4 * i, 4);
      return (double)f;
    }
    case BLOCK_SUM_ORACLE_BF16: {
      uint16_t h;
      memcpy(&h, b + 2 * i, 2);
      uint32_t u = (uint32_t)h << 16;
      float f;
      memcpy(&f, &u, 4);
      return (double)f;
    }
    case BLOCK_SUM_ORACLE_F16: {
      uint16_t h;
      memcpy(&h, b + 2 * i, 2);
      int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
      double v = e == 31 ? (m ? NAN : INFINITY)
                         : e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
      return s ? -v : v;
    }
    case BLOCK_SUM_ORACLE_FP8_E4M3: {
      unsigned u = b[i];
      int s = u >> 7, e = (u >> 3) & 15, m = u & 7;
      double v = (e == 15 && m == 7) ? NAN
                 : e == 0            ? ldexp((double)m, -9)
                                     : ldexp((double)(8 + m), e - 10);
      return s ? -v : v;
    }
    case BLOCK_SUM_ORACLE_FP8_E5M2: {
      unsigned u = b[i];
      int s = u >> 7, e = (u >> 2) & 31, m = u & 3;
      double v = e == 31 ? (m ? NAN : INFINITY)
                         : e == 0 ? ldexp((double)m, -16) : ldexp((double)(4 + m), e - 17);
      return s ? -v : v;
    }
    case BLOCK_SUM_ORACLE_I8:
      return (double)(int8_t)b[i];
    default:
      return NAN;
  }
}

static int known(int dtype) { return dtype >= 0 && dtype <= BLOCK_SUM_ORACLE_I8; }

int block_sum_oracle_decode(double* dst, const void* x, int64_t n, int dtype) {
  if (!known(dtype)) return -3;
  if (n < 0) return -2;
  if (n > 0 && (!dst || !x)) return -1;
  for (int64_t i = 0; i < n; ++i) dst[i] = decode(x, i, dtype);
  return 0;
}

int block_sum_oracle(double* sum_f64, double* abs_f64, int32_t* sum_i32, const void* x, int64_t n,
                     int dtype) {
  if (!known(dtype)) return -3;
  if (n < 0) return -2;
  if (n > 0 && !x) return -1;
  if (dtype == BLOCK_SUM_ORACLE_I8) {
    if (!sum_i32) return -1;
    int64_t s = 0;
    for (int64_t i = 0; i < n; ++i) s += (int8_t)((const unsigned char*)x)[i];
    /* int32 accumulation wraps modulo 2^32 */
    uint32_t w = (uint32_t)(uint64_t)s;
    int32_t r;
    memcpy(&r, &w, 4);
    *sum_i32 = r;
    if (sum_f64) *sum_f64 = (double)s;
    if (abs_f64) *abs_f64 = 0.0;
    return 0;
  }
  if (!sum_f64) return -1;
  double s = 0.0, a = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double v = decode(x, i, dtype);
    s += v;
    a += fabs(v);
  }
  *sum_f64 = s;
  if (abs_f64) *abs_f64 = a;
  return 0;
}
