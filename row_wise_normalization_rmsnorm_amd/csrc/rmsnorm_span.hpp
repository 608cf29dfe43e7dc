// rmsnorm_span.hpp -- host-only geometry of the tensors a call names: the
// alignment a base pointer and row pitch share, and whether two row-strided
// tensors share a byte (the aliasing rules of the C ABI are checked with
// it).  No HIP: the CPU tests compile it with the host compiler and compare
// overlap() with brute force over the bytes each span covers.
#pragma once

#include <stdint.h>

#include <algorithm>

namespace rmsn_host {

// Largest power of two, capped at 16, dividing the value.
inline int align_of_int(uint64_t u) {
  int a = 16;
  while (a > 1 && (u & (uint64_t)(a - 1))) a /= 2;
  return a;
}
inline int align_of(const void* p) { return align_of_int((uintptr_t)p); }

// A tensor as the kernels see it: `rows` rows of `len` bytes, row r at
// base + r * pitch bytes.
struct Span {
  const void* base;
  int64_t pitch;  // bytes
  int64_t len;    // bytes per row
  int64_t rows;
  int align() const { return std::min(align_of(base), rows > 1 ? align_of_int((uint64_t)pitch) : 16); }
  int64_t extent() const { return (rows - 1) * pitch + len; }
};

inline int64_t floor_div(int64_t a, int64_t b) { return a / b - ((a % b != 0) && ((a < 0) != (b < 0))); }
inline int64_t ceil_div(int64_t a, int64_t b) { return -floor_div(-a, b); }

// Do two spans share a byte?  Exact for equal pitches that are at least
// both row lengths (rows interleave); otherwise the extents are compared.
inline bool overlap(const Span& a, const Span& b) {
  const intptr_t x = (intptr_t)a.base, y = (intptr_t)b.base;
  if (!(x < y + b.extent() && y < x + a.extent())) return false;
  if (a.pitch == b.pitch && a.rows > 1 && b.rows > 1 && a.pitch >= a.len && a.pitch >= b.len) {
    // row i of a is [x + i p, x + i p + la), row j of b is [y + j p, ...);
    // they meet iff d + t p lies in (-lb, la) for d = y - x, t = j - i.
    const int64_t p = a.pitch, d = (int64_t)(y - x);
    int64_t lo = floor_div(-b.len - d, p) + 1, hi = ceil_div(a.len - d, p) - 1;
    // t = j - i with i a row of a and j a row of b
    lo = std::max(lo, -(a.rows - 1));
    hi = std::min(hi, b.rows - 1);
    return lo <= hi;
  }
  return true;
}

inline bool same_span(const Span& a, const Span& b) {
  return a.base == b.base && a.pitch == b.pitch && a.len == b.len;
}

}  // namespace rmsn_host
