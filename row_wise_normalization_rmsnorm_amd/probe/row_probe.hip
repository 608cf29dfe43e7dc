// row_probe.hip -- alternative designs of the fused add + RMSNorm row kernel
// for 4096-wide bf16 rows with one partial (the 8192 x 4096 workload), timed
// beside the library's kernel by `bench.py --design-sweep` (a measurement
// aid, not part of the RMSNorm library).  Every design computes the same
// thing as the library: r <- bf16(x + r) in place, out = bf16((r * inv) *
// gamma) with inv = rsqrt(sum(r^2) / H + eps) in fp32; the bench checks each
// against the library's kernel before timing it.  Rows whose fp32 sum of
// squares leaves fp32's range are not rescaled here (the bench's inputs have
// none).
//
// row_probe(design, load_cpol, store_cpol, grid, x, r, out, gamma, rows, eps,
// stream), design:
//   0  one row per 512-lane workgroup, one 16-byte chunk per lane (the
//      library's shape), buffer loads/stores with the given cache-policy
//      bits (bit 0 sc0, bit 1 nt, bit 4 sc1), residual stored before the
//      row reduction;
//   1  the same with the residual stored after the reduction;
//   2  design 0 with rows dealt to the eight XCDs in contiguous eighths
//      (workgroup b, which the hardware places on XCD b % 8, takes row
//      (b % 8) * rows / 8 + b / 8) instead of round robin;
//   3  persistent: `grid` workgroups loop over the rows, each issuing the
//      next row's loads before it reduces and stores the current one (two
//      register sets used in turn, so no load in flight is copied);
//   4  two rows per 1024-lane workgroup.
//   5, 6, 7  phased: each wave owns 2, 4 or 1 consecutive rows (256-lane
//      workgroups, grid = rows / (4 * rows per wave)); lane l holds chunks
//      l, l + 64, ..., l + 448 of each row.  The wave loads and sums all its
//      rows, keeping the rounded residual in registers, before it stores
//      any, so that when every wave of the launch is resident at once
//      (8192 rows: 4096 waves at two rows, 16 per CU) nearly all of the
//      launch's reads come before nearly all of its writes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../csrc/rmsnorm_kernels.hpp"

namespace {

using rmsn::Vec;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
using IV = Vec<__bf16, 8>;
constexpr int kHidden = 4096;
constexpr int kChunks = kHidden / 8;  // 16-byte chunks per row
constexpr uint32_t kRowBytes = kHidden * 2;

struct Args {
  const __bf16* x;
  __bf16* r;
  __bf16* out;
  const __bf16* gamma;
  int64_t rows;
  float eps;
};

// A buffer resource over one row (`rows` past the end: an empty range, whose
// loads return zeros without touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_of(const void* base, int64_t row,
                                                         int64_t rows) {
  const bool ok = row < rows;
  return rmsn::row_rsrc(static_cast<const char*>(base) + (ok ? row : 0) * kRowBytes,
                        ok ? (int)kRowBytes : 0);
}

template <int LP>
__device__ __forceinline__ u32x4 ld(__amdgpu_buffer_rsrc_t rs, int c) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, LP);
}
template <int SP>
__device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t rs, int c, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, c * 16, 0, SP);
}

// One row's arithmetic on chunk c held by this lane: returns the rounded
// residual chunk and leaves the normalised chunk in y; the reduction runs
// over the WGS / 64 waves of the row through red.
template <int TPR, int NRED>
__device__ __forceinline__ float row_sum(u32x4 xv, u32x4 rv, u32x4& rnew, float (&v)[8],
                                         float (&red)[2][NRED], int& parity, int slot, int tr) {
  IV::raw_t xw, rw;
  xw.w[0] = xv;
  rw.w[0] = rv;
  float acc[8], t[8];
  IV::unpack(xw, acc);
  IV::unpack(rw, t);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += t[e];
  const IV::raw_t rn = IV::pack(acc);
  rnew = rn.w[0];
  IV::unpack(rn, v);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
  return rmsn::row_reduce<TPR, TPR / 64, NRED, false>(ss, red, parity, slot, tr);
}

__device__ __forceinline__ u32x4 normalise(const float (&v)[8], float inv, const float (&g)[8]) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (v[e] * inv) * g[e];
  return IV::pack(y).w[0];
}

// designs 0, 1, 2
template <int LP, int SP, bool LATE, bool XCD>
__global__ __launch_bounds__(512) void one_row_kernel(Args a) {
  __shared__ float red[2][8];
  int parity = 0;
  const int c = threadIdx.x;
  float g[8];
  IV::unpack(IV::load<false>(a.gamma, c), g);
  for (int64_t b = blockIdx.x; b < a.rows; b += gridDim.x) {
    const int64_t row = XCD ? (b % 8) * (a.rows / 8) + b / 8 : b;
    const auto xr = row_of(a.x, row, a.rows), rr = row_of(a.r, row, a.rows);
    const auto orr = row_of(a.out, row, a.rows);
    const u32x4 xv = ld<LP>(xr, c), rv = ld<LP>(rr, c);
    u32x4 rn;
    float v[8];
    if constexpr (!LATE) {
      IV::raw_t xw, rw;
      xw.w[0] = xv;
      rw.w[0] = rv;
      float acc[8], t[8];
      IV::unpack(xw, acc);
      IV::unpack(rw, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += t[e];
      const IV::raw_t p = IV::pack(acc);
      rn = p.w[0];
      st<SP>(rr, c, rn);
      IV::unpack(p, v);
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
      const float tot = rmsn::row_reduce<512, 8, 8, false>(ss, red, parity, 0, c);
      st<SP>(orr, c, normalise(v, rmsn::row_scale(tot, kHidden, a.eps), g));
    } else {
      const float tot = row_sum<512, 8>(xv, rv, rn, v, red, parity, 0, c);
      st<SP>(rr, c, rn);
      st<SP>(orr, c, normalise(v, rmsn::row_scale(tot, kHidden, a.eps), g));
    }
  }
}

// design 3
template <int LP, int SP>
__global__ __launch_bounds__(512) void persistent_kernel(Args a) {
  __shared__ float red[2][8];
  int parity = 0;
  const int c = threadIdx.x;
  float g[8];
  IV::unpack(IV::load<false>(a.gamma, c), g);
  const int64_t G = gridDim.x;
  int64_t row = blockIdx.x;
  u32x4 xa = ld<LP>(row_of(a.x, row, a.rows), c), ra = ld<LP>(row_of(a.r, row, a.rows), c);
  u32x4 xb, rb;
  auto work = [&](int64_t rw, u32x4 xv, u32x4 rv) {
    u32x4 rn;
    float v[8];
    const float tot = row_sum<512, 8>(xv, rv, rn, v, red, parity, 0, c);
    st<SP>(row_of(a.r, rw, a.rows), c, rn);
    st<SP>(row_of(a.out, rw, a.rows), c, normalise(v, rmsn::row_scale(tot, kHidden, a.eps), g));
  };
  while (row < a.rows) {
    xb = ld<LP>(row_of(a.x, row + G, a.rows), c);
    rb = ld<LP>(row_of(a.r, row + G, a.rows), c);
    work(row, xa, ra);
    row += G;
    if (row >= a.rows) break;
    xa = ld<LP>(row_of(a.x, row + G, a.rows), c);
    ra = ld<LP>(row_of(a.r, row + G, a.rows), c);
    work(row, xb, rb);
    row += G;
  }
}

// design 4
template <int LP, int SP>
__global__ __launch_bounds__(1024) void two_row_kernel(Args a) {
  __shared__ float red[2][16];
  int parity = 0;
  const int c = threadIdx.x & 511, slot = threadIdx.x >> 9;
  float g[8];
  IV::unpack(IV::load<false>(a.gamma, c), g);
  for (int64_t r0 = (int64_t)blockIdx.x * 2; r0 < a.rows; r0 += (int64_t)gridDim.x * 2) {
    const int64_t row = r0 + __builtin_amdgcn_readfirstlane(slot);
    const auto rr = row_of(a.r, row, a.rows);
    const u32x4 xv = ld<LP>(row_of(a.x, row, a.rows), c), rv = ld<LP>(rr, c);
    u32x4 rn;
    float v[8];
    const float tot = row_sum<512, 16>(xv, rv, rn, v, red, parity, slot, c);
    if (row < a.rows) {
      st<SP>(rr, c, rn);
      st<SP>(row_of(a.out, row, a.rows), c, normalise(v, rmsn::row_scale(tot, kHidden, a.eps), g));
    }
  }
}

// designs 5-7.  The loads run two steps ahead of the sums, S chunks of each
// input per step (S = 1, 2, 4 for 1, 2, 4 rows per wave); scheduling
// barriers keep the compiler from hoisting every load of the wave to the
// top, which would need more registers than the wave count allows.
template <int LP, int SP, int RPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RPW == 1 ? 8 : 8 / RPW)))
void phased_kernel(Args a) {
  constexpr int C = kChunks / 64;          // chunks of a row per lane
  constexpr int S = RPW;                   // chunks per input per step
  constexpr int T = RPW * C / S;           // steps
  const int lane = threadIdx.x & 63;
  const int64_t row0 =
      ((int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * RPW;
  u32x4 rn[RPW][C];
  float tot[RPW];
  u32x4 xv[2][S], rv[2][S];
  auto load = [&](int t) {
    const int i = t * S / C, j0 = t * S % C;
    const auto xr = row_of(a.x, row0 + i, a.rows), rr = row_of(a.r, row0 + i, a.rows);
#pragma unroll
    for (int q = 0; q < S; ++q) {
      xv[t & 1][q] = ld<LP>(xr, lane + 64 * (j0 + q));
      rv[t & 1][q] = ld<LP>(rr, lane + 64 * (j0 + q));
    }
  };
  float ss = 0.0f;
  load(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (t + 1 < T) load(t + 1);
    __builtin_amdgcn_sched_barrier(0);
    const int i = t * S / C, j0 = t * S % C;
#pragma unroll
    for (int q = 0; q < S; ++q) {
      IV::raw_t xw, rw;
      xw.w[0] = xv[t & 1][q];
      rw.w[0] = rv[t & 1][q];
      float acc[8], u[8], v[8];
      IV::unpack(xw, acc);
      IV::unpack(rw, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += u[e];
      const IV::raw_t p = IV::pack(acc);
      rn[i][j0 + q] = p.w[0];
      IV::unpack(p, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
    }
    if (j0 + S == C) {
      tot[i] = rmsn::wave_reduce(ss);
      ss = 0.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // The residual words pass through an empty asm statement so that the
  // compiler re-expands them here instead of keeping the phase-1 fp32 copies
  // (twice the registers) alive across the loads.
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int j = 0; j < C; ++j) asm volatile("" : "+v"(rn[i][j]));
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const float inv = rmsn::row_scale(tot[i], kHidden, a.eps);
    const auto rr = row_of(a.r, row0 + i, a.rows), orr = row_of(a.out, row0 + i, a.rows);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      st<SP>(rr, lane + 64 * j, rn[i][j]);
      float g[8], v[8];
      IV::unpack(IV::load<false>(a.gamma, lane + 64 * j), g);
      IV::raw_t w;
      w.w[0] = rn[i][j];
      IV::unpack(w, v);
      st<SP>(orr, lane + 64 * j, normalise(v, inv, g));
    }
  }
}

template <int LP, int SP>
int launch(int design, int grid, const Args& a, hipStream_t s) {
  switch (design) {
    case 0: hipLaunchKernelGGL((one_row_kernel<LP, SP, false, false>), dim3(grid), dim3(512), 0, s, a); break;
    case 1: hipLaunchKernelGGL((one_row_kernel<LP, SP, true, false>), dim3(grid), dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL((one_row_kernel<LP, SP, false, true>), dim3(grid), dim3(512), 0, s, a); break;
    case 3: hipLaunchKernelGGL((persistent_kernel<LP, SP>), dim3(grid), dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL((two_row_kernel<LP, SP>), dim3(grid), dim3(1024), 0, s, a); break;
    case 5: hipLaunchKernelGGL((phased_kernel<LP, SP, 2>), dim3(grid), dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((phased_kernel<LP, SP, 4>), dim3(grid), dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL((phased_kernel<LP, SP, 1>), dim3(grid), dim3(256), 0, s, a); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace

// Cache-policy pairs (load bits, store bits) the probe is built with.
#define ROW_PROBE_POLICIES(X) X(2, 2) X(2, 19) X(2, 18) X(19, 19) X(0, 19) X(0, 2)

extern "C" int row_probe_policies(int* loads, int* stores, int max) {
  int n = 0;
#define ROW_PROBE_LIST(L, S) \
  if (n < max) { loads[n] = L; stores[n] = S; } ++n;
  ROW_PROBE_POLICIES(ROW_PROBE_LIST)
#undef ROW_PROBE_LIST
  return n;
}

// grid: workgroups (designs 0-2: rows; 4: rows / 2; 3: any; 5, 6, 7: rows /
// 8, rows / 16, rows / 4, rounded up).  rows must be a multiple of 8 for
// design 2 and of 2 for design 4.  Returns 0, -1 for a
// design, policy or shape the probe does not have, -7 for a launch error.
extern "C" int row_probe(int design, int load_cpol, int store_cpol, int grid, const void* x,
                         void* r, void* out, const void* gamma, int64_t rows, float eps,
                         void* stream) {
  if (grid < 1 || rows < 1 || !x || !r || !out || !gamma) return -1;
  if ((design == 0 || design == 1 || design == 2) && grid != rows) return -1;
  if (design == 2 && rows % 8) return -1;
  if (design == 4 && (rows % 2 || grid != rows / 2)) return -1;
  if (design >= 5 && design <= 7) {
    const int64_t per = 4 * (design == 5 ? 2 : design == 6 ? 4 : 1);
    if (grid != (rows + per - 1) / per) return -1;
  }
  const Args a{static_cast<const __bf16*>(x), static_cast<__bf16*>(r), static_cast<__bf16*>(out),
               static_cast<const __bf16*>(gamma), rows, eps};
  const hipStream_t s = (hipStream_t)stream;
#define ROW_PROBE_CASE(L, S) \
  if (load_cpol == L && store_cpol == S) return launch<L, S>(design, grid, a, s);
  ROW_PROBE_POLICIES(ROW_PROBE_CASE)
#undef ROW_PROBE_CASE
  return -1;
}
