// stream_probe.hip -- the HBM bandwidth a plain streaming kernel reaches on
// this GPU for a given mix of read and write streams: the practical ceiling
// that the RMSNorm kernels are compared with (a measurement aid, not part of
// the RMSNorm library).
//
// stream_probe(reads[], nr, writes[], nw, n16, grid, stream): every lane moves
// 16-byte chunks, 4 per step, with nontemporal loads and stores, over nr read
// streams and nw write streams of n16 chunks each.  The written value is the
// XOR of the read chunks, so the loads cannot be dropped; with nw == 0 the
// XOR is stored to writes' sink slot only if it equals an impossible value.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxStreams = 16;
constexpr int kUnroll = 4;
constexpr int kBlock = 256;

struct Streams {
  const u32x4* r[kMaxStreams];
  u32x4* w[kMaxStreams];
};

__global__ __launch_bounds__(kBlock) void probe_kernel(Streams s, int nr, int nw, int64_t n,
                                                       u32x4* sink) {
  u32x4 keep = {0u, 0u, 0u, 0u};
  const int64_t step = (int64_t)gridDim.x * kBlock * kUnroll;
  for (int64_t i0 = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; i0 < n; i0 += step) {
    u32x4 acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] = u32x4{(uint32_t)u, 0u, 0u, 0u};
    for (int j = 0; j < nr; ++j) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        v[u] = i < n ? __builtin_nontemporal_load(s.r[j] + i) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc[u] ^= v[u];
    }
    for (int j = 0; j < nw; ++j) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        if (i < n) __builtin_nontemporal_store(acc[u], s.w[j] + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) keep ^= acc[u];
  }
  if (nw == 0 && keep.x == 0x9e3779b9u && keep.y == 0x7f4a7c15u) sink[0] = keep;
}

}  // namespace

extern "C" int stream_probe(const void* const* reads, int nr, void* const* writes, int nw,
                            int64_t n16, void* sink, int grid, void* stream) {
  if (nr < 0 || nw < 0 || nr > kMaxStreams || nw > kMaxStreams || n16 < 0 || grid < 1 || !sink)
    return -1;
  Streams s{};
  for (int j = 0; j < nr; ++j) {
    if (!reads[j]) return -1;
    s.r[j] = static_cast<const u32x4*>(reads[j]);
  }
  for (int j = 0; j < nw; ++j) {
    if (!writes[j]) return -1;
    s.w[j] = static_cast<u32x4*>(writes[j]);
  }
  hipLaunchKernelGGL(probe_kernel, dim3(grid), dim3(kBlock), 0, (hipStream_t)stream, s, nr, nw,
                     n16, static_cast<u32x4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
