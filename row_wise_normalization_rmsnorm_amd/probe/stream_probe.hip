// stream_probe.hip -- the HBM bandwidth a plain streaming kernel reaches on
// this GPU for a given mix of read and write streams: the practical ceiling
// that the RMSNorm kernels are compared with (a measurement aid, not part of
// the RMSNorm library).
//
// stream_probe(reads[], nr, writes[], nw, n16, grid, stream): every lane moves
// 16-byte chunks, 4 per step (256-lane workgroups; stream_probe_shape picks
// other shapes and cache policies), with nontemporal loads and stores, over
// nr read streams and nw write streams of n16 chunks each.  The written value
// is the XOR of the read chunks, so the loads cannot be dropped; with nw == 0
// the XOR is stored to writes' sink slot only if it equals an impossible
// value.
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

// Cache policies.  Policy 0 is the global_load/store_dwordx4 pair with the
// nontemporal bit (what the RMSNorm kernels use).  The others move the same
// chunks with buffer_load/store_dwordx4, whose cache-policy bits are set per
// instruction: bit 0 = sc0, bit 1 = nt, bit 4 = sc1 (the CDNA3/CDNA4 scope
// and streaming controls).  {load bits, store bits}.
constexpr int kPolicies = 9;
__host__ __device__ constexpr int load_bits(int pol) {
  return pol == 1 ? 0 : pol == 2 ? 2 : pol == 3 ? 2 : pol == 4 ? 0 : pol == 5 ? 19
       : pol == 6 ? 17 : pol == 7 ? 2 : pol == 8 ? 0 : 2;
}
__host__ __device__ constexpr int store_bits(int pol) {
  return pol == 1 ? 0 : pol == 2 ? 2 : pol == 3 ? 0 : pol == 4 ? 2 : pol == 5 ? 19
       : pol == 6 ? 17 : pol == 7 ? 19 : pol == 8 ? 19 : 2;
}

// A buffer resource over [base, base + bytes): raw (stride 0) 32-bit words,
// the gfx9 data-format word; loads past `bytes` return zeros and stores past
// it are dropped (never reached: every access is also guarded).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// CONTIG = false: grid-stride loop (workgroup b takes tiles b, b + grid, ...);
// CONTIG = true: workgroup b streams one contiguous range of n / grid chunks.
template <int BLOCK, int UNROLL, bool CONTIG, int POL>
__global__ __launch_bounds__(BLOCK) void probe_kernel(Streams s, int nr, int nw, int64_t n,
                                                      u32x4* sink) {
  constexpr int LB = load_bits(POL), SB = store_bits(POL);
  u32x4 keep = {0u, 0u, 0u, 0u};
  const int64_t tile = (int64_t)BLOCK * UNROLL;
  const int64_t tiles = (n + tile - 1) / tile;
  int64_t t_begin, t_end, t_step;
  if constexpr (CONTIG) {
    const int64_t per = (tiles + gridDim.x - 1) / gridDim.x;
    t_begin = (int64_t)blockIdx.x * per;
    t_end = t_begin + per < tiles ? t_begin + per : tiles;
    t_step = 1;
  } else {
    t_begin = blockIdx.x;
    t_end = tiles;
    t_step = gridDim.x;
  }
  for (int64_t t = t_begin; t < t_end; t += t_step) {
    const int64_t i0 = t * tile;                       // first chunk of the tile (uniform)
    const int64_t left = n - i0;                       // chunks from i0 to the end
    const int cnt = left < tile ? (int)left : (int)tile;
    u32x4 acc[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc[u] = u32x4{(uint32_t)u, 0u, 0u, 0u};
    for (int j = 0; j < nr; ++j) {
      u32x4 v[UNROLL];
      if constexpr (POL == 0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int l = threadIdx.x + u * BLOCK;
          v[u] = l < cnt ? __builtin_nontemporal_load(s.r[j] + i0 + l) : u32x4{0u, 0u, 0u, 0u};
        }
      } else {
        const auto rs = rsrc(s.r[j] + i0, (uint32_t)cnt * 16u);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int l = threadIdx.x + u * BLOCK;
          v[u] = l < cnt ? __builtin_amdgcn_raw_buffer_load_b128(rs, l * 16, 0, LB)
                         : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) acc[u] ^= v[u];
    }
    for (int j = 0; j < nw; ++j) {
      if constexpr (POL == 0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int l = threadIdx.x + u * BLOCK;
          if (l < cnt) __builtin_nontemporal_store(acc[u], s.w[j] + i0 + l);
        }
      } else {
        const auto ws = rsrc(s.w[j] + i0, (uint32_t)cnt * 16u);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int l = threadIdx.x + u * BLOCK;
          if (l < cnt) __builtin_amdgcn_raw_buffer_store_b128(acc[u], ws, l * 16, 0, SB);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) keep ^= acc[u];
  }
  if (nw == 0 && keep.x == 0x9e3779b9u && keep.y == 0x7f4a7c15u) sink[0] = keep;
}

template <int BLOCK, int UNROLL, int POL>
void launch(Streams s, int nr, int nw, int64_t n16, int grid, bool contig, void* sink,
            void* stream) {
  if (contig)
    hipLaunchKernelGGL((probe_kernel<BLOCK, UNROLL, true, POL>), dim3(grid), dim3(BLOCK), 0,
                       (hipStream_t)stream, s, nr, nw, n16, static_cast<u32x4*>(sink));
  else
    hipLaunchKernelGGL((probe_kernel<BLOCK, UNROLL, false, POL>), dim3(grid), dim3(BLOCK), 0,
                       (hipStream_t)stream, s, nr, nw, n16, static_cast<u32x4*>(sink));
}

template <int POL>
bool launch_pol(Streams s, int nr, int nw, int64_t n16, int grid, int block, int unroll,
                bool contig, void* sink, void* stream) {
#define PROBE_CASE(B, U) \
  if (block == B && unroll == U) { launch<B, U, POL>(s, nr, nw, n16, grid, contig, sink, stream); return true; }
  PROBE_CASE(256, 1) PROBE_CASE(256, 2) PROBE_CASE(256, 4) PROBE_CASE(256, 8)
  PROBE_CASE(512, 1) PROBE_CASE(512, 2) PROBE_CASE(512, 4) PROBE_CASE(512, 8)
  PROBE_CASE(1024, 1) PROBE_CASE(1024, 2) PROBE_CASE(1024, 4) PROBE_CASE(1024, 8)
#undef PROBE_CASE
  return false;
}

}  // namespace

// stream_probe_policy: the cache-policy bits policy `policy` uses for its
// loads and stores (policy 0: the global nontemporal pair, reported as nt).
extern "C" int stream_probe_policy(int policy, int* load_cpol, int* store_cpol) {
  if (policy < 0 || policy >= kPolicies || !load_cpol || !store_cpol) return -1;
  *load_cpol = load_bits(policy);
  *store_cpol = store_bits(policy);
  return 0;
}

// stream_probe_pol: a chosen workgroup size (256, 512 or 1024), chunks in
// flight per lane and stream (1, 2, 4 or 8), layout (contig != 0: each
// workgroup streams one contiguous range) and cache policy (0..8).
extern "C" int stream_probe_pol(const void* const* reads, int nr, void* const* writes, int nw,
                                int64_t n16, void* sink, int grid, int block, int unroll,
                                int contig, int policy, void* stream) {
  if (nr < 0 || nw < 0 || nr > kMaxStreams || nw > kMaxStreams || n16 < 0 || grid < 1 || !sink ||
      policy < 0 || policy >= kPolicies)
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
  bool ok = false;
  const bool c = contig != 0;
  switch (policy) {
    case 0: ok = launch_pol<0>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 1: ok = launch_pol<1>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 2: ok = launch_pol<2>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 3: ok = launch_pol<3>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 4: ok = launch_pol<4>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 5: ok = launch_pol<5>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 6: ok = launch_pol<6>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 7: ok = launch_pol<7>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
    case 8: ok = launch_pol<8>(s, nr, nw, n16, grid, block, unroll, c, sink, stream); break;
  }
  if (!ok) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

extern "C" int stream_probe_shape(const void* const* reads, int nr, void* const* writes, int nw,
                                  int64_t n16, void* sink, int grid, int block, int unroll,
                                  int contig, void* stream) {
  return stream_probe_pol(reads, nr, writes, nw, n16, sink, grid, block, unroll, contig, 0,
                          stream);
}

extern "C" int stream_probe(const void* const* reads, int nr, void* const* writes, int nw,
                            int64_t n16, void* sink, int grid, void* stream) {
  return stream_probe_shape(reads, nr, writes, nw, n16, sink, grid, kBlock, kUnroll, 0, stream);
}
