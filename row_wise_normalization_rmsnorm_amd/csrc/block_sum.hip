// block_sum.hip -- block all-reduce sum on gfx950, and its C ABI
// (include/block_sum.h).
//
// Method: page "Block All Reduce CUDA代码学习" -- the sum of every element of
// a tensor: widen narrow storage before accumulating (fp32 for floating
// inputs, int32 for int8), reduce within a wave, then across the waves of a
// workgroup, then across workgroups.  The page combines workgroups with an
// atomicAdd of each block's sum into the output; here each workgroup
// publishes its partial and the last one to finish (a completion counter)
// adds the partials in index order, so the fp32 result is reproducible.
//
// MI355X design: a pure HBM read stream.  Every lane loads 16-byte chunks
// (4 f32, 8 f16/bf16, 16 fp8/int8) with the nontemporal policy, four chunks
// in flight per step, in a grid-stride loop over 256 to 512 workgroups of
// 256 threads (a 16384 x 16384 bf16 sum measured 79 us at 512 workgroups,
// 88 at 1024 and 100 at 2048).  fp8 E4M3 decodes by placing its 7 magnitude bits
// in an fp32 and scaling by 2^120 (exact, subnormals included), E5M2 through
// fp16, and int8 chunks sum with v_dot4 against ones.  Wave reductions use
// DPP (quad_perm, row_half_mirror, row_mirror), ds_swizzle SWAP16 and
// readlane; the four wave sums meet in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/block_sum.h"

namespace brs {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;
constexpr int kMaxGroups = BRS_MAX_GROUPS;
constexpr int kMinGroups = 256;        // one per CU
constexpr int kGridCap = 512;          // two per CU: measured best for large inputs
static_assert(kMinGroups <= kGridCap && kGridCap <= kMaxGroups, "grid bounds");
constexpr int kChunksPerThread = 32;   // target share of a thread
// Workspace: completion counters, each on its own 128-byte line -- the top
// counter at line 0 and kSub first-level counters at lines 1..kSub -- then
// one 4-byte partial per workgroup.  Workgroup b reports to counter b % kSub;
// the last arrival of each first-level counter reports to the top one.  A
// single counter would serialise every workgroup's atomic at one address
// (measured about 12.6 ns each, 30 us for 2048 workgroups on MI355X).
constexpr int kSub = 32;
constexpr int kLine = 128;
constexpr int kHeader = BRS_WORKSPACE_HEADER;
static_assert((1 + kSub) * kLine <= kHeader, "counters must fit the header");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---- element decoding ------------------------------------------------------
// Each input type adds one 16-byte chunk (in element order) or one element
// into its accumulator.

template <int DT>
struct In;

template <>
struct In<BRS_F32> {
  using acc_t = float;
  static constexpr int S = 4;
  __device__ static void add_chunk(float& a, u32x4 r) {
    a += as_f(r.x); a += as_f(r.y); a += as_f(r.z); a += as_f(r.w);
  }
  __device__ static void add_elem(float& a, const unsigned char* p) {
    a += *reinterpret_cast<const float*>(p);
  }
};

__device__ __forceinline__ void add_bf16_word(float& a, uint32_t w) {
  a += as_f(w << 16);
  a += as_f(w & 0xffff0000u);
}

template <>
struct In<BRS_BF16> {
  using acc_t = float;
  static constexpr int S = 2;
  __device__ static void add_chunk(float& a, u32x4 r) {
    add_bf16_word(a, r.x); add_bf16_word(a, r.y); add_bf16_word(a, r.z); add_bf16_word(a, r.w);
  }
  __device__ static void add_elem(float& a, const unsigned char* p) {
    a += as_f((uint32_t)*reinterpret_cast<const uint16_t*>(p) << 16);
  }
};

__device__ __forceinline__ void add_f16_word(float& a, uint32_t w) {
  const f32x2 v = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  a += v.x;
  a += v.y;
}

template <>
struct In<BRS_F16> {
  using acc_t = float;
  static constexpr int S = 2;
  __device__ static void add_chunk(float& a, u32x4 r) {
    add_f16_word(a, r.x); add_f16_word(a, r.y); add_f16_word(a, r.z); add_f16_word(a, r.w);
  }
  __device__ static void add_elem(float& a, const unsigned char* p) {
    a += (float)*reinterpret_cast<const _Float16*>(p);
  }
};

// OCP E4M3: the 7 magnitude bits shifted into an fp32 exponent/mantissa read
// as a number 2^-120 times the E4M3 value (bias 7 vs 127), subnormals
// included; S.1111.111 is NaN.
__device__ __forceinline__ float e4m3(uint32_t b) {
  const uint32_t mag = b & 0x7fu;
  const float f = as_f(((b & 0x80u) << 24) | (mag << 20)) * 0x1p120f;
  return mag == 0x7fu ? __builtin_nanf("") : f;
}

// OCP E5M2 is the upper byte of an IEEE binary16.
__device__ __forceinline__ float e5m2(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b << 8));
}

template <>
struct In<BRS_FP8_E4M3> {
  using acc_t = float;
  static constexpr int S = 1;
  __device__ static void add_word(float& a, uint32_t w) {
    a += e4m3(w & 0xffu); a += e4m3((w >> 8) & 0xffu);
    a += e4m3((w >> 16) & 0xffu); a += e4m3(w >> 24);
  }
  __device__ static void add_chunk(float& a, u32x4 r) {
    add_word(a, r.x); add_word(a, r.y); add_word(a, r.z); add_word(a, r.w);
  }
  __device__ static void add_elem(float& a, const unsigned char* p) { a += e4m3(*p); }
};

template <>
struct In<BRS_FP8_E5M2> {
  using acc_t = float;
  static constexpr int S = 1;
  __device__ static void add_word(float& a, uint32_t w) {
    a += e5m2(w & 0xffu); a += e5m2((w >> 8) & 0xffu);
    a += e5m2((w >> 16) & 0xffu); a += e5m2(w >> 24);
  }
  __device__ static void add_chunk(float& a, u32x4 r) {
    add_word(a, r.x); add_word(a, r.y); add_word(a, r.z); add_word(a, r.w);
  }
  __device__ static void add_elem(float& a, const unsigned char* p) { a += e5m2(*p); }
};

// int8: four signed bytes dotted with four ones, into a wrapping int32.
template <>
struct In<BRS_I8> {
  using acc_t = int32_t;
  static constexpr int S = 1;
  __device__ static void add_chunk(int32_t& a, u32x4 r) {
    a = __builtin_amdgcn_sdot4((int)r.x, 0x01010101, a, false);
    a = __builtin_amdgcn_sdot4((int)r.y, 0x01010101, a, false);
    a = __builtin_amdgcn_sdot4((int)r.z, 0x01010101, a, false);
    a = __builtin_amdgcn_sdot4((int)r.w, 0x01010101, a, false);
  }
  __device__ static void add_elem(int32_t& a, const unsigned char* p) {
    a = (int32_t)((uint32_t)a + (uint32_t)(int32_t)*reinterpret_cast<const int8_t*>(p));
  }
};

// ---- reductions --------------------------------------------------------------
__device__ __forceinline__ float add(float x, float y) { return x + y; }
__device__ __forceinline__ int32_t add(int32_t x, int32_t y) {
  return (int32_t)((uint32_t)x + (uint32_t)y);
}

template <int CTRL, typename T>
__device__ __forceinline__ T dpp(T v) {
  return __builtin_bit_cast(
      T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Wave64 sum (every lane combines with a mirror partner, so all agree), as
// a wave-uniform value.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v = add(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = add(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = add(v, dpp<0x141>(v));  // row_half_mirror
  v = add(v, dpp<0x140>(v));  // row_mirror
  v = add(v, __builtin_bit_cast(T, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                0x401F)));  // swap 16
  const T lo = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const T hi = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  return add(lo, hi);
}

// Workgroup sum in a fixed order (wave 0 + wave 1 + wave 2 + wave 3).
template <typename T>
__device__ __forceinline__ T group_sum(T v, T* red) {
  const T w = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  T t = red[0];
#pragma unroll
  for (int j = 1; j < kWaves; ++j) t = add(t, red[j]);
  return t;
}

// ---- the kernel ----------------------------------------------------------------
// Elements [0, head) and [head + 16*nchunks/S ..., n) are added one by one by
// workgroup 0; the middle is nchunks 16-byte chunks starting at x + head*S
// (16-byte aligned).  Workgroup b publishes its sum in partials[b] and then
// counts itself in (two-level counters, above); the workgroup that completes
// the top counter adds partials[0 .. gridDim.x) in order, writes *out, and
// every counter is back at zero when the kernel ends.
template <int DT>
__global__ __launch_bounds__(kThreads) void block_sum_kernel(const unsigned char* x, int64_t n,
                                                             int64_t head, int64_t nchunks,
                                                             void* out, unsigned char* ws) {
  using I = In<DT>;
  using T = typename I::acc_t;
  constexpr int E = 16 / I::S;  // elements per chunk
  __shared__ T red[kWaves];
  __shared__ int last;
  T* partials = reinterpret_cast<T*>(ws + kHeader);
  uint32_t* top = reinterpret_cast<uint32_t*>(ws);
  const int tid = threadIdx.x;

  // Chunk c belongs to workgroup (c / kThreads) % gridDim.x: every
  // workgroup gets an equal share whatever the grid size; each thread keeps
  // kUnroll chunks in flight.
  T acc = T(0);
  const u32x4* v = reinterpret_cast<const u32x4*>(x + head * I::S);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + tid; c0 < nchunks; c0 += stride * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + (int64_t)u * stride;
      if (c < nchunks) r[u] = __builtin_nontemporal_load(v + c);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + (int64_t)u * stride;
      if (c < nchunks) I::add_chunk(acc, r[u]);
    }
  }
  if (blockIdx.x == 0) {
    const int64_t tail0 = head + nchunks * E;
    if (tid < head) I::add_elem(acc, x + (int64_t)tid * I::S);
    if (tail0 + tid < n) I::add_elem(acc, x + (tail0 + tid) * I::S);
  }

  const T mine = group_sum(acc, red);
  if (tid == 0) {
    // Publish the partial with an agent-scope atomic exchange: it is
    // performed at the device-coherent level, and waiting for its returned
    // value (the asm below consumes it) orders it before the counters.  This
    // avoids the whole-L2 writeback that a release fence would cost each
    // workgroup.
    const T prev =
        __hip_atomic_exchange(&partials[blockIdx.x], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("; partial published %0" ::"v"(prev) : "memory");
    const int G = (int)gridDim.x;
    const int grp = (int)blockIdx.x % kSub;
    const uint32_t members = (uint32_t)((G - grp + kSub - 1) / kSub);
    uint32_t* sub = reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(top) +
                                                (1 + grp) * kLine);
    const uint32_t t = __hip_atomic_fetch_add(sub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int is_last = 0;
    if (t == members - 1) {  // every member of this group has reported
      __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t groups = (uint32_t)(G < kSub ? G : kSub);
      const uint32_t t2 = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      is_last = (t2 == groups - 1);
    }
    last = is_last;
  }
  __syncthreads();
  if (!last) return;

  // Every workgroup's exchange completed before it counted itself in, and
  // each group's last arrival counted the group in only after seeing all of
  // its members, so all partials are at the device-coherent level; read them
  // with agent-scope atomic loads after an acquire fence.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  T s = T(0);
  for (int i = tid; i < (int)gridDim.x; i += kThreads)
    s = add(s, __hip_atomic_load(&partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  __syncthreads();  // red[] is reused
  const T total = group_sum(s, red);
  if (tid == 0) {
    *static_cast<T*>(out) = total;
    __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace brs

// Sets the library's per-thread last-error text (rmsnorm_api.hip); returns code.
int rmsn_set_error(int code, const char* msg);

namespace {

int elem_size(int dtype) {
  switch (dtype) {
    case BRS_F32: return 4;
    case BRS_F16:
    case BRS_BF16: return 2;
    default: return 1;
  }
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t p = (uintptr_t)a, q = (uintptr_t)b;
  return p < q + nb && q < p + na;
}

// Tuning override of the grid (block_sum_tune); 0: the size rule below.
std::atomic<int> g_groups_override{0};

template <int DT>
hipError_t launch(const unsigned char* x, int64_t n, void* out, void* ws, hipStream_t stream) {
  constexpr int S = brs::In<DT>::S;
  constexpr int E = 16 / S;
  // elements before the first 16-byte boundary, then whole chunks, then the rest
  int64_t head = (int64_t)((16 - ((uintptr_t)x & 15u)) & 15u) / S;
  if (head > n) head = n;
  const int64_t nchunks = (n - head) / E;
  // Enough workgroups to fill the GPU (at least one per CU) but few enough
  // that each has real work (about kChunksPerThread chunks per thread).
  int64_t groups = nchunks / ((int64_t)brs::kThreads * brs::kChunksPerThread);
  if (groups < brs::kMinGroups) groups = brs::kMinGroups;
  if (groups > brs::kGridCap) groups = brs::kGridCap;
  const int64_t busy = (nchunks + brs::kThreads - 1) / brs::kThreads;  // groups with any chunk
  if (groups > busy) groups = busy < 1 ? 1 : busy;
  if (const int g = g_groups_override.load(std::memory_order_relaxed)) groups = g;
  hipLaunchKernelGGL(brs::block_sum_kernel<DT>, dim3((unsigned)groups), dim3(brs::kThreads), 0,
                     stream, x, n, head, nchunks, out, static_cast<unsigned char*>(ws));
  return hipGetLastError();
}

}  // namespace

// The device-side scratch of block_all_reduce_sum_noalloc: the same layout as
// a caller's workspace (completion counters, then one partial per
// workgroup), one copy per GPU the library runs on, held until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host it
// names a stand-in, not device memory): it passes the device address that
// hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) unsigned char scratch[BRS_WORKSPACE_BYTES];

namespace {

// Zeroes the counter header of a workspace (a kernel, so that it is ordered
// on the caller's stream and may be captured into a graph).
__global__ void clear_header_kernel(uint32_t* ws) {
  for (int i = threadIdx.x; i < BRS_WORKSPACE_HEADER / 4; i += blockDim.x) ws[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];          // device address of `scratch` on each GPU
bool g_scratch_cleared[kMaxDevices];   // its header zeroed on a stream already

// The device address of this GPU's `scratch`, looked up once per device with
// that device current; on the first call for a device the counter header is
// zeroed by a small kernel on `stream`, ahead of the sum.  Returns nullptr
// (and sets the last error) on failure.
void* scratch_for(int dev, hipStream_t stream) {
  if (dev < 0 || dev >= kMaxDevices) {
    rmsn_set_error(RMSN_ERR_HIP, "device index outside the scratch table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      rmsn_set_error(RMSN_ERR_HIP, "hipGetDevice failed");
      return nullptr;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      rmsn_set_error(RMSN_ERR_HIP, "hipSetDevice failed");
      return nullptr;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      char msg[200];
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      rmsn_set_error(RMSN_ERR_HIP, msg);
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  if (!g_scratch_cleared[dev]) {
    hipLaunchKernelGGL(clear_header_kernel, dim3(1), dim3(256), 0, stream,
                       static_cast<uint32_t*>(g_scratch[dev]));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      char msg[200];
      snprintf(msg, sizeof(msg), "clearing the scratch counters failed: %s", hipGetErrorString(e));
      rmsn_set_error(RMSN_ERR_HIP, msg);
      return nullptr;
    }
    g_scratch_cleared[dev] = true;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int block_sum_tune(int groups) {
  if (groups < 0 || groups > brs::kMaxGroups)
    return rmsn_set_error(RMSN_ERR_SHAPE, "groups outside [0, BRS_MAX_GROUPS]");
  g_groups_override.store(groups, std::memory_order_relaxed);
  return RMSN_OK;
}

extern "C" int block_all_reduce_sum(void* out, const void* x, int64_t n, int dtype,
                                    void* workspace, int64_t workspace_bytes, void* stream) {
  if (dtype < BRS_F32 || dtype > BRS_I8) return rmsn_set_error(RMSN_ERR_DTYPE, "unknown sum dtype");
  if (n < 0) return rmsn_set_error(RMSN_ERR_SHAPE, "n < 0");
  if (!out || !workspace || (n > 0 && !x))
    return rmsn_set_error(RMSN_ERR_NULL, "out, workspace and x must be non-NULL");
  const int s = elem_size(dtype);
  if (((uintptr_t)x % (uintptr_t)s) != 0)
    return rmsn_set_error(RMSN_ERR_SHAPE, "x is not aligned to its element size");
  if (workspace_bytes < BRS_WORKSPACE_BYTES || ((uintptr_t)workspace & 15u))
    return rmsn_set_error(RMSN_ERR_SHAPE, "workspace smaller than BRS_WORKSPACE_BYTES or unaligned");
  const size_t xb = (size_t)n * (size_t)s;
  const size_t ob = dtype == BRS_I8 ? sizeof(int32_t) : sizeof(float);
  if (overlap(out, ob, workspace, BRS_WORKSPACE_BYTES) || (n > 0 && overlap(out, ob, x, xb)) ||
      (n > 0 && overlap(workspace, BRS_WORKSPACE_BYTES, x, xb)))
    return rmsn_set_error(RMSN_ERR_ALIAS, "out, workspace and x must not overlap");
  const unsigned char* xp = static_cast<const unsigned char*>(x);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (dtype) {
    case BRS_F32: e = launch<BRS_F32>(xp, n, out, workspace, st); break;
    case BRS_F16: e = launch<BRS_F16>(xp, n, out, workspace, st); break;
    case BRS_BF16: e = launch<BRS_BF16>(xp, n, out, workspace, st); break;
    case BRS_FP8_E4M3: e = launch<BRS_FP8_E4M3>(xp, n, out, workspace, st); break;
    case BRS_FP8_E5M2: e = launch<BRS_FP8_E5M2>(xp, n, out, workspace, st); break;
    default: e = launch<BRS_I8>(xp, n, out, workspace, st); break;
  }
  if (e != hipSuccess) {
    char msg[200];
    snprintf(msg, sizeof(msg), "block_all_reduce_sum launch failed: %s", hipGetErrorString(e));
    return rmsn_set_error(RMSN_ERR_HIP, msg);
  }
  return RMSN_OK;
}

extern "C" int block_all_reduce_sum_noalloc(void* out, const void* x, int64_t n, int dtype,
                                            void* stream) {
  // arguments first, exactly as the workspace form checks them (nothing is
  // set up or launched for a call that would be rejected)
  if (dtype < BRS_F32 || dtype > BRS_I8) return rmsn_set_error(RMSN_ERR_DTYPE, "unknown sum dtype");
  if (n < 0) return rmsn_set_error(RMSN_ERR_SHAPE, "n < 0");
  if (!out || (n > 0 && !x)) return rmsn_set_error(RMSN_ERR_NULL, "out and x must be non-NULL");
  if (n > INT64_MAX / 4) return rmsn_set_error(RMSN_ERR_SHAPE, "n too large");
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[200];
    snprintf(msg, sizeof(msg), "cannot tell the stream's device: %s", hipGetErrorString(e));
    return rmsn_set_error(RMSN_ERR_HIP, msg);
  }
  void* ws = scratch_for(dev, (hipStream_t)stream);
  if (!ws) return RMSN_ERR_HIP;
  // The launch never uses more than BRS_MAX_GROUPS partials, which the
  // scratch holds, so every n fits; the workspace form's checks do the rest.
  return block_all_reduce_sum(out, x, n, dtype, ws, (int64_t)sizeof(scratch), stream);
}
