// rmsnorm_kernels.hpp -- gfx950 (CDNA4, wave64) kernels for row-wise RMSNorm and
// the fused "K partials + residual -> residual in place -> RMSNorm" form.
//
// Method: page "RMSNorm kernel", section 1 Background and section 2
// "Abstraction" (per-row sum of squares -> mean -> + eps -> rsqrt; then
// x * gamma * rsqrt), and page "Tokenweave fused-RMSNorm-AR kernel", "Code
// walkthrough" (partials + residual summed, residual written back in place,
// fp32 sum of squares of the stored values, then residual * scale * weight).
//
// The path is bound by HBM bandwidth (no contraction, so no MFMA).  Design:
//   * 128-bit global loads/stores (global_load_dwordx4): 8 bf16/fp16 or 4 fp32
//     elements per lane per access, a wave covering 1 KiB contiguous.  Rows
//     whose byte length or base alignment only allows 8- or 4-byte accesses
//     use those widths; only what no 4-byte access divides goes element-wise.
//   * row_vgpr: the whole row lives in VGPRs between the two phases, so every
//     input byte is read from HBM exactly once and the normalised output is
//     produced from registers.  Threads-per-row (TPR) is a template choice:
//     TPR < 64 packs several rows into one wave (segmented DPP reduction),
//     TPR = 64 is a row per wave (no LDS, no barrier), TPR > 64 spreads a row
//     over several waves of one workgroup (DPP within waves, then LDS).
//   * row_stream: two passes over a row of any length.  Pass 1 streams the
//     inputs and stages the rounded row in LDS (or, when it does not fit,
//     re-reads the thread's own freshly written residual / input in pass 2).
//   * Reductions: fp32; within a wave by DPP (quad_perm, row_half_mirror,
//     row_mirror) and ds_swizzle SWAP16, and readlane for the two 32-lane
//     halves; across waves through a small double-buffered LDS array that
//     every wave sums in the same fixed order, so all waves agree bitwise.
//   * Conversions: bf16 widening is a shift; narrowing uses gfx950's
//     v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 (round to nearest even, the
//     rounding the stored residual must reproduce exactly).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rmsn {

constexpr int kMaxK = 16;

// Row-major tensors addressed per row: row r of a tensor starts at
// base + r * stride bytes, and its hidden elements are contiguous.
struct PartialPtrs {
  const void* p[kMaxK];
  int64_t s[kMaxK];      // row strides in bytes
};

struct RowArgs {
  void* out;
  int64_t out_stride;    // bytes
  void* residual;        // nullptr for plain RMSNorm
  int64_t res_stride;    // bytes
  PartialPtrs partials;  // partials.p[0] is x for plain RMSNorm
  const void* gamma;
  int64_t rows;
  int hidden;            // elements per row
  int chunks;            // chunks per row (E elements each, see Vec)
  int k;                 // number of partials (fused), 1 for plain
  float eps;
};

// The fused form with an all-gather epilogue (AG kernels): every normalised
// row is stored at the same row of each of the n gather buffers, with out's
// row pitch, instead of into out.
struct GatherPtrs {
  void* p[kMaxK];
  int n;
};
struct RowArgsAG : RowArgs {
  GatherPtrs gather;
};
template <bool AG>
using ArgsOf = typename std::conditional<AG, RowArgsAG, RowArgs>::type;

__device__ __forceinline__ const char* row_ptr(const void* base, int64_t stride, int64_t row) {
  return reinterpret_cast<const char*>(base) + row * stride;
}
__device__ __forceinline__ char* row_ptr(void* base, int64_t stride, int64_t row) {
  return reinterpret_cast<char*>(base) + row * stride;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---- storage types -------------------------------------------------------
// Each dtype converts one 32-bit word of storage (one fp32, or two packed
// 16-bit values) to and from fp32, and one scalar element.  Narrowing rounds
// to nearest even.

template <typename T>
struct DT;

template <>
struct DT<float> {
  static constexpr int PER_WORD = 1;
  using scalar_t = float;
  __device__ static void unpack_word(uint32_t u, float* f) { f[0] = as_f(u); }
  __device__ static uint32_t pack_word(const float* f) { return as_u(f[0]); }
  __device__ static float widen(scalar_t s) { return s; }
  __device__ static scalar_t narrow(float f) { return f; }
};

template <>
struct DT<__bf16> {
  static constexpr int PER_WORD = 2;
  using scalar_t = uint16_t;
  __device__ static void unpack_word(uint32_t u, float* f) {
    f[0] = as_f(u << 16);
    f[1] = as_f(u & 0xffff0000u);
  }
  __device__ static uint32_t pack_word(const float* f) {
    f32x2 v = {f[0], f[1]};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  __device__ static float widen(scalar_t s) { return as_f((uint32_t)s << 16); }
  __device__ static scalar_t narrow(float f) {
    const float two[2] = {f, 0.0f};
    return (scalar_t)(pack_word(two) & 0xffffu);
  }
};

template <>
struct DT<_Float16> {
  static constexpr int PER_WORD = 2;
  using scalar_t = uint16_t;
  __device__ static void unpack_word(uint32_t u, float* f) {
    f32x2 v = __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
    f[0] = v.x;
    f[1] = v.y;
  }
  __device__ static uint32_t pack_word(const float* f) {
    f32x2 v = {f[0], f[1]};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  __device__ static float widen(scalar_t s) { return (float)__builtin_bit_cast(_Float16, s); }
  __device__ static scalar_t narrow(float f) { return __builtin_bit_cast(scalar_t, (_Float16)f); }
};

// Groups of W 32-bit words moved by one load or store instruction.
template <int W>
struct Words;
template <>
struct Words<1> {
  using type = uint32_t;
  __device__ static uint32_t get(type v, int) { return v; }
  __device__ static void set(type& v, int, uint32_t x) { v = x; }
};
template <>
struct Words<2> {
  typedef uint32_t type __attribute__((ext_vector_type(2)));
  __device__ static uint32_t get(type v, int i) { return v[i]; }
  __device__ static void set(type& v, int i, uint32_t x) { v[i] = x; }
};
template <>
struct Words<4> {
  typedef uint32_t type __attribute__((ext_vector_type(4)));
  __device__ static uint32_t get(type v, int i) { return v[i]; }
  __device__ static void set(type& v, int i, uint32_t x) { v[i] = x; }
};

// A "chunk" is E consecutive elements of a row, moved by one lane.  The
// kernels pick E from the data dtype and an access width VB (16, 8 or 4
// bytes: a global_load/store_dwordx4, dwordx2 or dword; 0: one element, for
// bases or row lengths that no wider access divides).  gamma and the output
// may have other dtypes: their chunk is then E elements of their own type,
// e.g. 32 bytes (two 16-byte accesses) of fp32 output for a 16-byte bf16
// input chunk, or 8 bytes of bf16 output for a 16-byte fp32 chunk.
// NT selects the nontemporal (streaming) cache policy for data that is
// touched exactly once; gamma, reused by every row, is loaded normally.
template <typename T, int E>
struct Vec {
  static constexpr int V = E;
  static constexpr int BYTES = E * (int)sizeof(typename DT<T>::scalar_t);
  static_assert(BYTES == 2 || BYTES % 4 == 0, "a chunk is one 16-bit element or whole words");
  static constexpr int W = BYTES / 4;                  // 32-bit words per chunk
  static constexpr int AW = W >= 4 ? 4 : (W > 0 ? W : 1);  // words per access
  static constexpr int N = W >= 4 ? W / 4 : 1;         // accesses per chunk
  static_assert(W <= 4 || W % 4 == 0, "wide chunks are whole 16-byte accesses");
  static constexpr bool SCALAR = BYTES == 2;
  using WS = Words<AW>;
  using acc_t = typename std::conditional<SCALAR, typename DT<T>::scalar_t,
                                          typename WS::type>::type;
  struct raw_t {
    acc_t w[N];
  };
  template <bool NT = false>
  __device__ static raw_t load(const void* row, int c) {
    const acc_t* p = reinterpret_cast<const acc_t*>(row) + (int64_t)c * N;
    raw_t r;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if constexpr (NT) r.w[n] = __builtin_nontemporal_load(p + n); else r.w[n] = p[n];
    }
    return r;
  }
  template <bool NT = false>
  __device__ static void store(void* row, int c, const raw_t& r) {
    acc_t* p = reinterpret_cast<acc_t*>(row) + (int64_t)c * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if constexpr (NT) __builtin_nontemporal_store(r.w[n], p + n); else p[n] = r.w[n];
    }
  }
  // The same chunk through a buffer resource `rs` that covers one row of one
  // tensor from a wave-uniform base (chunk c at byte offset c * BYTES), with
  // the cache-policy bits CPOL on the instruction.  Chunks of whole 32-bit
  // words only.
  static constexpr bool BUFFERABLE = !SCALAR;
  template <int CPOL>
  __device__ static raw_t load_buf(__amdgpu_buffer_rsrc_t rs, int c) {
    static_assert(BUFFERABLE, "buffer access moves whole words");
    raw_t r;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int off = c * BYTES + n * AW * 4;
      if constexpr (AW == 4) r.w[n] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL);
      else if constexpr (AW == 2) r.w[n] = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, CPOL);
      else r.w[n] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, CPOL);
    }
    return r;
  }
  template <int CPOL>
  __device__ static void store_buf(__amdgpu_buffer_rsrc_t rs, int c, const raw_t& r) {
    static_assert(BUFFERABLE, "buffer access moves whole words");
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int off = c * BYTES + n * AW * 4;
      if constexpr (AW == 4) __builtin_amdgcn_raw_buffer_store_b128(r.w[n], rs, off, 0, CPOL);
      else if constexpr (AW == 2) __builtin_amdgcn_raw_buffer_store_b64(r.w[n], rs, off, 0, CPOL);
      else __builtin_amdgcn_raw_buffer_store_b32(r.w[n], rs, off, 0, CPOL);
    }
  }
  __device__ static void unpack(const raw_t& r, float (&f)[V]) {
    if constexpr (SCALAR) {
      f[0] = DT<T>::widen(r.w[0]);
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int w = 0; w < AW; ++w)
          DT<T>::unpack_word(WS::get(r.w[n], w), f + (n * AW + w) * DT<T>::PER_WORD);
    }
  }
  __device__ static raw_t pack(const float (&f)[V]) {
    raw_t r;
    if constexpr (SCALAR) {
      r.w[0] = DT<T>::narrow(f[0]);
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int w = 0; w < AW; ++w)
          WS::set(r.w[n], w, DT<T>::pack_word(f + (n * AW + w) * DT<T>::PER_WORD));
    }
    return r;
  }
};

// Elements per chunk for data type T and access width VB (0: one element).
template <typename T, int VB>
constexpr int chunk_elems() {
  return VB == 0 ? 1 : VB / (int)sizeof(typename DT<T>::scalar_t);
}

// ---- streaming row access through buffer resources ------------------------
// Rows of data touched exactly once are moved with buffer_load/store_dwordx4
// (dwordx2, dword for narrower chunks) from a wave-uniform row base held in
// scalar registers, with explicit cache-policy bits.  Loads are nontemporal
// (nt).  The register kernel stores nontemporal at system scope (sc0 sc1
// nt: written through to memory, no dirty lines left in L2) and writes the
// residual back after the row reduction, next to the output: 667 vs 683 us
// for 131072 x 4096 bf16 rows (K = 1) against global nt accesses with the
// residual stored first, and equal on 8192 rows.  The streaming kernel
// keeps plain nontemporal stores and its residual store in pass 1: at K = 8
// (4096 x 8192) system-scope stores or a residual stored in pass 2 measured
// 117.6-119.5 us against 113.7, and 1455-1471 against 1415 us on 65536 x
// 16384.  No other combination of the sc0 / sc1 / nt bits did better once
// the footprint exceeded the 256 MB Infinity Cache.
constexpr int kCpolLoadStream = 2;        // nt
constexpr int kCpolStoreStream = 2;       // nt
constexpr int kCpolStoreWriteThrough = 19;  // sc0 | nt | sc1

// A buffer resource over `bytes` bytes from `base` (which must be uniform
// across the wave): raw 32-bit words, stride 0; accesses at or beyond
// `bytes` would read zeros and drop stores (every access here is in range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// ---- wave64 reductions ----------------------------------------------------
// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm:[1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kSwizzleSwap16 = 0x401F;  // ds_swizzle bit mode: xor 16 within 32 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_get(float v) {
  return as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ __forceinline__ float combine(float x, float y) {
  if constexpr (MAX) return fmaxf(x, y); else return x + y;
}

// Sum (or max) over aligned groups of G lanes (G in {1,2,4,8,16,32}); every
// lane of the group receives the result.  Each step combines a value with
// its mirror partner, so partners compute a+b and b+a: all lanes agree
// bitwise.
template <int G, bool MAX = false>
__device__ __forceinline__ float group_reduce(float v) {
  if constexpr (G >= 2) v = combine<MAX>(v, dpp_get<kDppQuadXor1>(v));
  if constexpr (G >= 4) v = combine<MAX>(v, dpp_get<kDppQuadXor2>(v));
  if constexpr (G >= 8) v = combine<MAX>(v, dpp_get<kDppRowHalfMirror>(v));
  if constexpr (G >= 16) v = combine<MAX>(v, dpp_get<kDppRowMirror>(v));
  if constexpr (G >= 32)
    v = combine<MAX>(v, as_f((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_u(v), kSwizzleSwap16)));
  return v;
}

// Sum (or max) over the full wave, returned as a wave-uniform value.
template <bool MAX = false>
__device__ __forceinline__ float wave_reduce(float v) {
  v = group_reduce<32, MAX>(v);
  const float lo = as_f((uint32_t)__builtin_amdgcn_readlane((int)as_u(v), 0));
  const float hi = as_f((uint32_t)__builtin_amdgcn_readlane((int)as_u(v), 32));
  return combine<MAX>(lo, hi);
}

// Reduction over the TPR threads of a row: within a lane group (TPR < 64),
// within a wave (TPR == 64), or across the WPR waves of a row through the
// double-buffered LDS array red[2][RPW * WPR] (one barrier).  Every wave
// combines the wave results in the same order, so all agree bitwise.  A
// buffer is rewritten only after a later reduction's barrier, which no wave
// passes before every wave has read it.
template <int TPR, int WPR, int N, bool MAX>
__device__ __forceinline__ float row_reduce(float x, float (&red)[2][N], int& parity, int slot,
                                            int tr) {
  if constexpr (TPR < 64) {
    return group_reduce<TPR, MAX>(x);
  } else if constexpr (WPR == 1) {
    return wave_reduce<MAX>(x);
  } else {
    const float ws = wave_reduce<MAX>(x);
    if ((tr & 63) == 0) red[parity][slot * WPR + tr / 64] = ws;
    __syncthreads();
    float t = red[parity][slot * WPR];
#pragma unroll
    for (int j = 1; j < WPR; ++j) t = combine<MAX>(t, red[parity][slot * WPR + j]);
    parity ^= 1;
    return t;
  }
}

// ---- per-row scale ---------------------------------------------------------
// inv = rsqrt(sum/hidden + eps): eps inside the root, after the mean.
__device__ __forceinline__ float row_scale(float ss, int hidden, float eps) {
  return rsqrtf(ss / (float)hidden + eps);
}

// The fp32 sum of squares leaves binary32's useful range for rows of huge
// values (it overflows to +inf) and for rows of tiny values (their squares
// underflow).  Such a row is rescaled by an exact power of two, 2^-e with
// 2^e just above its largest magnitude, and normalised as
//   y = ((x * 2^-e) * rsqrt(sum((x * 2^-e)^2)/hidden + eps * 2^-2e)) * gamma,
// which is the same quantity.  A row of zeros with eps > 0 is exact as is.
__device__ __forceinline__ bool needs_rescale(float tot, float eps) {
  return tot == __builtin_inff() || (tot < 0x1p-60f && (tot > 0.0f || eps == 0.0f));
}

// Having the row's largest magnitude m and its rescaled sum of squares tot2,
// return true and the rescaled (inv, shift) if the rescaled form applies; a
// row holding inf, a row of zeros, or one whose eps * 2^-2e overflows (eps
// then dominates and the plain form is accurate) keeps the plain form.
__device__ __forceinline__ bool rescaled_scale(float m, float tot2, int e, int hidden, float eps,
                                               float& inv, int& shift) {
  if (!(m > 0.0f) || m == __builtin_inff()) return false;
  const float eps2 = ldexpf(eps, -2 * e);
  if (eps2 == __builtin_inff()) return false;
  inv = rsqrtf(tot2 / (float)hidden + eps2);
  shift = -e;
  return true;
}

__device__ __forceinline__ int exponent_above(float m) {
  int e = 0;
  (void)frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
  return e;
}

// ---- kernel 1: the row held in VGPRs ---------------------------------------
// TPR threads per row, NPT chunks per thread (chunk c of a row belongs to
// thread c % TPR), WGS threads per workgroup (WGS / TPR rows per workgroup).
// KC: 0 = plain RMSNorm; >0 = fused with exactly KC partials; -1 = fused with
// a runtime number of partials (args.k), summed one partial at a time.
// NT: streaming (nontemporal) loads and stores for the row data.
// AG: store each output row into every gather buffer (RowArgsAG) instead of
// out.
template <typename T, typename GT, typename OT, int TPR, int NPT, int WGS, int KC, bool NT,
          bool AG = false>
__global__ __launch_bounds__(WGS) void row_vgpr_kernel(ArgsOf<AG> a) {
  constexpr int V = chunk_elems<T, 16>();
  using IV = Vec<T, V>;   // data: partials, residual, x
  using GV = Vec<GT, V>;  // gamma
  using OV = Vec<OT, V>;  // output
  using raw_t = typename IV::raw_t;
  constexpr int RPW = WGS / TPR;                // rows per workgroup
  constexpr int WPR = TPR > 64 ? TPR / 64 : 1;  // waves per row
  static_assert(TPR <= WGS && WGS % TPR == 0, "a row must fit in one workgroup");
  static_assert(TPR < 64 ? (64 % TPR == 0) : (TPR % 64 == 0), "TPR must tile waves");
  constexpr int kRed = WPR > 1 ? RPW * WPR : 1;
  // streaming rows whose base is uniform over a wave go through buffer
  // resources (rows packed several to a wave keep global accesses)
  constexpr bool BUF = NT && TPR >= 64;
  __shared__ float red[2][kRed];

  const int tid = threadIdx.x;
  const int tr = tid % TPR;  // thread index within its row
  const int slot = tid / TPR;
  const int C = a.chunks;
  int parity = 0;

  // gamma chunks are the same for every row this thread touches
  float g[NPT][V];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int c = tr + i * TPR;
    if (c < C) {
      GV::unpack(GV::template load<false>(a.gamma, c), g[i]);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) g[i][e] = 0.0f;
    }
  }

  for (int64_t row0 = (int64_t)blockIdx.x * RPW; row0 < a.rows;
       row0 += (int64_t)gridDim.x * RPW) {
    // uniform when one row per workgroup, and made explicitly wave-uniform
    // when a row spans whole waves (the buffer path needs a scalar base)
    const int64_t row = RPW == 1 ? row0 : row0 + (BUF ? __builtin_amdgcn_readfirstlane(slot) : slot);
    const bool row_ok = row < a.rows;
    const char* xrow = row_ptr(a.partials.p[0], a.partials.s[0], row);
    char* rrow = row_ptr(a.residual, a.res_stride, row);
    char* orow = row_ptr(a.out, a.out_stride, row);
    // chunk c of a data row: nontemporal, through a buffer resource when
    // the row base is wave-uniform
    auto load_in = [&](const char* rowp, int c) -> raw_t {
      if constexpr (BUF) return IV::template load_buf<kCpolLoadStream>(row_rsrc(rowp, C * IV::BYTES), c);
      else return IV::template load<NT>(rowp, c);
    };
    float v[NPT][V];
    raw_t rnew[NPT];  // the rounded residual chunks, stored after the reduction

    if constexpr (KC == 0) {
      raw_t raw[NPT];
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tr + i * TPR;
        if (row_ok && c < C) raw[i] = load_in(xrow, c);
      }
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tr + i * TPR;
        if (row_ok && c < C) {
          IV::unpack(raw[i], v[i]);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) v[i][e] = 0.0f;
        }
      }
    } else {
      constexpr int NB = KC > 0 ? KC : 1;  // partial buffers loaded up front
      raw_t raw[NB][NPT];
      raw_t rres[NPT];
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tr + i * TPR;
        if (row_ok && c < C) {
#pragma unroll
          for (int q = 0; q < NB; ++q)
            raw[q][i] = load_in(row_ptr(a.partials.p[q], a.partials.s[q], row), c);
          rres[i] = load_in(rrow, c);
        }
      }
      float acc[NPT][V];
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tr + i * TPR;
        if (row_ok && c < C) {
          IV::unpack(raw[0][i], acc[i]);  // accumulator seeded with p0
#pragma unroll
          for (int q = 1; q < NB; ++q) {
            float t[V];
            IV::unpack(raw[q][i], t);
#pragma unroll
            for (int e = 0; e < V; ++e) acc[i][e] += t[e];
          }
        }
      }
      if constexpr (KC < 0) {
        // runtime K: remaining partials one at a time, in order
        for (int q = 1; q < a.k; ++q) {
          raw_t rq[NPT];
          const char* prow = row_ptr(a.partials.p[q], a.partials.s[q], row);
#pragma unroll
          for (int i = 0; i < NPT; ++i) {
            const int c = tr + i * TPR;
            if (row_ok && c < C) rq[i] = load_in(prow, c);
          }
#pragma unroll
          for (int i = 0; i < NPT; ++i) {
            const int c = tr + i * TPR;
            if (row_ok && c < C) {
              float t[V];
              IV::unpack(rq[i], t);
#pragma unroll
              for (int e = 0; e < V; ++e) acc[i][e] += t[e];
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tr + i * TPR;
        if (row_ok && c < C) {
          float t[V];
          IV::unpack(rres[i], t);
#pragma unroll
          for (int e = 0; e < V; ++e) acc[i][e] += t[e];  // residual added last
          rnew[i] = IV::pack(acc[i]);                    // round once to dtype
          IV::unpack(rnew[i], v[i]);                     // normalise the stored row
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) v[i][e] = 0.0f;
        }
      }
    }

    // sum of squares of this thread's elements (fp32)
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NPT; ++i)
#pragma unroll
      for (int e = 0; e < V; ++e) ss = __builtin_fmaf(v[i][e], v[i][e], ss);

    const float tot = row_reduce<TPR, WPR, kRed, false>(ss, red, parity, slot, tr);
    float inv = row_scale(tot, a.hidden, a.eps);
    int shift = 0;

    // Rare: rescale rows whose sum of squares left fp32's range.  The
    // decision is uniform over everything that takes part in the extra
    // reductions: a lane group or a wave, or (several waves per row) the
    // whole workgroup, which then rescales if any of its rows needs it.
    bool wide = row_ok && needs_rescale(tot, a.eps);
    bool take = wide;
    if constexpr (WPR > 1 && RPW > 1) {
      const int used = parity ^ 1;  // the buffer the sum just went through
      take = false;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        float t = red[used][r * WPR];
#pragma unroll
        for (int j = 1; j < WPR; ++j) t += red[used][r * WPR + j];
        take = take || (row0 + r < a.rows && needs_rescale(t, a.eps));
      }
    }
    if (take) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < NPT; ++i)
#pragma unroll
        for (int e = 0; e < V; ++e) m = fmaxf(m, fabsf(v[i][e]));
      m = row_reduce<TPR, WPR, kRed, true>(m, red, parity, slot, tr);
      const int ex = exponent_above(m);
      float ss2 = 0.0f;
#pragma unroll
      for (int i = 0; i < NPT; ++i)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float t = ldexpf(v[i][e], -ex);
          ss2 = __builtin_fmaf(t, t, ss2);
        }
      const float tot2 = row_reduce<TPR, WPR, kRed, false>(ss2, red, parity, slot, tr);
      if (wide) {
        float inv2;
        int sh2;
        if (rescaled_scale(m, tot2, ex, a.hidden, a.eps, inv2, sh2)) {
          inv = inv2;
          shift = sh2;
        }
      }
    }

    // The residual is written back here, after the reduction, next to the
    // output: each workgroup's loads, then its stores (measured 1.7% faster
    // than storing it before the reduction on a 4 GiB footprint, equal on
    // 256 MiB).
    if constexpr (KC != 0) {
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tr + i * TPR;
        if (row_ok && c < C) {
          if constexpr (BUF)
            IV::template store_buf<kCpolStoreWriteThrough>(row_rsrc(rrow, C * IV::BYTES), c, rnew[i]);
          else
            IV::template store<NT>(rrow, c, rnew[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tr + i * TPR;
      if (row_ok && c < C) {
        float y[V];
        if (shift == 0) {
#pragma unroll
          for (int e = 0; e < V; ++e) y[e] = (v[i][e] * inv) * g[i][e];
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) y[e] = (ldexpf(v[i][e], shift) * inv) * g[i][e];
        }
        const auto packed = OV::pack(y);
        if constexpr (AG) {
          for (int j = 0; j < a.gather.n; ++j) {
            char* grow = row_ptr(a.gather.p[j], a.out_stride, row);
            if constexpr (BUF)
              OV::template store_buf<kCpolStoreWriteThrough>(row_rsrc(grow, C * OV::BYTES), c, packed);
            else
              OV::template store<NT>(grow, c, packed);
          }
        } else {
          if constexpr (BUF)
            OV::template store_buf<kCpolStoreWriteThrough>(row_rsrc(orow, C * OV::BYTES), c, packed);
          else
            OV::template store<NT>(orow, c, packed);
        }
      }
    }
  }
}

// ---- kernel 2: streaming two-pass row (any length) -------------------------
// One row per workgroup of WGS threads, in VB-byte chunks (0: one element).
// Pass 1 reads the inputs chunk by chunk (UNR chunks in flight per thread),
// writes the residual, accumulates the sum of squares and keeps the rounded
// row: in LDS when LDS_STAGE, else pass 2 re-reads what this same thread
// wrote (fused) or read (plain) -- a thread only ever touches its own chunks,
// so no barrier guards the stage.
// KC: 0 = plain; 1 = one partial; -1 = runtime K, the partials after p0
// loaded and added one at a time; -2 = runtime K, two at a time (both loads
// in flight together, the adds still in order).
// NT: streaming loads/stores for data touched once (never for a residual
// that pass 2 reads back from memory), through buffer resources for chunks
// of whole words.
// AG: as for the register kernel.
template <typename T, typename GT, typename OT, int VB, int WGS, bool LDS_STAGE, int KC, int UNR,
          bool NT, bool AG = false>
__global__ __launch_bounds__(WGS) void row_stream_kernel(ArgsOf<AG> a) {
  constexpr int V = chunk_elems<T, VB>();
  using IV = Vec<T, V>;   // data: partials, residual, x
  using GV = Vec<GT, V>;  // gamma
  using OV = Vec<OT, V>;  // output
  using raw_t = typename IV::raw_t;
  constexpr int NW = WGS / 64;
  constexpr bool BUF = NT && IV::BUFFERABLE && OV::BUFFERABLE;
  __shared__ float red[2][NW];
  extern __shared__ __align__(16) unsigned char stage_bytes[];
  raw_t* stage = reinterpret_cast<raw_t*>(stage_bytes);

  const int tid = threadIdx.x;
  const int C = a.chunks;
  int parity = 0;

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const char* xrow = row_ptr(a.partials.p[0], a.partials.s[0], row);
    char* rrow = row_ptr(a.residual, a.res_stride, row);
    char* orow = row_ptr(a.out, a.out_stride, row);
    float ss = 0.0f;
    auto load_in = [&](const char* rowp, int c) -> raw_t {
      if constexpr (BUF) return IV::template load_buf<kCpolLoadStream>(row_rsrc(rowp, C * IV::BYTES), c);
      else return IV::template load<NT>(rowp, c);
    };

    for (int c0 = tid; c0 < C; c0 += WGS * UNR) {
      raw_t rv[UNR];
      if constexpr (KC == 0) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int c = c0 + u * WGS;
          if (c < C) rv[u] = load_in(xrow, c);
        }
      } else {
        raw_t r0[UNR], rr[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int c = c0 + u * WGS;
          if (c < C) {
            r0[u] = load_in(xrow, c);
            rr[u] = load_in(rrow, c);
          }
        }
        float acc[UNR][V];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int c = c0 + u * WGS;
          if (c < C) IV::unpack(r0[u], acc[u]);
        }
        const int K = KC > 0 ? KC : a.k;
        int q = 1;
        if constexpr (KC == -2) {
          // two partials per step, still added in order
          for (; q + 1 < K; q += 2) {
            raw_t ra[UNR], rb[UNR];
            const char* pa = row_ptr(a.partials.p[q], a.partials.s[q], row);
            const char* pb = row_ptr(a.partials.p[q + 1], a.partials.s[q + 1], row);
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
              const int c = c0 + u * WGS;
              if (c < C) {
                ra[u] = load_in(pa, c);
                rb[u] = load_in(pb, c);
              }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
              const int c = c0 + u * WGS;
              if (c < C) {
                float t[V], t2[V];
                IV::unpack(ra[u], t);
                IV::unpack(rb[u], t2);
#pragma unroll
                for (int e = 0; e < V; ++e) acc[u][e] = (acc[u][e] + t[e]) + t2[e];
              }
            }
          }
        }
        for (; q < K; ++q) {
          raw_t rq[UNR];
          const char* prow = row_ptr(a.partials.p[q], a.partials.s[q], row);
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const int c = c0 + u * WGS;
            if (c < C) rq[u] = load_in(prow, c);
          }
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const int c = c0 + u * WGS;
            if (c < C) {
              float t[V];
              IV::unpack(rq[u], t);
#pragma unroll
              for (int e = 0; e < V; ++e) acc[u][e] += t[e];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int c = c0 + u * WGS;
          if (c < C) {
            float t[V];
            IV::unpack(rr[u], t);
#pragma unroll
            for (int e = 0; e < V; ++e) acc[u][e] += t[e];
            rv[u] = IV::pack(acc[u]);
            IV::template store<NT && LDS_STAGE>(rrow, c, rv[u]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + u * WGS;
        if (c < C) {
          float t[V];
          IV::unpack(rv[u], t);
#pragma unroll
          for (int e = 0; e < V; ++e) ss = __builtin_fmaf(t[e], t[e], ss);
          if constexpr (LDS_STAGE) stage[c] = rv[u];
        }
      }
    }

    const float tot = row_reduce<WGS, NW, NW, false>(ss, red, parity, 0, tid);
    float inv = row_scale(tot, a.hidden, a.eps);
    int shift = 0;
    const char* src = KC == 0 ? xrow : rrow;
    // this thread's chunk c of the stored row, from the stage or memory
    auto own = [&](int c) -> raw_t {
      if constexpr (LDS_STAGE) return stage[c]; else return IV::template load<false>(src, c);
    };

    // Rare: rescale a row whose sum of squares left fp32's range (the whole
    // workgroup holds one row, so the branch is uniform).
    if (needs_rescale(tot, a.eps)) {
      float m = 0.0f;
      for (int c = tid; c < C; c += WGS) {
        float t[V];
        IV::unpack(own(c), t);
#pragma unroll
        for (int e = 0; e < V; ++e) m = fmaxf(m, fabsf(t[e]));
      }
      m = row_reduce<WGS, NW, NW, true>(m, red, parity, 0, tid);
      const int ex = exponent_above(m);
      float ss2 = 0.0f;
      for (int c = tid; c < C; c += WGS) {
        float t[V];
        IV::unpack(own(c), t);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float q = ldexpf(t[e], -ex);
          ss2 = __builtin_fmaf(q, q, ss2);
        }
      }
      const float tot2 = row_reduce<WGS, NW, NW, false>(ss2, red, parity, 0, tid);
      float inv2;
      int sh2;
      if (rescaled_scale(m, tot2, ex, a.hidden, a.eps, inv2, sh2)) {
        inv = inv2;
        shift = sh2;
      }
    }

    for (int c0 = tid; c0 < C; c0 += WGS * UNR) {
      raw_t rv[UNR];
      typename GV::raw_t rg[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + u * WGS;
        if (c < C) {
          rv[u] = own(c);
          rg[u] = GV::template load<false>(a.gamma, c);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + u * WGS;
        if (c < C) {
          float t[V], g[V], y[V];
          IV::unpack(rv[u], t);
          GV::unpack(rg[u], g);
          if (shift == 0) {
#pragma unroll
            for (int e = 0; e < V; ++e) y[e] = (t[e] * inv) * g[e];
          } else {
#pragma unroll
            for (int e = 0; e < V; ++e) y[e] = (ldexpf(t[e], shift) * inv) * g[e];
          }
          const auto packed = OV::pack(y);
          if constexpr (AG) {
            for (int j = 0; j < a.gather.n; ++j) {
              char* grow = row_ptr(a.gather.p[j], a.out_stride, row);
              if constexpr (BUF)
                OV::template store_buf<kCpolStoreStream>(row_rsrc(grow, C * OV::BYTES), c, packed);
              else
                OV::template store<NT>(grow, c, packed);
            }
          } else {
            if constexpr (BUF)
              OV::template store_buf<kCpolStoreStream>(row_rsrc(orow, C * OV::BYTES), c, packed);
            else
              OV::template store<NT>(orow, c, packed);
          }
        }
      }
    }
  }
}

}  // namespace rmsn
