// gemm_scatter_kernels.hpp -- device-side pieces of the GEMM with a
// reduce-scatter epilogue (csrc/gemm_scatter.hip) that other kernels share:
// tile sizes, element codecs, the tile schedule and the kernel parameters.
// Method: page "LLM System: 通信计算融合算子实现 01 - sm80GEMM +
// ReduceScatter" (epilogue scatter, section "cutlass自定义epilogue–sm80";
// remote-first tile order, section "gemmrs版本的swizzle如何编排").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gemm_scatter.h"

namespace gsc {

constexpr int BM = GEMM_SCATTER_TILE_M;
constexpr int BN = GEMM_SCATTER_TILE_N;            // wide tile
constexpr int BN_NARROW = GEMM_SCATTER_TILE_N_NARROW;
constexpr int BK = 64;                 // k elements per step (128 bytes of a row)
constexpr int kThreads = 256;          // four waves, one per SIMD
constexpr int kChunksPerRow = BK / 8;  // 16-byte chunks per LDS row
constexpr int kXcds = 8;
constexpr int kRoundPerXcd = 32;       // positions each XCD takes per round (one per CU)
constexpr int kGroupM = 8;             // tile-rows per schedule group
// Buffer resource word 3 for gfx9-family raw (untyped) buffer access; the
// offset used for a chunk outside every operand's range.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kOutOfRange = 0x7FFFFFF0;
static_assert(BM == 256 && BN == 256 && BN_NARROW == 128 && kThreads == 256,
              "the thread mapping assumes these");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Elem;

template <>
struct Elem<RMSN_BF16> {
  __device__ static f32x4 mfma(u32x4 x, u32x4 y, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
  }
  __device__ static float decode(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
  __device__ static uint32_t pack2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  __device__ static uint16_t pack1(float v) { return (uint16_t)(pack2(v, 0.0f) & 0xFFFFu); }
};

template <>
struct Elem<RMSN_F16> {
  __device__ static f32x4 mfma(u32x4 x, u32x4 y, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                  __builtin_bit_cast(f16x8, y), acc, 0, 0, 0);
  }
  __device__ static float decode(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
  __device__ static uint32_t pack2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  __device__ static uint16_t pack1(float v) { return (uint16_t)(pack2(v, 0.0f) & 0xFFFFu); }
};

// ---- tile schedule (shared by the kernel and the host's plan query) --------

struct Sched {
  int tiles_m, tiles_n, tiles;
  int tm_start;      // first tile-row of the rotated order
  int remote_rows;   // rotated tile-rows before the local chunk's
  int local_group;   // tile-rows per group among the local chunk's
};

__host__ __device__ inline Sched make_sched(int m, int n, int tm, int tn, int world, int rank) {
  Sched s;
  s.tiles_m = (m + tm - 1) / tm;
  s.tiles_n = (n + tn - 1) / tn;
  s.tiles = s.tiles_m * s.tiles_n;
  // A tile-row belongs to the chunk of its first row.  Rotated order starts
  // at the first tile-row of chunk rank + 1 (ring order), so the tile-rows
  // of the local chunk (rank) come last.
  const int64_t chunk_rows = world > 0 ? (int64_t)m / world : m;
  const int64_t first_local = ((int64_t)rank * chunk_rows + tm - 1) / tm;
  int64_t end_local = ((int64_t)(rank + 1) * chunk_rows + tm - 1) / tm;
  if (end_local > s.tiles_m) end_local = s.tiles_m;
  const int64_t local = end_local > first_local ? end_local - first_local : 0;
  s.tm_start = (int)(end_local >= s.tiles_m ? 0 : end_local);
  s.remote_rows = s.tiles_m - (int)local;
  s.local_group = local < kGroupM ? (local > 0 ? (int)local : 1) : kGroupM;
  return s;
}

// launch order -> schedule position: each round of kXcds * kRoundPerXcd
// positions is dealt out so that XCD x (which receives workgroups x, x + 8,
// ...) takes a contiguous run of kRoundPerXcd positions; a final partial
// round keeps the identity.
__host__ __device__ inline int position_of_wg(int w, int tiles) {
  constexpr int round = kXcds * kRoundPerXcd;
  const int full = tiles / round * round;
  if (w >= full) return w;
  const int base = w / round * round;
  const int within = w - base;
  return base + (within % kXcds) * kRoundPerXcd + within / kXcds;
}

// schedule position -> tile.  The rotated tile-rows of the other ranks'
// chunks come first, in groups of kGroupM tile-rows, then the local chunk's
// tile-rows in groups of local_group; inside a group the tiles go
// column-major (down the group's tile-rows, then to the next tile-column),
// so a run of positions covers a compact block of the output.
__host__ __device__ inline int tile_at(int p, const Sched& s) {
  const int remote_tiles = s.remote_rows * s.tiles_n;
  int first_row, region_rows, gsize;
  if (p < remote_tiles) {
    first_row = 0;
    region_rows = s.remote_rows;
    gsize = kGroupM;
  } else {
    p -= remote_tiles;
    first_row = s.remote_rows;
    region_rows = s.tiles_m - s.remote_rows;
    gsize = s.local_group;
  }
  const int group = gsize * s.tiles_n;
  const int g = p / group;
  const int idx = p - g * group;
  const int gfirst = g * gsize;
  const int rows = region_rows - gfirst < gsize ? region_rows - gfirst : gsize;
  const int ptm = first_row + gfirst + idx % rows;
  const int tn = idx / rows;
  const int tm = (ptm + s.tm_start) % s.tiles_m;
  return tm * s.tiles_n + tn;
}

struct Params {
  const uint16_t* a;
  const uint16_t* b;
  const uint16_t* c;
  int64_t lda, ldb, ldc, ldd;
  uint16_t* dst[GEMM_SCATTER_WORLD_MAX];
  uint32_t* flags;
  uint32_t epoch;
  int m, n, k;
  int chunk_rows;
  float alpha, beta;
  int vec_out;  // 2: dst rows 16-byte aligned (and C rows 8); 1: both 8-byte; 0: neither
  Sched sched;
};

// ---- matrix-core products with the accumulators in AGPRs --------------------

// One 16 x 16 x 32 product, acc (AGPRs) += x . y, through inline assembly so
// that the 256 accumulators of a 128 x 128 wave block stay pinned in the
// AGPRs.  FIRST: the accumulator starts from zero (so nothing else writes
// the AGPRs before a tile's first product).
template <int DT, bool FIRST>
__device__ __forceinline__ void mma_agpr(f32x4& acc, const u32x4& x, const u32x4& y) {
  if constexpr (FIRST) {
    if constexpr (DT == RMSN_BF16)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(x), "v"(y));
    else
      asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(acc) : "v"(x), "v"(y));
  } else {
    if constexpr (DT == RMSN_BF16)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
    else
      asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
  }
}

// The last products' results must be written before the AGPRs are read:
// the hardware leaves those wait states to software, and inline assembly
// hides the products from the compiler's hazard tracking.  24 wait states
// cover the longest (16-pass) product; the empty statements keep every
// accumulator behind the wait.
__device__ __forceinline__ void settle_agprs(f32x4 (&acc)[8][8]) {
#define GSC_PIN(I) "+a"(acc[I / 8][I % 8])
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : GSC_PIN(0), GSC_PIN(1), GSC_PIN(2), GSC_PIN(3), GSC_PIN(4), GSC_PIN(5), GSC_PIN(6),
                 GSC_PIN(7), GSC_PIN(8), GSC_PIN(9), GSC_PIN(10), GSC_PIN(11), GSC_PIN(12), GSC_PIN(13),
                 GSC_PIN(14), GSC_PIN(15));
  asm volatile(""
               : GSC_PIN(16), GSC_PIN(17), GSC_PIN(18), GSC_PIN(19), GSC_PIN(20), GSC_PIN(21), GSC_PIN(22),
                 GSC_PIN(23), GSC_PIN(24), GSC_PIN(25), GSC_PIN(26), GSC_PIN(27), GSC_PIN(28), GSC_PIN(29),
                 GSC_PIN(30), GSC_PIN(31));
  asm volatile(""
               : GSC_PIN(32), GSC_PIN(33), GSC_PIN(34), GSC_PIN(35), GSC_PIN(36), GSC_PIN(37), GSC_PIN(38),
                 GSC_PIN(39), GSC_PIN(40), GSC_PIN(41), GSC_PIN(42), GSC_PIN(43), GSC_PIN(44), GSC_PIN(45),
                 GSC_PIN(46), GSC_PIN(47));
  asm volatile(""
               : GSC_PIN(48), GSC_PIN(49), GSC_PIN(50), GSC_PIN(51), GSC_PIN(52), GSC_PIN(53), GSC_PIN(54),
                 GSC_PIN(55), GSC_PIN(56), GSC_PIN(57), GSC_PIN(58), GSC_PIN(59), GSC_PIN(60), GSC_PIN(61),
                 GSC_PIN(62), GSC_PIN(63));
#undef GSC_PIN
}

// The same for the 8 x NY accumulators of a (16 NY) x 128 wave block, NY =
// 8, 6 or 5 (tiles 256, 192 or 160 rows high).
#define GSC_PIN(I) "+a"(acc[(I) / NY][(I) % NY])
template <int NY>
__device__ __forceinline__ void settle_agprs_rows(f32x4 (&acc)[8][NY]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : GSC_PIN(0), GSC_PIN(1), GSC_PIN(2), GSC_PIN(3), GSC_PIN(4), GSC_PIN(5), GSC_PIN(6),
                 GSC_PIN(7), GSC_PIN(8), GSC_PIN(9), GSC_PIN(10), GSC_PIN(11), GSC_PIN(12), GSC_PIN(13),
                 GSC_PIN(14), GSC_PIN(15));
  asm volatile(""
               : GSC_PIN(16), GSC_PIN(17), GSC_PIN(18), GSC_PIN(19), GSC_PIN(20), GSC_PIN(21), GSC_PIN(22),
                 GSC_PIN(23), GSC_PIN(24), GSC_PIN(25), GSC_PIN(26), GSC_PIN(27), GSC_PIN(28), GSC_PIN(29),
                 GSC_PIN(30), GSC_PIN(31));
  if constexpr (NY == 5) {
    asm volatile("" : GSC_PIN(32), GSC_PIN(33), GSC_PIN(34), GSC_PIN(35), GSC_PIN(36), GSC_PIN(37),
                 GSC_PIN(38), GSC_PIN(39));
  } else {
    asm volatile(""
                 : GSC_PIN(32), GSC_PIN(33), GSC_PIN(34), GSC_PIN(35), GSC_PIN(36), GSC_PIN(37), GSC_PIN(38),
                   GSC_PIN(39), GSC_PIN(40), GSC_PIN(41), GSC_PIN(42), GSC_PIN(43), GSC_PIN(44), GSC_PIN(45),
                   GSC_PIN(46), GSC_PIN(47));
    if constexpr (NY == 8) {
      asm volatile(""
                   : GSC_PIN(48), GSC_PIN(49), GSC_PIN(50), GSC_PIN(51), GSC_PIN(52), GSC_PIN(53), GSC_PIN(54),
                     GSC_PIN(55), GSC_PIN(56), GSC_PIN(57), GSC_PIN(58), GSC_PIN(59), GSC_PIN(60), GSC_PIN(61),
                     GSC_PIN(62), GSC_PIN(63));
    }
  }
}
#undef GSC_PIN

// The same for the 4 x 8 accumulators of a 128 x 64 wave block.
__device__ __forceinline__ void settle_agprs(f32x4 (&acc)[4][8]) {
#define GSC_PIN(I) "+a"(acc[I / 8][I % 8])
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : GSC_PIN(0), GSC_PIN(1), GSC_PIN(2), GSC_PIN(3), GSC_PIN(4), GSC_PIN(5), GSC_PIN(6),
                 GSC_PIN(7), GSC_PIN(8), GSC_PIN(9), GSC_PIN(10), GSC_PIN(11), GSC_PIN(12), GSC_PIN(13),
                 GSC_PIN(14), GSC_PIN(15));
  asm volatile(""
               : GSC_PIN(16), GSC_PIN(17), GSC_PIN(18), GSC_PIN(19), GSC_PIN(20), GSC_PIN(21), GSC_PIN(22),
                 GSC_PIN(23), GSC_PIN(24), GSC_PIN(25), GSC_PIN(26), GSC_PIN(27), GSC_PIN(28), GSC_PIN(29),
                 GSC_PIN(30), GSC_PIN(31));
#undef GSC_PIN
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8), handed to the compiler's own wait tracking
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

}  // namespace gsc
