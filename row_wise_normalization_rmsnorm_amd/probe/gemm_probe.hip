// gemm_probe.hip -- alternative designs of the GEMM with a reduce-scatter
// epilogue (csrc/gemm_scatter.hip), timed beside the library's kernel by
// `bench.py --gemm-design-sweep` (a measurement aid, not part of the
// library).  Every design forms the same 16 x 16 x 32 matrix-core products
// in the same k order as the library's 256 x 256 kernel, so the bench checks
// each one bit for bit against it.  bf16 and f16, alpha = 1, no C term.
//
// All designs: a 256 x 256 output tile per workgroup of four waves, one per
// SIMD, each a 128 x 128 block of 8 x 8 products whose 256 fp32 accumulators
// stay in AGPRs; operand tiles go straight from memory into LDS with gfx950's
// 16-byte buffer-load-to-LDS form (no VGPR round trip, no ds_write); the
// fragments are read with ds_read_b128 into two VGPR sets used in turn.
//   design 0  k stages of 64 (128-byte LDS rows) in two LDS buffers; the
//             16 LDS reads of each 32-wide half stage spread between the 64
//             products before it (one every four), and the next stage's 16
//             loads between the first half's products
//   design 1  as design 0, but the reads (and loads) issued in one block
//             before the products they run beside
//   design 2  k stages of 32 (64-byte LDS rows) in nbuf = 4 or 5 LDS
//             buffers, loads nbuf stages ahead, reads and loads spread
//   design 3  design 2 made persistent: one workgroup per CU takes tiles b,
//             b + G, ...; the stage pipeline runs on across tiles (a tile's
//             last stages overlap the next tile's first loads) and results
//             leave straight from the accumulators
// mode (design 2 only) takes its time apart; modes 1-4 give wrong results:
//   0 the product; 1 every workgroup computes tile 0 (operands always in L2);
//   2 no loads after the first stages; 3 products only (no loads, no LDS
//   reads in the loop); 4 loads but no LDS reads in the loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../csrc/gemm_scatter_kernels.hpp"

namespace {

using namespace gsc;

constexpr int kThreads4 = 256;           // four waves, one per SIMD
constexpr int kWaitVm0 = wait_vmcnt(0);
using Acc = f32x4[8][8];

template <int DT, bool FIRST>
__device__ __forceinline__ void mma(f32x4& acc, const u32x4& x, const u32x4& y) {
  mma_agpr<DT, FIRST>(acc, x, y);
}
__device__ __forceinline__ void settle(Acc& acc) { settle_agprs(acc); }
constexpr int wait_vm(int n) { return wait_vmcnt(n); }

// A buffer resource over a tile's operand rows, ending at the last element
// of its last existing row (loads past it read zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int64_t ld, int rows,
                                                            int k) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                           (int)(((int64_t)(rows - 1) * ld + k) * 2), kRsrcWord3);
}

struct Tile {
  int m0, n0, a_rows, b_rows;
};
__device__ __forceinline__ Tile tile_geom(int tile, const Params& p) {
  Tile t;
  t.m0 = (tile / p.sched.tiles_n) * BM;
  t.n0 = (tile % p.sched.tiles_n) * BN;
  t.a_rows = p.m - t.m0 < BM ? p.m - t.m0 : BM;
  t.b_rows = p.n - t.n0 < BN ? p.n - t.n0 : BN;
  return t;
}

// Results of one tile: acc[s][t][r] is D[row m0 + wm*128 + t*16 + (lane & 15)]
// [col n0 + wn*128 + s*16 + 4*(lane >> 4) + r].  STAGED: interior tiles with
// 16-byte output rows go through LDS (128 KiB, free by then) and leave in
// whole 512-byte row segments with nontemporal stores, as in the library;
// otherwise each lane stores its four consecutive values (8 bytes) itself.
template <int DT, bool STAGED>
__device__ __forceinline__ void epilogue(Acc& acc, const Params& p, const Tile& T, unsigned char* lds,
                                         int tid) {
  using E = Elem<DT>;
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int row0 = T.m0 + wm * 128 + (lane & 15);
  const int col0 = T.n0 + wn * 128 + 4 * (lane >> 4);
  const bool interior = T.m0 + BM <= p.m && T.n0 + BN <= p.n;
  if (STAGED && p.vec_out == 2 && interior) {
    uint32_t* st = reinterpret_cast<uint32_t*>(lds);
    constexpr int pitch = BN / 2;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int r = wm * 128 + t * 16 + (lane & 15);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = wn * 128 + s * 16 + 4 * (lane >> 4);
        const int chunk = (c >> 3) ^ (r & 15);
        *reinterpret_cast<u32x2*>(st + r * pitch + chunk * 4 + ((c >> 2) & 1) * 2) =
            u32x2{E::pack2(acc[s][t][0], acc[s][t][1]), E::pack2(acc[s][t][2], acc[s][t][3])};
      }
    }
    __syncthreads();
    constexpr int CPR = BN / 8, RPP = kThreads4 / CPR;
#pragma unroll 4
    for (int i = 0; i < BM / RPP; ++i) {
      const int r = i * RPP + tid / CPR;
      const int gm = T.m0 + r;
      const int q = gm / p.chunk_rows;
      uint16_t* drow = p.dst[q] + (int64_t)(gm - q * p.chunk_rows) * p.ldd + T.n0;
      const int c = tid % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * pitch + ((c ^ (r & 15)) * 4));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(drow + c * 8));
    }
  } else if (p.vec_out && interior) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int gm = row0 + t * 16;
      const int q = gm / p.chunk_rows;
      uint16_t* drow = p.dst[q] + (int64_t)(gm - q * p.chunk_rows) * p.ldd + col0;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        *reinterpret_cast<u32x2*>(drow + s * 16) =
            u32x2{E::pack2(acc[s][t][0], acc[s][t][1]), E::pack2(acc[s][t][2], acc[s][t][3])};
      __builtin_amdgcn_sched_barrier(0);   // one row block at a time: few registers live
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int gm = row0 + t * 16;
      const bool row_ok = gm < p.m;
      const int gmc = row_ok ? gm : 0;
      const int q = gmc / p.chunk_rows;
      uint16_t* drow = p.dst[q] + (int64_t)(gmc - q * p.chunk_rows) * p.ldd;
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gn = col0 + s * 16 + r;
          if (row_ok && gn < p.n) drow[gn] = E::pack1(acc[s][t][r]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---- designs 0 and 1: k stages of 64, two LDS buffers ----------------------

constexpr int kRow64 = 128;                 // LDS bytes per operand row
constexpr int kPart64 = BM * kRow64;        // one operand's stage: 32 KiB
constexpr int kStage64 = 2 * kPart64;       // 64 KiB

template <int DT, bool SPREAD>
__global__ __launch_bounds__(kThreads4) void k64_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStage64];
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const Tile T = tile_geom(tile_at(position_of_wg((int)blockIdx.x, p.sched.tiles), p.sched), p);
  const int nk = (p.k + 63) / 64;
  const auto rsa = tile_rsrc(p.a + (int64_t)T.m0 * p.lda, p.lda, T.a_rows, p.k);
  const auto rsb = tile_rsrc(p.b + (int64_t)T.n0 * p.ldb, p.ldb, T.b_rows, p.k);
  // load j (0..7) of this wave: tile rows 64 wave + 8 j + lane / 8; LDS chunk
  // position lane % 8 holds global chunk (lane % 8) ^ (row % 8)
  const int lr = lane >> 3, gchunk = (lane & 7) ^ lr;
  int a_off[8], b_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 64 * wave + 8 * j + lr;
    a_off[j] = ((r < T.a_rows ? r : T.a_rows - 1) * (int)p.lda + gchunk * 8) * 2;
    b_off[j] = ((r < T.b_rows ? r : T.b_rows - 1) * (int)p.ldb + gchunk * 8) * 2;
  }
  auto load1 = [&](int st, int j) __attribute__((always_inline)) {  // j: 0..15
    const bool kin = st * 64 + gchunk * 8 < p.k;
    unsigned char* base = lds + (st & 1) * kStage64 + (64 * wave) * kRow64;
    if (j < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(base + j * 1024), 16,
                                               kin ? a_off[j] + st * 128 : kOutOfRange, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(base + kPart64 + (j - 8) * 1024), 16,
                                               kin ? b_off[j - 8] + st * 128 : kOutOfRange, 0, 0, 0);
  };
  // read f (0..15) of half `half` of stage st, in the order the products use
  // them: x 0, y 0..7, x 1..7
  auto read1 = [&](int st, int half, int f, u32x4 (&xf)[8], u32x4 (&yf)[8]) __attribute__((always_inline)) {
    const unsigned char* b = lds + (st & 1) * kStage64;
    const int c = half * 4 + (lane >> 4);
    if (f >= 1 && f <= 8) {
      const int r = wm * 128 + (f - 1) * 16 + (lane & 15);
      yf[f - 1] = *reinterpret_cast<const u32x4*>(b + r * kRow64 + ((c ^ (r & 7)) * 16));
    } else {
      const int s = f == 0 ? 0 : f - 8;
      const int r = wn * 128 + s * 16 + (lane & 15);
      xf[s] = *reinterpret_cast<const u32x4*>(b + kPart64 + r * kRow64 + ((c ^ (r & 7)) * 16));
    }
  };
  Acc acc;
  // one half stage: the 64 products of (xc, yc), the 16 reads of half `half`
  // of stage rst into (xn, yn) and, with LOAD, the 16 loads of stage lst.
  // SPREAD: one read every four products, loads in between; otherwise the
  // loads, then the reads, then the products.
  auto half_stage = [&](auto first, auto load, const u32x4 (&xc)[8], const u32x4 (&yc)[8],
                        u32x4 (&xn)[8], u32x4 (&yn)[8], int rst, int half, int lst)
                        __attribute__((always_inline)) {
    constexpr bool F = decltype(first)::value, L = decltype(load)::value;
    if constexpr (SPREAD) {
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        mma<DT, F>(acc[i / 8][i % 8], xc[i / 8], yc[i % 8]);
        if (i % 4 == 0) read1(rst, half, i / 4, xn, yn);
        if (L && i % 4 == 2) load1(lst, i / 4);
      }
    } else {
      if constexpr (L)
#pragma unroll
        for (int j = 0; j < 16; ++j) load1(lst, j);
#pragma unroll
      for (int f = 0; f < 16; ++f) read1(rst, half, f, xn, yn);
#pragma unroll
      for (int i = 0; i < 64; ++i) mma<DT, F>(acc[i / 8][i % 8], xc[i / 8], yc[i % 8]);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  u32x4 xa[8], ya[8], xb[8], yb[8];
  if (nk > 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) load1(0, j);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int f = 0; f < 16; ++f) read1(0, 0, f, xa, ya);
    // stage 0's first half multiplies while its second half is read and
    // stage 1 loads
    half_stage(T_{}, std::true_type{}, xa, ya, xb, yb, 0, 1, 1);
    for (int st = 1; st < nk; ++st) {
      // stage st landed for every wave; every wave is done reading stage
      // st - 1, whose buffer stage st + 1 loads into
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
      half_stage(F_{}, std::true_type{}, xb, yb, xa, ya, st, 0, st + 1);   // stage st - 1, 2nd half
      half_stage(F_{}, std::false_type{}, xa, ya, xb, yb, st, 1, 0);      // stage st, 1st half
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) mma<DT, false>(acc[i / 8][i % 8], xb[i / 8], yb[i % 8]);
    settle(acc);
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[s2][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // loads past k (zeros) may still be landing in LDS, which the epilogue reuses
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __builtin_amdgcn_s_barrier();
  epilogue<DT, true>(acc, p, T, lds, tid);
}

// ---- designs 2 and 3: k stages of 32 in NBUF LDS buffers -------------------

constexpr int kRow32 = 64;                  // LDS bytes per operand row
constexpr int kPart32 = BM * kRow32;        // 16 KiB
constexpr int kStage32 = 2 * kPart32;       // 32 KiB

// Operand addressing of one tile for 32-wide stages.  Load j (0..7) of a
// wave: j < 4 A, else B; tile rows 16 (4 wave + j % 4) + lane / 4; LDS chunk
// position lane % 4 holds global chunk (lane % 4) ^ ((row / 2) % 4).
struct Ops32 {
  __amdgpu_buffer_rsrc_t rsa, rsb;
  int a_off[4], b_off[4];
};
__device__ __forceinline__ void ops32(Ops32& o, const Params& p, const Tile& T, int wave, int lane) {
  const int lr = lane >> 2, gchunk = (lane & 3) ^ ((lr >> 1) & 3);
  o.rsa = tile_rsrc(p.a + (int64_t)T.m0 * p.lda, p.lda, T.a_rows, p.k);
  o.rsb = tile_rsrc(p.b + (int64_t)T.n0 * p.ldb, p.ldb, T.b_rows, p.k);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * (4 * wave + j) + lr;
    o.a_off[j] = ((r < T.a_rows ? r : T.a_rows - 1) * (int)p.lda + gchunk * 8) * 2;
    o.b_off[j] = ((r < T.b_rows ? r : T.b_rows - 1) * (int)p.ldb + gchunk * 8) * 2;
  }
}
__device__ __forceinline__ int gchunk32(int lane) { return (lane & 3) ^ (((lane >> 2) >> 1) & 3); }

// load j of stage st (k from 32 st) of the tile whose operands are o, into LDS
// buffer `buf`; valid = false or k past the end: zeros
__device__ __forceinline__ void load32(const Ops32& o, bool valid, const Params& p, unsigned char* lds,
                                       int buf, int st, int j, int wave, int lane) {
  const bool kin = valid && st * 32 + gchunk32(lane) * 8 < p.k;
  unsigned char* base = lds + buf * kStage32 + (4 * wave) * 1024;
  if (j < 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.rsa, (lds_ptr_t)(base + j * 1024), 16,
                                             kin ? o.a_off[j] + st * 64 : kOutOfRange, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.rsb, (lds_ptr_t)(base + kPart32 + (j - 4) * 1024), 16,
                                             kin ? o.b_off[j - 4] + st * 64 : kOutOfRange, 0, 0, 0);
}
// read f (0..15) of the stage in LDS buffer buf: x 0, y 0..7, x 1..7
__device__ __forceinline__ void read32(const unsigned char* lds, int buf, int f, u32x4 (&xf)[8],
                                       u32x4 (&yf)[8], int wm, int wn, int lane) {
  const unsigned char* b = lds + buf * kStage32;
  const int c = lane >> 4;
  if (f >= 1 && f <= 8) {
    const int r = wm * 128 + (f - 1) * 16 + (lane & 15);
    yf[f - 1] = *reinterpret_cast<const u32x4*>(b + r * kRow32 + ((c ^ ((r >> 1) & 3)) * 16));
  } else {
    const int s = f == 0 ? 0 : f - 8;
    const int r = wn * 128 + s * 16 + (lane & 15);
    xf[s] = *reinterpret_cast<const u32x4*>(b + kPart32 + r * kRow32 + ((c ^ ((r >> 1) & 3)) * 16));
  }
}

// One stage: the 64 products of (xc, yc) with, spread between them, the 16
// reads of buffer rbuf into (xn, yn) (one every three products from the
// first) and the 8 loads of stage lst (products 2, 10, ...).
template <int DT, bool FIRST, bool READS, bool LOADS, typename LoadFn>
__device__ __forceinline__ void stage32(Acc& acc, const u32x4 (&xc)[8], const u32x4 (&yc)[8],
                                        u32x4 (&xn)[8], u32x4 (&yn)[8], const unsigned char* lds,
                                        int rbuf, LoadFn&& load, int wm, int wn, int lane) {
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    mma<DT, FIRST>(acc[i / 8][i % 8], xc[i / 8], yc[i % 8]);
    if (READS && i % 3 == 0 && i / 3 < 16) read32(lds, rbuf, i / 3, xn, yn, wm, wn, lane);
    if (LOADS && i % 8 == 2) load(i / 8);
  }
}

template <int DT, int MODE, int NBUF>
__global__ __launch_bounds__(kThreads4) void k32_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NBUF * kStage32];
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const Tile T = tile_geom(MODE == 1 ? 0 : tile_at(position_of_wg((int)blockIdx.x, p.sched.tiles), p.sched), p);
  const int nk = (p.k + 31) / 32;
  Ops32 o;
  ops32(o, p, T, wave, lane);
  // before the stage-st products, stages up to st - 1 + NBUF have gone out;
  // stage st + 1 has landed once at most NBUF - 2 later stages are in flight
  constexpr int kWaitKeep = wait_vm((NBUF - 2) * 8), kWaitFirst = wait_vm((NBUF - 1) * 8);
  constexpr bool READS = MODE != 3 && MODE != 4, LOADS = MODE != 2 && MODE != 3;
  Acc acc;
  u32x4 xa[8], ya[8], xb[8], yb[8];
  if (nk > 0) {
#pragma unroll
    for (int st = 0; st < NBUF; ++st)
#pragma unroll
      for (int j = 0; j < 8; ++j) load32(o, true, p, lds, st, st, j, wave, lane);
    __builtin_amdgcn_s_waitcnt(kWaitFirst);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int f = 0; f < 16; ++f) read32(lds, 0, f, xa, ya, wm, wn, lane);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_waitcnt(kWaitKeep);
    __builtin_amdgcn_s_barrier();
    auto loader = [&](int st) {
      return [&, st](int j) __attribute__((always_inline)) {
        load32(o, true, p, lds, st % NBUF, st, j, wave, lane);
      };
    };
    stage32<DT, true, READS, LOADS>(acc, xa, ya, xb, yb, lds, 1 % NBUF, loader(NBUF), wm, wn, lane);
    for (int st = 1; st < nk; st += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_waitcnt(kWaitKeep);
      __builtin_amdgcn_s_barrier();
      stage32<DT, false, READS, LOADS>(acc, xb, yb, xa, ya, lds, (st + 1) % NBUF, loader(st + NBUF), wm,
                                       wn, lane);
      if (st + 1 >= nk) break;
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_waitcnt(kWaitKeep);
      __builtin_amdgcn_s_barrier();
      stage32<DT, false, READS, LOADS>(acc, xa, ya, xb, yb, lds, (st + 2) % NBUF, loader(st + 1 + NBUF),
                                       wm, wn, lane);
    }
    settle(acc);
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[s2][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __builtin_amdgcn_s_barrier();
  epilogue<DT, true>(acc, p, T, lds, tid);
}

// Design 3.  Stages per tile are padded to an even count: a k whose last
// 64-wide step is half empty still takes the all-zero half, as the library's
// 64-wide steps do, so results stay bit for bit equal.  A tile needs at least
// NBUF stages (the loads run at most one tile ahead).
template <int DT, int NBUF>
__global__ __launch_bounds__(kThreads4) void persistent_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NBUF * kStage32];
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int G = (int)gridDim.x;
  const int ntiles = (p.sched.tiles - (int)blockIdx.x + G - 1) / G;
  const int nk = 2 * ((p.k + 63) / 64);
  auto tile_of = [&](int j) __attribute__((always_inline)) {
    return tile_at(position_of_wg((int)blockIdx.x + (j < ntiles ? j : 0) * G, p.sched.tiles), p.sched);
  };
  constexpr int kWaitKeep = wait_vm((NBUF - 2) * 8), kWaitFirst = wait_vm((NBUF - 1) * 8);
  Acc acc;
  if (ntiles <= 0) return;
  if (nk == 0) {
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[s2][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < ntiles; ++j) epilogue<DT, false>(acc, p, tile_geom(tile_of(j), p), lds, tid);
    return;
  }
  // operands of the tile being multiplied (0) and of the next one (1)
  Ops32 o0, o1;
  bool v0 = true, v1 = ntiles > 1;
  ops32(o0, p, tile_geom(tile_of(0), p), wave, lane);
  ops32(o1, p, tile_geom(tile_of(1), p), wave, lane);
  // load j of tile-relative stage ls (ls >= nk: stage ls - nk of the next tile)
  auto load = [&](int ls, int buf, int j) __attribute__((always_inline)) {
    const bool next = ls >= nk;
    const int st = next ? ls - nk : ls;
    const bool kin = (next ? v1 : v0) && st * 32 + gchunk32(lane) * 8 < p.k;
    unsigned char* base = lds + buf * kStage32 + (4 * wave) * 1024;
    if (j < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(next ? o1.rsa : o0.rsa, (lds_ptr_t)(base + j * 1024), 16,
                                               kin ? (next ? o1.a_off[j] : o0.a_off[j]) + st * 64 : kOutOfRange,
                                               0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          next ? o1.rsb : o0.rsb, (lds_ptr_t)(base + kPart32 + (j - 4) * 1024), 16,
          kin ? (next ? o1.b_off[j - 4] : o0.b_off[j - 4]) + st * 64 : kOutOfRange, 0, 0, 0);
  };
  auto loader = [&](int ls, int buf) {
    return [&, ls, buf](int j) __attribute__((always_inline)) { load(ls, buf, j); };
  };
  auto sync = [&](bool stores) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (stores)   // stores may complete out of order with the loads in flight
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    else
      __builtin_amdgcn_s_waitcnt(kWaitKeep);
    __builtin_amdgcn_s_barrier();
  };
  u32x4 xa[8], ya[8], xb[8], yb[8];
#pragma unroll
  for (int st = 0; st < NBUF; ++st)
#pragma unroll
    for (int j = 0; j < 8; ++j) load(st, st, j);
  __builtin_amdgcn_s_waitcnt(kWaitFirst);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int f = 0; f < 16; ++f) read32(lds, 0, f, xa, ya, wm, wn, lane);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_waitcnt(kWaitKeep);
  __builtin_amdgcn_s_barrier();
  // tile j: stages g0 .. g0 + nk - 1 in buffers g % NBUF; even stages multiply
  // (xa, ya), odd ones (xb, yb); the last reads the next tile's first
  // fragments into (xa, ya).  Stage st's products carry the loads of stage
  // st + NBUF into the buffer stage st leaves.
  int g0 = 0;
#pragma unroll 1
  for (int j = 0; j < ntiles; ++j, g0 += nk) {
    if (j > 0) sync(true);
    stage32<DT, true, true, true>(acc, xa, ya, xb, yb, lds, (g0 + 1) % NBUF, loader(NBUF, g0 % NBUF), wm, wn,
                                  lane);
#pragma unroll 1
    for (int st = 1; st < nk - 1; st += 2) {
      sync(false);
      stage32<DT, false, true, true>(acc, xb, yb, xa, ya, lds, (g0 + st + 1) % NBUF,
                                     loader(st + NBUF, (g0 + st) % NBUF), wm, wn, lane);
      sync(false);
      stage32<DT, false, true, true>(acc, xa, ya, xb, yb, lds, (g0 + st + 2) % NBUF,
                                     loader(st + 1 + NBUF, (g0 + st + 1) % NBUF), wm, wn, lane);
    }
    sync(false);
    stage32<DT, false, true, true>(acc, xb, yb, xa, ya, lds, (g0 + nk) % NBUF,
                                   loader(nk - 1 + NBUF, (g0 + nk - 1) % NBUF), wm, wn, lane);
    settle(acc);
    epilogue<DT, false>(acc, p, tile_geom(tile_of(j), p), lds, tid);
    o0 = o1;
    v0 = v1;
    v1 = j + 2 < ntiles;
    ops32(o1, p, tile_geom(tile_of(j + 2), p), wave, lane);
  }
  // loads past the last tile (zeros) may still be landing in LDS
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

template <int DT>
int launch(int design, int mode, int nbuf, const Params& p, int cus, hipStream_t s) {
  const dim3 block(kThreads4), grid((unsigned)p.sched.tiles);
  if (design == 0) {
    hipLaunchKernelGGL((k64_kernel<DT, true>), grid, block, 0, s, p);
  } else if (design == 1) {
    hipLaunchKernelGGL((k64_kernel<DT, false>), grid, block, 0, s, p);
  } else if (design == 2) {
#define GP_K32(M)                                                                        \
  if (mode == M) {                                                                      \
    if (nbuf == 4) hipLaunchKernelGGL((k32_kernel<DT, M, 4>), grid, block, 0, s, p);    \
    else hipLaunchKernelGGL((k32_kernel<DT, M, 5>), grid, block, 0, s, p);              \
  }
    GP_K32(0) GP_K32(1) GP_K32(2) GP_K32(3) GP_K32(4)
#undef GP_K32
  } else {
    const dim3 pgrid((unsigned)(p.sched.tiles < cus ? p.sched.tiles : cus));
    if (nbuf == 4) hipLaunchKernelGGL((persistent_kernel<DT, 4>), pgrid, block, 0, s, p);
    else hipLaunchKernelGGL((persistent_kernel<DT, 5>), pgrid, block, 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // namespace

// gemm_probe: dst[q] = rows [q m/world, (q+1) m/world) of a @ b^T for design
// 0-3 (mode 0-4 with design 2, else 0; nbuf 4 or 5 with designs 2 and 3).
// a [m, k] and b [n, k] with row strides lda, ldb (elements, multiples of 8,
// 16-byte aligned bases), dst chunks with row stride ldd; dtype RMSN_BF16 or
// RMSN_F16.  Returns 0, -1 for arguments the probe does not take (nothing is
// launched), -7 for a launch error.
extern "C" int gemm_probe(int design, int mode, int nbuf, void* const* dst, int64_t ldd, int world,
                          const void* a, int64_t lda, const void* b, int64_t ldb, int64_t m, int64_t n,
                          int64_t k, int dtype, void* stream) {
  if (design < 0 || design > 3 || mode < 0 || mode > 4 || (mode != 0 && design != 2)) return -1;
  if ((design >= 2) && nbuf != 4 && nbuf != 5) return -1;
  if (dtype != RMSN_BF16 && dtype != RMSN_F16) return -1;
  if (!dst || !a || !b || world < 1 || world > GEMM_SCATTER_WORLD_MAX) return -1;
  if (m <= 0 || n <= 0 || k < 0 || m > 0x7FFFFFFF || n > 0x7FFFFFFF || k > 0x7FFFFFFF || m % world) return -1;
  if (k % 8 || lda % 8 || ldb % 8 || lda < k || ldb < k || ldd < n) return -1;
  if (((uintptr_t)a & 15u) || ((uintptr_t)b & 15u)) return -1;
  if ((int64_t)(gsc::BM - 1) * lda + k >= ((int64_t)1 << 29) ||
      (int64_t)(gsc::BN - 1) * ldb + k >= ((int64_t)1 << 29))
    return -1;
  if (mode == 1 && (m < gsc::BM || n < gsc::BN)) return -1;
  const int64_t nk_even = 2 * ((k + 63) / 64);
  if (design == 3 && nk_even != 0 && nk_even < nbuf) return -1;
  gsc::Params p{};
  p.a = static_cast<const uint16_t*>(a);
  p.b = static_cast<const uint16_t*>(b);
  p.c = nullptr;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = 0;
  p.ldd = ldd;
  bool vec16 = ldd % 8 == 0, vec8 = ldd % 4 == 0;
  for (int q = 0; q < world; ++q) {
    if (!dst[q]) return -1;
    p.dst[q] = static_cast<uint16_t*>(dst[q]);
    if ((uintptr_t)dst[q] & 15u) vec16 = false;
    if ((uintptr_t)dst[q] & 7u) vec8 = false;
  }
  p.flags = nullptr;
  p.epoch = 0;
  p.m = (int)m;
  p.n = (int)n;
  p.k = (int)k;
  p.chunk_rows = (int)(m / world);
  p.alpha = 1.0f;
  p.beta = 0.0f;
  p.vec_out = vec16 ? 2 : vec8 ? 1 : 0;
  p.sched = gsc::make_sched((int)m, (int)n, gsc::BM, gsc::BN, world, 0);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return -7;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == RMSN_BF16 ? launch<RMSN_BF16>(design, mode, nbuf, p, cus, s)
                            : launch<RMSN_F16>(design, mode, nbuf, p, cus, s);
}
