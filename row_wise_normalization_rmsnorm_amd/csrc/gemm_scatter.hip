// gemm_scatter.hip -- GEMM with a reduce-scatter epilogue on gfx950, and its
// C ABI (include/gemm_scatter.h).
//
// Method: page "LLM System: 通信计算融合算子实现 01 - sm80GEMM +
// ReduceScatter".  The epilogue of the FFN's second GEMM computes
// alpha * acc + beta * C and writes each output tile straight into the
// buffer of the rank whose chunk it belongs to (section
// "cutlass自定义epilogue–sm80"), raising a per-tile flag after the tile is
// visible; tiles of the other ranks' chunks are scheduled before the local
// chunk (section "gemmrs版本的swizzle如何编排").
//
// MI355X design:
//   - 256 x 256 output tiles (gemm_wide_kernel): four waves, one per SIMD,
//     each a 128 x 128 block of 8 x 8 v_mfma_f32_16x16x32 products whose 256
//     fp32 accumulators stay in AGPRs (inline-assembly products tied to
//     them).  Operand tiles go straight from memory into LDS with gfx950's
//     16-byte load-to-LDS forms, k steps of 64 in a ring of five 32 KiB
//     operand slots, so every load has one and a half steps to land; each
//     32-wide half step's products carry, one every four, the LDS reads of
//     the next half's fragments and, one every eight, a load, with almost
//     no address arithmetic in the loop.  Measured on the 4096 x 8192 x 3584
//     bf16 product in one process with its predecessors: 168.0 us, against
//     179.0 for the first ring (64-bit load addresses, per-read slot
//     arithmetic), 190.8 with two 64 KiB step buffers (loads one step
//     ahead) and 209.1 for the earlier eight-wave kernel (two waves per
//     SIMD, 128 x 64 blocks, loads staged through registers); the
//     alternatives are in probe/gemm_probe.hip (bench.py
//     --gemm-design-sweep).
//   - 256 x 128 tiles (gemm_narrow_kernel) for products whose 256 x 256
//     tiles would leave much of the last round of workgroups idle (1024
//     tokens: 128 tiles on 256 CUs): four waves too, each a 128 x 64 block
//     of 4 x 8 products, the same operand path with a ring of three 48 KiB
//     step slots.  Both widths accumulate every output in the same k order,
//     so they give bitwise equal results.
//   - The matrix-core operands are swapped (the weight rows feed the first
//     operand, the activation rows the second), so each lane's four
//     accumulator values are four consecutive output columns of one row.
//   - LDS rows are 128 bytes (64 elements); the 16-byte chunk c of row r is
//     stored at chunk position c ^ (r & 7), so the eight lanes of each LDS
//     access phase, which read the same chunk of eight consecutive rows, hit
//     eight different bank groups.
//   - Tile order: tile-rows rotated so that the chunks after the local
//     rank's come first, in ring order, and the local chunk's last; each
//     part in groups of up to eight tile-rows, column-major within a group,
//     for cache reuse.  Consecutive workgroups land on different XCDs
//     (round-robin dispatch), so each round of 256 positions is dealt out in
//     runs of 32 per XCD: an 8 x 4 block of tiles shares its operand rows in
//     the XCD's L2 (measured 1214 -> 1241 TFLOP/s against groups of two
//     tile-rows on the 4096 x 8192 x 3584 bf16 product).
//   - Interior tiles with 16-byte aligned output rows stage the rounded tile
//     in LDS and write whole 512-byte row segments, with nontemporal stores:
//     the output (64 MiB for the 4096 x 8192 product) then does not push the
//     operand rows out of the XCDs' L2 (measured 2-4% faster at 1024, 4096
//     and 8192 tokens, 8192 x 3584 weights).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "../../include/gemm_scatter.h"
#include "gemm_scatter_kernels.hpp"

int rmsn_set_error(int code, const char* msg);


namespace gsc {

// The results of one tile, alpha * D + beta * C, into the destination
// chunks, then the tile's flag.  acc[s][t][r] is D[row m0 + wm*WR + t*16 +
// (lane & 15)][col n0 + wn*WC + s*16 + 4*(lane >> 4) + r] for the THREADS / 64
// waves' WR x WC blocks of a TM x TN tile; staging: TM * TN * 2 bytes of LDS
// that no wave reads any more.
template <int DT, int TM, int TN, int WR, int WC, int THREADS, typename AccT>
__device__ __forceinline__ void store_tile(const AccT& acc, const Params& p, int tile, int m0, int n0,
                                           int wm, int wn, int tid, uint32_t* staging) {
  using E = Elem<DT>;
  constexpr int NX = WC / 16, NY = WR / 16;
  constexpr int CPR = TN / 8;          // 16-byte chunks per staged output row
  constexpr int RPP = THREADS / CPR;   // staged rows stored per pass
  static_assert(CPR >= 16 && TM % RPP == 0, "staging layout");
  const int lane = tid & 63;
  const int row0 = m0 + wm * WR + (lane & 15);
  const int col0 = n0 + wn * WC + 4 * (lane >> 4);
  // interior tiles whose TM rows all belong to chunk q0 address every row
  // from that chunk's row m0
  const int q0 = m0 / p.chunk_rows;
  const bool one_chunk = (m0 + TM - 1) / p.chunk_rows == q0;
  uint16_t* const chunk_base = p.dst[q0] + (int64_t)(m0 - q0 * p.chunk_rows) * p.ldd;
  if (p.vec_out == 2 && m0 + TM <= p.m && n0 + TN <= p.n) {
    // interior tile, 16-byte aligned output rows: the rounded tile is staged
    // in LDS, then leaves in 16-byte stores that cover whole row segments of
    // TN * 2 bytes (nontemporal: the output is not read back here).  The
    // 16-byte chunk c of staged row r sits at chunk position c ^ (r & 15), so
    // the 16 rows one staging write touches land in 16 different bank groups.
    uint32_t* st = staging;
    constexpr int pitch = TN / 2;  // staged row pitch in 32-bit words
#pragma unroll
    for (int t = 0; t < NY; ++t) {
      const int r = wm * WR + t * 16 + (lane & 15);
      const uint16_t* crow = p.c ? p.c + (int64_t)(m0 + r) * p.ldc + col0 : nullptr;
#pragma unroll
      for (int s = 0; s < NX; ++s) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = p.alpha * acc[s][t][q];
        if (crow) {
          const u32x2 cv = *reinterpret_cast<const u32x2*>(crow + s * 16);
          v[0] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.x & 0xFFFFu)), v[0]);
          v[1] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.x >> 16)), v[1]);
          v[2] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.y & 0xFFFFu)), v[2]);
          v[3] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.y >> 16)), v[3]);
        }
        const int c = wn * WC + s * 16 + 4 * (lane >> 4);  // column in the tile
        const int chunk = (c >> 3) ^ (r & 15);
        *reinterpret_cast<u32x2*>(st + r * pitch + chunk * 4 + ((c >> 2) & 1) * 2) =
            u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
      }
    }
    __syncthreads();
    // thread t stores chunk (t % CPR) of rows t / CPR + RPP i.  When the
    // tile's rows lie in one chunk (always, if the chunk height is a
    // multiple of the tile's), one base pointer serves every row: no
    // division and no per-lane fetch of a chunk pointer before each store
    const int c = (int)((unsigned)tid % CPR);
    if (one_chunk) {
      uint16_t* base = chunk_base + n0 + c * 8;
#pragma unroll 8
      for (int i = 0; i < TM / RPP; ++i) {
        const int r = i * RPP + (int)((unsigned)tid / CPR);
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * pitch + ((c ^ (r & 15)) * 4));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base + (int64_t)r * p.ldd));
      }
    } else {
#pragma unroll 4
      for (int i = 0; i < TM / RPP; ++i) {
        const int r = i * RPP + (int)((unsigned)tid / CPR);
        const int gm = m0 + r;
        const int q = gm / p.chunk_rows;
        uint16_t* drow = p.dst[q] + (int64_t)(gm - q * p.chunk_rows) * p.ldd + n0;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * pitch + ((c ^ (r & 15)) * 4));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(drow + c * 8));
      }
    }
  } else if (p.vec_out && m0 + TM <= p.m && n0 + TN <= p.n) {
    // interior tile: every element exists and every access is 8-byte aligned
#pragma unroll
    for (int t = 0; t < NY; ++t) {
      const int gm = row0 + t * 16;
      const int q = one_chunk ? 0 : gm / p.chunk_rows;
      uint16_t* drow = (one_chunk ? chunk_base + (int64_t)(gm - m0) * p.ldd
                                  : p.dst[q] + (int64_t)(gm - q * p.chunk_rows) * p.ldd) + col0;
      const uint16_t* crow = p.c ? p.c + (int64_t)gm * p.ldc + col0 : nullptr;
#pragma unroll
      for (int s = 0; s < NX; ++s) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = p.alpha * acc[s][t][r];
        if (crow) {
          const u32x2 cv = *reinterpret_cast<const u32x2*>(crow + s * 16);
          v[0] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.x & 0xFFFFu)), v[0]);
          v[1] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.x >> 16)), v[1]);
          v[2] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.y & 0xFFFFu)), v[2]);
          v[3] = __builtin_fmaf(p.beta, E::decode((uint16_t)(cv.y >> 16)), v[3]);
        }
        *reinterpret_cast<u32x2*>(drow + s * 16) = u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
      }
    }
  } else {
    // edge tile (or unaligned rows): element by element, inside m x n only
#pragma unroll
    for (int t = 0; t < NY; ++t) {
      const int gm = row0 + t * 16;
      const bool row_ok = gm < p.m;
      const int gmc = row_ok ? gm : 0;
      const int q = gmc / p.chunk_rows;
      uint16_t* drow = p.dst[q] + (int64_t)(gmc - q * p.chunk_rows) * p.ldd;
      const uint16_t* crow = p.c ? p.c + (int64_t)gmc * p.ldc : nullptr;
#pragma unroll
      for (int s = 0; s < NX; ++s) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gn = col0 + s * 16 + r;
          if (row_ok && gn < p.n) {
            float v = p.alpha * acc[s][t][r];
            if (crow) v = __builtin_fmaf(p.beta, E::decode(crow[gn]), v);
            drow[gn] = E::pack1(v);
          }
        }
      }
    }
  }

  if (p.flags) {
    __threadfence_system();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(p.flags + tile, p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// The TM x 256 tile (TM = 256, 192 or 160 rows): four waves, one per SIMD,
// each a (TM / 2) x 128 block of 8 x NY products (NY = TM / 32) whose fp32
// accumulators stay in AGPRs.  Operand tiles go straight from memory into
// LDS (gfx950's 16-byte load-to-LDS buffer form: no VGPR round trip, no LDS
// write instructions), k steps of 64.  The LDS is a ring of five 32 KiB
// slots, one operand of one step each: A of step t is part 2t and B part
// 2t + 1, in slot part % 5.  While step kt is read, A of step kt + 1 has
// landed or is landing, and step kt issues B of step kt + 1 and A of step
// kt + 2 into the two slots step kt - 1 freed: every load has at least one
// and a half steps to land, against one with two 64 KiB step buffers.  With
// one wave per SIMD nothing hides a stall, so each 32-wide half step's
// products carry, evenly spaced, the LDS reads of the fragments the next
// half step multiplies and the loads of one part (B of the next step in the
// first half, A of the step after in the second), in that order (a
// scheduling barrier after each product keeps the compiler from bunching
// them): no wave holds the LDS queue or the memory pipe for long, and the
// products keep issuing.  The loop carries almost no address arithmetic:
// the slot is a scalar, each lane's four LDS read bases are fixed for the
// kernel (fragments sit at immediate offsets), and a load of a whole step
// takes its lane's row offset, fixed too, plus the step's byte offset in a
// scalar register.  Tiles of 192 or 160 rows exist for products whose
// 256-row tiles would leave much of a round of workgroups idle (1536 tokens:
// one round of 192-row tiles; 2560: two of 160-row tiles).
constexpr int kRowBytes = BK * 2;                 // LDS bytes per operand row (128)
constexpr int kPartBytes = BM * kRowBytes;        // one operand of one k step: 32 KiB
constexpr int kSlots = 5;                         // 160 KiB, the whole LDS
static_assert(BN == BM, "the widest tile is square");
static_assert(kSlots * kPartBytes <= 160 * 1024, "gfx950 LDS per workgroup");

template <int DT, int TM>
__device__ __forceinline__ void wide_tile(const Params& p) {
  constexpr int WR = TM / 2;    // rows of a wave block
  constexpr int NY = WR / 16;   // its row fragments
  constexpr int NA = TM / 32;   // A loads per wave and step
  constexpr int NP = 8 * NY;    // products per half step
  constexpr int NR = 8 + NY;    // fragment reads per half step
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kSlots * kPartBytes];
  const int tile = tile_at(position_of_wg((int)blockIdx.x, p.sched.tiles), p.sched);
  const int m0 = (tile / p.sched.tiles_n) * TM;
  const int n0 = (tile % p.sched.tiles_n) * BN;
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // wave block: rows wm * WR, columns wn * 128
  const int nk = (p.k + BK - 1) / BK;
  const int a_tile_rows = p.m - m0 < TM ? p.m - m0 : TM;
  const int b_tile_rows = p.n - n0 < BN ? p.n - n0 : BN;
  // buffer resources end at the last element of the tile's last existing
  // row; rows past m (n) re-read the last existing row (their outputs are
  // never stored) and chunks past k take an offset outside every resource,
  // which reads as zeros
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + (int64_t)m0 * p.lda), (short)0,
      (int)(((int64_t)(a_tile_rows - 1) * p.lda + p.k) * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b + (int64_t)n0 * p.ldb), (short)0,
      (int)(((int64_t)(b_tile_rows - 1) * p.ldb + p.k) * 2), kRsrcWord3);
  // A load j (0 .. NA - 1) moves this wave's tile rows (TM / 4) wave + 8 j +
  // lane / 8, B load j (0..7) rows 64 wave + 8 j + lane / 8; the 64 lanes
  // fill 1 KiB of LDS in order, so LDS chunk position lane % 8 of a row
  // holds global chunk (lane % 8) ^ (row % 8)
  const int lr = lane >> 3, gchunk = (lane & 7) ^ lr;
  int a_off[NA], b_off[8];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = (TM / 4) * wave + 8 * j + lr;
    a_off[j] = ((r < a_tile_rows ? r : a_tile_rows - 1) * (int)p.lda + gchunk * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 64 * wave + 8 * j + lr;
    b_off[j] = ((r < b_tile_rows ? r : b_tile_rows - 1) * (int)p.ldb + gchunk * 8) * 2;
  }
  // Steps whose every chunk lies inside k pass the step's byte offset as
  // the scalar offset, so the loop adds nothing per lane (measured 170.2
  // against 173.2 us for 64-bit global addresses, bf16 4096 x 8192 x 3584).
  // The last, partial step and the steps past it put each chunk past k at
  // an offset outside the resource, which reads as zeros.
  const int nk_full = p.k / BK;
  // load j of part q (A of step q / 2 for even q, B for odd q)
  auto load1 = [&](auto whole, int q, int slot, int j) __attribute__((always_inline)) {
    const int kt = q >> 1;
    const bool is_a = (q & 1) == 0;
    unsigned char* dst = lds + slot * kPartBytes + (is_a ? (TM / 4) * wave : 64 * wave) * kRowBytes + j * 1024;
    if constexpr (decltype(whole)::value) {
      if (is_a)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)dst, 16, a_off[j], kt * BK * 2, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)dst, 16, b_off[j], kt * BK * 2, 0, 0);
    } else {
      const bool kin = kt * BK + gchunk * 8 < p.k;
      if (is_a)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)dst, 16,
                                                 kin ? a_off[j] + kt * BK * 2 : kOutOfRange, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)dst, 16,
                                                 kin ? b_off[j] + kt * BK * 2 : kOutOfRange, 0, 0, 0);
    }
  };
  // Fragment reads: lane l supplies row (l & 15) of a 16-row block and
  // 16-byte chunk half * 4 + l / 16 of the step.  rd_a[h] and rd_b[h] are
  // the lane's byte offsets, inside a slot, of the first fragment of half h;
  // fragment s lies 16 rows (2 KiB) further.
  uint32_t rd_a[2], rd_b[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = h * 4 + (lane >> 4);
    const int ra = wm * WR + (lane & 15), rb = wn * 128 + (lane & 15);
    rd_a[h] = (uint32_t)(ra * kRowBytes + ((c ^ (ra & 7)) * 16));
    rd_b[h] = (uint32_t)(rb * kRowBytes + ((c ^ (rb & 7)) * 16));
  }
  // fragment f (0 .. NR - 1) of half `half` of the step whose A is in slot
  // sa and B in slot sb, in the order the products use them (x 0, y 0 ..
  // NY - 1, x 1..7)
  auto read1 = [&](int sa, int sb, int half, int f, u32x4 (&xf)[8], u32x4 (&yf)[NY])
                   __attribute__((always_inline)) {
    if (f >= 1 && f <= NY) {
      const unsigned char* a = lds + sa * kPartBytes + rd_a[half];
      yf[f - 1] = *reinterpret_cast<const u32x4*>(a + (f - 1) * 16 * kRowBytes);
    } else {
      const int s = f == 0 ? 0 : f - NY;
      const unsigned char* b = lds + sb * kPartBytes + rd_b[half];
      xf[s] = *reinterpret_cast<const u32x4*>(b + s * 16 * kRowBytes);
    }
  };
  f32x4 acc[8][NY];
  // one half step: the NP products of (xc, yc) (x: B rows, y: A rows, so
  // each lane's four results are four consecutive output columns), the NR
  // reads of half `half` of the step in slots (sa, sb) into (xn, yn) and,
  // with LOAD, the NL loads of part lq into slot lslot.  Read f sits at
  // product (f NP) / NR, load l at product (l NP) / NL + 2.
  auto half_step = [&](auto first, auto load, auto whole, auto nl, const u32x4 (&xc)[8],
                       const u32x4 (&yc)[NY], u32x4 (&xn)[8], u32x4 (&yn)[NY], int sa, int sb, int half,
                       int lq, int lslot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      mma_agpr<DT, decltype(first)::value>(acc[i / NY][i % NY], xc[i / NY], yc[i % NY]);
      {
        const int f = (i * NR + NP - 1) / NP;
        if (f < NR && (f * NP) / NR == i) read1(sa, sb, half, f, xn, yn);
      }
      if constexpr (decltype(load)::value) {
        constexpr int NL = decltype(nl)::value;
        const int j = i - 2;
        const int l = j < 0 ? NL : (j * NL + NP - 1) / NP;
        if (l < NL && (l * NP) / NL == j) load1(whole, lq, lslot, l);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Yes = std::true_type;
  using No = std::false_type;
  using LoadsB = std::integral_constant<int, 8>;
  using LoadsA = std::integral_constant<int, NA>;
  auto wrap = [](int s) __attribute__((always_inline)) { return s >= kSlots ? s - kSlots : s; };
  u32x4 xa[8], ya[NY], xb[8], yb[NY];
  if (nk > 0) {
    // parts 0..4 (A0 B0 A1 B1 A2) at once, into slots 0..4; the first
    // barrier waits for A0 and B0 only
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int nq = (q & 1) == 0 ? NA : 8;
      if ((q >> 1) < nk_full) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < nq) load1(Yes{}, q, q, j);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < nq) load1(No{}, q, q, j);
      }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * NA + 8));   // loads complete in order
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int f = 0; f < NR; ++f) read1(0, 1, 0, f, xa, ya);
    // step 0: its first half's products (from zero) carry the second half's
    // reads
    half_step(Yes{}, No{}, No{}, LoadsB{}, xa, ya, xb, yb, 0, 1, 1, 0, 0);
    // step kt: A in slot sa (2 kt mod 5), B in sa + 1; B of step kt + 1 goes
    // to sa + 3 and A of step kt + 2 to sa + 4 (mod 5), the slots of step
    // kt - 1
    auto step = [&](auto whole, int kt, int sa) __attribute__((always_inline)) {
      // A and B of step kt have landed for every wave (A of step kt + 1,
      // the last NA loads, may still be landing), and every wave is done
      // reading step kt - 1
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(NA));
      __builtin_amdgcn_s_barrier();
      const int sb = wrap(sa + 1);
      half_step(No{}, Yes{}, whole, LoadsB{}, xb, yb, xa, ya, sa, sb, 0, 2 * kt + 3, wrap(sa + 3));  // kt - 1, 2nd half
      half_step(No{}, Yes{}, whole, LoadsA{}, xa, ya, xb, yb, sa, sb, 1, 2 * kt + 4, wrap(sa + 4));  // kt, 1st half
    };
    // two loops rather than a branch per step, which would split the
    // registers' assignment between two copies of the products
    int kt = 1, sa = 2;
    for (; kt + 2 < nk_full; ++kt, sa = wrap(sa + 2)) step(Yes{}, kt, sa);   // loads of whole steps
    for (; kt < nk; ++kt, sa = wrap(sa + 2)) step(No{}, kt, sa);             // the partial step, past it
#pragma unroll
    for (int i = 0; i < NP; ++i) mma_agpr<DT, false>(acc[i / NY][i % NY], xb[i / NY], yb[i % NY]);
    settle_agprs_rows(acc);
  } else {
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int y = 0; y < NY; ++y) acc[x][y] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // the last loads (zeros past k) may still be landing in the LDS the
  // results are staged in
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  __builtin_amdgcn_s_barrier();
  store_tile<DT, TM, BN, WR, 128, kThreads>(acc, p, tile, m0, n0, wm, wn, tid,
                                            reinterpret_cast<uint32_t*>(lds));
}

template <int DT>
__global__ __launch_bounds__(kThreads) void gemm_wide_kernel(Params p) {
  wide_tile<DT, 256>(p);
}
template <int DT>
__global__ __launch_bounds__(kThreads) void gemm_wide192_kernel(Params p) {
  wide_tile<DT, 192>(p);
}
template <int DT>
__global__ __launch_bounds__(kThreads) void gemm_wide160_kernel(Params p) {
  wide_tile<DT, 160>(p);
}

// The 256 x 128 tile, for products whose 256 x 256 tiles would leave much of
// their last round of workgroups idle: four waves, one per SIMD, each a
// 128 x 64 block of 4 x 8 products (128 accumulators in AGPRs).  The
// operand path is the wide kernel's, scaled to the narrower tile: loads
// straight into LDS, a ring of three 48 KiB step slots (A 32 KiB, B 16 KiB;
// step kt loads step kt + 2 into the slot step kt - 1 freed, so every load
// has one to two steps to land), whole steps loaded with the step in the
// scalar offset, per-lane read bases fixed for the kernel.  Each 32-wide
// half step's 32 products carry its 12 fragment reads and six of the step's
// 12 loads.  Against the eight-wave kernel it replaced (4 x 2 blocks of
// 64 x 64, loads staged through registers and written to LDS, two waves per
// SIMD), in one process, bitwise equal: 60.7 against 63.1 us at 1024
// tokens, 155.4 against 169.7 at 2560 (8192 x 3584 bf16 weights).
constexpr int kNarrowStepBytes = (BM + BN_NARROW) * kRowBytes;   // 48 KiB
constexpr int kNarrowSlots = 3;
static_assert(kNarrowSlots * kNarrowStepBytes <= 160 * 1024, "gfx950 LDS per workgroup");

template <int DT>
__global__ __launch_bounds__(kThreads) void gemm_narrow_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kNarrowSlots * kNarrowStepBytes];
  const int tile = tile_at(position_of_wg((int)blockIdx.x, p.sched.tiles), p.sched);
  const int m0 = (tile / p.sched.tiles_n) * BM;
  const int n0 = (tile % p.sched.tiles_n) * BN_NARROW;
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // wave block: rows wm * 128, columns wn * 64
  const int nk = (p.k + BK - 1) / BK;
  const int a_tile_rows = p.m - m0 < BM ? p.m - m0 : BM;
  const int b_tile_rows = p.n - n0 < BN_NARROW ? p.n - n0 : BN_NARROW;
  // buffer resources as in the wide kernel
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + (int64_t)m0 * p.lda), (short)0,
      (int)(((int64_t)(a_tile_rows - 1) * p.lda + p.k) * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b + (int64_t)n0 * p.ldb), (short)0,
      (int)(((int64_t)(b_tile_rows - 1) * p.ldb + p.k) * 2), kRsrcWord3);
  // loads 0..7 of a step move this wave's A rows 64 wave + 8 j + lane / 8,
  // loads 8..11 its B rows 32 wave + 8 (j - 8) + lane / 8; LDS chunk
  // position lane % 8 of a row holds global chunk (lane % 8) ^ (row % 8)
  const int lr = lane >> 3, gchunk = (lane & 7) ^ lr;
  int off[12];
#pragma unroll
  for (int j = 0; j < 12; ++j) {
    if (j < 8) {
      const int r = 64 * wave + 8 * j + lr;
      off[j] = ((r < a_tile_rows ? r : a_tile_rows - 1) * (int)p.lda + gchunk * 8) * 2;
    } else {
      const int r = 32 * wave + 8 * (j - 8) + lr;
      off[j] = ((r < b_tile_rows ? r : b_tile_rows - 1) * (int)p.ldb + gchunk * 8) * 2;
    }
  }
  const int nk_full = p.k / BK;
  // load j of step kt into slot `slot` (A rows first, then B rows)
  auto load1 = [&](auto whole, int kt, int slot, int j) __attribute__((always_inline)) {
    unsigned char* dst = lds + slot * kNarrowStepBytes +
                         (j < 8 ? (64 * wave + 8 * j) * kRowBytes
                                : BM * kRowBytes + (32 * wave + 8 * (j - 8)) * kRowBytes);
    if constexpr (decltype(whole)::value) {
      if (j < 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)dst, 16, off[j], kt * BK * 2, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)dst, 16, off[j], kt * BK * 2, 0, 0);
    } else {
      const bool kin = kt * BK + gchunk * 8 < p.k;
      if (j < 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)dst, 16,
                                                 kin ? off[j] + kt * BK * 2 : kOutOfRange, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)dst, 16,
                                                 kin ? off[j] + kt * BK * 2 : kOutOfRange, 0, 0, 0);
    }
  };
  // per-lane byte offsets, inside a slot, of the first A and B fragment of
  // each half step; fragment s lies 16 rows (2 KiB) further
  uint32_t rd_a[2], rd_b[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = h * 4 + (lane >> 4);
    const int ra = wm * 128 + (lane & 15), rb = wn * 64 + (lane & 15);
    rd_a[h] = (uint32_t)(ra * kRowBytes + ((c ^ (ra & 7)) * 16));
    rd_b[h] = (uint32_t)(BM * kRowBytes + rb * kRowBytes + ((c ^ (rb & 7)) * 16));
  }
  // fragment f (0..11) of half `half` of the step in `slot`, in the order
  // the products use them (x 0, y 0..7, x 1..3)
  auto read1 = [&](int slot, int half, int f, u32x4 (&xf)[4], u32x4 (&yf)[8])
                   __attribute__((always_inline)) {
    const unsigned char* base = lds + slot * kNarrowStepBytes;
    if (f >= 1 && f <= 8) {
      yf[f - 1] = *reinterpret_cast<const u32x4*>(base + rd_a[half] + (f - 1) * 16 * kRowBytes);
    } else {
      const int s = f == 0 ? 0 : f - 8;
      xf[s] = *reinterpret_cast<const u32x4*>(base + rd_b[half] + s * 16 * kRowBytes);
    }
  };
  f32x4 acc[4][8];
  // one half step: the 32 products of (xc, yc), the 12 reads of half `half`
  // of the step in `slot` into (xn, yn) spread between them, and with LOAD
  // loads 6 PART .. 6 PART + 5 of step lkt into slot lslot, one every five
  // products
  auto half_step = [&](auto first, auto load, auto whole, auto part, const u32x4 (&xc)[4],
                       const u32x4 (&yc)[8], u32x4 (&xn)[4], u32x4 (&yn)[8], int slot, int half,
                       int lkt, int lslot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      mma_agpr<DT, decltype(first)::value>(acc[i / 8][i % 8], xc[i / 8], yc[i % 8]);
#pragma unroll
      for (int f = 0; f < 12; ++f)
        if (i == (f * 8) / 3) read1(slot, half, f, xn, yn);
      if (decltype(load)::value && i % 5 == 3) load1(whole, lkt, lslot, decltype(part)::value * 6 + i / 5);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Yes = std::true_type;
  using No = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  auto wrap = [](int s) __attribute__((always_inline)) { return s >= kNarrowSlots ? s - kNarrowSlots : s; };
  u32x4 xa[4], ya[8], xb[4], yb[8];
  if (nk > 0) {
    // steps 0..2 into slots 0..2 at once; the first barrier waits for step 0
#pragma unroll
    for (int t = 0; t < kNarrowSlots; ++t) {
      if (t < nk_full) {
#pragma unroll
        for (int j = 0; j < 12; ++j) load1(Yes{}, t, t, j);
      } else {
#pragma unroll
        for (int j = 0; j < 12; ++j) load1(No{}, t, t, j);
      }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(24));   // loads complete in order
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int f = 0; f < 12; ++f) read1(0, 0, f, xa, ya);
    half_step(Yes{}, No{}, No{}, P0{}, xa, ya, xb, yb, 0, 1, 0, 0);
    // step kt is in slot s = kt mod 3 and loads step kt + 2 into slot s + 2
    // (mod 3), which step kt - 1 used
    auto step = [&](auto whole, int kt, int s) __attribute__((always_inline)) {
      // step kt has landed for every wave (step kt + 1 may still be
      // landing), and every wave is done reading step kt - 1
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(12));
      __builtin_amdgcn_s_barrier();
      const int ls = wrap(s + 2);
      half_step(No{}, Yes{}, whole, P0{}, xb, yb, xa, ya, s, 0, kt + 2, ls);   // step kt - 1, second half
      half_step(No{}, Yes{}, whole, P1{}, xa, ya, xb, yb, s, 1, kt + 2, ls);   // step kt, first half
    };
    int kt = 1, s = 1;
    for (; kt + 2 < nk_full; ++kt, s = wrap(s + 1)) step(Yes{}, kt, s);   // loads of whole steps
    for (; kt < nk; ++kt, s = wrap(s + 1)) step(No{}, kt, s);             // the partial step, past it
#pragma unroll
    for (int i = 0; i < 32; ++i) mma_agpr<DT, false>(acc[i / 8][i % 8], xb[i / 8], yb[i % 8]);
    settle_agprs(acc);
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 8; ++y) acc[x][y] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // the last loads (zeros past k) may still be landing in the LDS the
  // results are staged in
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  __builtin_amdgcn_s_barrier();
  store_tile<DT, BM, BN_NARROW, 128, 64, kThreads>(acc, p, tile, m0, n0, wm, wn, tid,
                                               reinterpret_cast<uint32_t*>(lds));
}

}  // namespace gsc

namespace {

constexpr int64_t kIntMax = 0x7FFFFFFF;

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t p = (uintptr_t)a, q = (uintptr_t)b;
  return p < q + nb && q < p + na;
}

size_t extent(int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)(((rows - 1) * ld + cols) * elem);
}

}  // namespace

namespace {

// tile width a call uses: the requested one, or for 0 the automatic choice;
// -1 for anything else
int resolve_tile_n(int64_t m, int64_t n, int tile_n) {
  if (tile_n == gsc::BN || tile_n == gsc::BN_NARROW) return tile_n;
  if (tile_n != 0) return -1;
  const int64_t tiles_m = (m + gsc::BM - 1) / gsc::BM;
  const int64_t wide = tiles_m * ((n + gsc::BN - 1) / gsc::BN);
  const int64_t narrow = tiles_m * ((n + gsc::BN_NARROW - 1) / gsc::BN_NARROW);
  const int64_t cus = GEMM_SCATTER_CUS;
  return wide > 0 && (narrow + cus - 1) / cus <= (wide + cus - 1) / cus ? gsc::BN_NARROW : gsc::BN;
}

// forced height of the 256-wide tiles (gemm_scatter_tune); 0: automatic
std::atomic<int> g_tile_m{0};

// Estimated time of the 256-wide tiles at height h, in arbitrary units:
// rounds of workgroups, a partial round counting 0.7 + 0.3 f of a full one
// (f the fraction of CUs it keeps busy: fewer tiles share the memory
// system), times a round's cost, a fixed part plus a part in proportion to
// the tile's rows.  Fitted to the 4096 x 8192 x 3584 bf16 product's rounds
// on 8192 x 3584 weights: 85.6, 68.3 and 62.5 us per full round of 256-,
// 192- and 160-row tiles, and 67.6 us for a quarter-full round of 256-row
// tiles beside 85.6 for a full one.
int64_t wide_cost(int64_t m, int64_t n, int h) {
  const int64_t cus = GEMM_SCATTER_CUS;
  const int64_t t = ((m + h - 1) / h) * ((n + gsc::BN - 1) / gsc::BN);
  const int64_t full = t / cus, rem = t % cus;
  const int64_t rounds = 1000 * full + (rem ? 700 + 300 * rem / cus : 0);
  return rounds * (390 + 1000 * h / gsc::BM);
}

// tile height a call uses: 256 rows for the 128-wide tiles; for the 256-wide
// ones the forced height, else the cheapest of 256, 192 and 160 rows by
// wide_cost (ties to the taller tile)
int resolve_tile_m(int64_t m, int64_t n, int tn) {
  if (tn != gsc::BN) return gsc::BM;
  const int forced = g_tile_m.load(std::memory_order_relaxed);
  if (forced) return forced;
  int best = gsc::BM;
  int64_t best_cost = wide_cost(m, n, gsc::BM);
  for (int h : {192, 160}) {
    const int64_t c = wide_cost(m, n, h);
    if (c < best_cost) {
      best = h;
      best_cost = c;
    }
  }
  return best;
}

}  // namespace

extern "C" int gemm_scatter_tile_n(int64_t m, int64_t n) {
  if (m < 0 || n < 0 || m > kIntMax || n > kIntMax) return -1;
  return resolve_tile_n(m, n, 0);
}

extern "C" int gemm_scatter_tile_m(int64_t m, int64_t n, int tile_n) {
  if (m < 0 || n < 0 || m > kIntMax || n > kIntMax) return -1;
  const int tn = resolve_tile_n(m, n, tile_n);
  return tn < 0 ? -1 : resolve_tile_m(m, n, tn);
}

extern "C" int gemm_scatter_tune(int tile_m) {
  if (tile_m != 0 && tile_m != 256 && tile_m != 192 && tile_m != 160)
    return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter_tune: tile_m must be 0, 256, 192 or 160");
  g_tile_m.store(tile_m, std::memory_order_relaxed);
  return RMSN_OK;
}

extern "C" int64_t gemm_scatter_tiles(int64_t m, int64_t n, int tile_n) {
  if (m < 0 || n < 0 || m > kIntMax || n > kIntMax) return -1;
  const int tn = resolve_tile_n(m, n, tile_n);
  if (tn < 0) return -1;
  const int tm = resolve_tile_m(m, n, tn);
  const int64_t t = ((m + tm - 1) / tm) * ((n + tn - 1) / tn);
  return t > kIntMax ? -1 : t;
}

extern "C" int gemm_scatter_schedule(int64_t m, int64_t n, int world, int rank, int tile_n,
                                     int32_t* wg_tile, int32_t* pos_tile, int64_t len) {
  const int64_t tiles = gemm_scatter_tiles(m, n, tile_n);
  if (tiles < 0 || world < 1 || world > GEMM_SCATTER_WORLD_MAX || rank < 0 || rank >= world ||
      m % world != 0 || len < tiles)
    return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter_schedule: bad sizes, tile width, world or rank");
  const int tn = resolve_tile_n(m, n, tile_n);
  const gsc::Sched s = gsc::make_sched((int)m, (int)n, resolve_tile_m(m, n, tn), tn, world, rank);
  for (int w = 0; w < s.tiles; ++w) {
    if (wg_tile) wg_tile[w] = gsc::tile_at(gsc::position_of_wg(w, s.tiles), s);
    if (pos_tile) pos_tile[w] = gsc::tile_at(w, s);
  }
  return RMSN_OK;
}

extern "C" int gemm_scatter_fwd(void* const* dst, int64_t ldd, int world, int rank,
                                const void* a, int64_t lda, const void* b, int64_t ldb,
                                const void* c, int64_t ldc, float alpha, float beta, int64_t m,
                                int64_t n, int64_t k, int dtype, uint32_t* flags, uint32_t epoch,
                                int tile_n, void* stream) {
  if (dtype != RMSN_F16 && dtype != RMSN_BF16)
    return rmsn_set_error(RMSN_ERR_DTYPE, "gemm_scatter: dtype must be f16 or bf16");
  if (m < 0 || n < 0 || k < 0 || m > kIntMax || n > kIntMax || k > kIntMax)
    return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: m, n, k must lie in [0, 2^31)");
  const int tn = resolve_tile_n(m, n, tile_n);
  if (tn < 0) return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: tile_n must be 0, 128 or 256");
  if (world < 1 || world > GEMM_SCATTER_WORLD_MAX || rank < 0 || rank >= world)
    return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: world or rank out of range");
  if (m % world != 0) return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: m % world != 0");
  if (!dst) return rmsn_set_error(RMSN_ERR_NULL, "gemm_scatter: dst is NULL");
  if (m == 0 || n == 0) return RMSN_OK;
  for (int q = 0; q < world; ++q)
    if (!dst[q]) return rmsn_set_error(RMSN_ERR_NULL, "gemm_scatter: a dst chunk is NULL");
  if (k > 0 && (!a || !b)) return rmsn_set_error(RMSN_ERR_NULL, "gemm_scatter: a or b is NULL");
  if (ldd < n || (c && ldc < n) || lda < k || ldb < k)
    return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: a stride is shorter than its row");
  if (k > 0 && (k % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0 || ((uintptr_t)a & 15u) ||
                ((uintptr_t)b & 15u)))
    return rmsn_set_error(RMSN_ERR_SHAPE,
                          "gemm_scatter: k, lda, ldb must be multiples of 8 and a, b 16-byte aligned");
  // operand offsets inside one tile's rows are 32-bit byte offsets
  if (k > 0 && ((int64_t)(gsc::BM - 1) * lda + k >= (int64_t)1 << 29 ||
                (int64_t)(gsc::BN - 1) * ldb + k >= (int64_t)1 << 29))
    return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: lda or ldb too large (255 * ld + k >= 2^29)");
  // output access width: 2 = 16-byte rows (staged tile stores), 1 = 8-byte
  // (direct stores), 0 = element by element; C is read 8 bytes at a time
  bool vec = (ldd % 4 == 0) && (!c || (ldc % 4 == 0 && ((uintptr_t)c & 7u) == 0));
  bool vec16 = vec && ldd % 8 == 0;
  for (int q = 0; q < world; ++q) {
    if ((uintptr_t)dst[q] & 1u) return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: dst misaligned");
    if ((uintptr_t)dst[q] & 7u) vec = false;
    if ((uintptr_t)dst[q] & 15u) vec16 = false;
  }
  if ((c && ((uintptr_t)c & 1u)) || (flags && ((uintptr_t)flags & 3u)))
    return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: c or flags misaligned");

  const int64_t chunk_rows = m / world;
  const int64_t tiles = gemm_scatter_tiles(m, n, tn);
  if (tiles < 0) return rmsn_set_error(RMSN_ERR_SHAPE, "gemm_scatter: too many tiles");
  const size_t dext = extent(chunk_rows, n, ldd, 2);
  const size_t aext = k > 0 ? extent(m, k, lda, 2) : 0, bext = k > 0 ? extent(n, k, ldb, 2) : 0;
  const size_t cext = c ? extent(m, n, ldc, 2) : 0;
  const size_t fext = flags ? (size_t)tiles * 4 : 0;
  for (int q = 0; q < world; ++q) {
    if (overlap(dst[q], dext, a, aext) || overlap(dst[q], dext, b, bext) ||
        overlap(dst[q], dext, c, cext) || overlap(dst[q], dext, flags, fext))
      return rmsn_set_error(RMSN_ERR_ALIAS, "gemm_scatter: a dst chunk overlaps an input or flags");
    for (int r = 0; r < q; ++r)
      if (overlap(dst[q], dext, dst[r], dext))
        return rmsn_set_error(RMSN_ERR_ALIAS, "gemm_scatter: dst chunks overlap");
  }
  // the flag stores must not land on operands other workgroups still read
  if (overlap(flags, fext, a, aext) || overlap(flags, fext, b, bext) ||
      overlap(flags, fext, c, cext))
    return rmsn_set_error(RMSN_ERR_ALIAS, "gemm_scatter: flags overlap a, b or c");

  gsc::Params p{};
  p.a = static_cast<const uint16_t*>(a);
  p.b = static_cast<const uint16_t*>(b);
  p.c = static_cast<const uint16_t*>(c);
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = c ? ldc : 0;
  p.ldd = ldd;
  for (int q = 0; q < world; ++q) p.dst[q] = static_cast<uint16_t*>(dst[q]);
  p.flags = flags;
  p.epoch = epoch;
  p.m = (int)m;
  p.n = (int)n;
  p.k = (int)k;
  p.chunk_rows = (int)chunk_rows;
  p.alpha = alpha;
  p.beta = beta;
  p.vec_out = vec16 ? 2 : vec ? 1 : 0;
  const int tm = resolve_tile_m(m, n, tn);
  p.sched = gsc::make_sched((int)m, (int)n, tm, tn, world, rank);

  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)tiles);
  if (tn == gsc::BN) {
    const dim3 block(gsc::kThreads);
    const bool bf = dtype == RMSN_BF16;
    if (tm == 192) {
      if (bf) hipLaunchKernelGGL((gsc::gemm_wide192_kernel<RMSN_BF16>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((gsc::gemm_wide192_kernel<RMSN_F16>), grid, block, 0, st, p);
    } else if (tm == 160) {
      if (bf) hipLaunchKernelGGL((gsc::gemm_wide160_kernel<RMSN_BF16>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((gsc::gemm_wide160_kernel<RMSN_F16>), grid, block, 0, st, p);
    } else {
      if (bf) hipLaunchKernelGGL((gsc::gemm_wide_kernel<RMSN_BF16>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((gsc::gemm_wide_kernel<RMSN_F16>), grid, block, 0, st, p);
    }
  } else {
    const dim3 block(gsc::kThreads);
    if (dtype == RMSN_BF16)
      hipLaunchKernelGGL((gsc::gemm_narrow_kernel<RMSN_BF16>), grid, block, 0, st, p);
    else
      hipLaunchKernelGGL((gsc::gemm_narrow_kernel<RMSN_F16>), grid, block, 0, st, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    char msg[200];
    snprintf(msg, sizeof(msg), "gemm_scatter launch failed: %s", hipGetErrorString(e));
    return rmsn_set_error(RMSN_ERR_HIP, msg);
  }
  return RMSN_OK;
}
