// rmsnorm_variants.hpp -- the compiled kernel variants and their descriptors.
//
// Each dtype's translation unit instantiates every variant listed here and
// exports a table of descriptors; the host dispatcher (rmsnorm_api.hip) picks
// one per call from (hidden, rows, k, dtype, alignment) and launches it with
// hipLaunchKernel.
#pragma once

#include <hip/hip_runtime.h>

namespace rmsn {

enum Kind { kVgpr = 0, kStream = 1 };

struct Variant {
  char name[112];
  int dtype;      // data (partials, residual, x): 0 f32, 1 f16, 2 bf16
  int gdtype;     // gamma
  int odtype;     // output
  int kind;       // kVgpr or kStream
  int vb;         // bytes per chunk: 16, 8 or 4; 0 = one element per chunk
  int tpr;        // threads per row
  int npt;        // chunks per thread held in registers (vgpr)
  int wgs;        // threads per workgroup
  int kc;         // 0 plain, >0 fixed partial count, -1 runtime partial count
                  // (-2: runtime, two partials per step)
  int lds_stage;  // stream: stage the row in LDS (1) or re-read it (0)
  int unroll;     // stream: chunks in flight per thread per step
  int nt;         // streaming (nontemporal) loads/stores for row data
  int ag;         // all-gather epilogue: takes RowArgsAG, stores into every gather buffer
  const void* fn; // host stub for hipLaunchKernel
};

// Shapes of the register-resident kernel: (threads/row, chunks/thread,
// threads/WG, nontemporal).  Every shape streams with nontemporal accesses;
// a few are also built with cached accesses, for comparison.
#define RMSN_VGPR_SHAPES(X)                                                              \
  X(8, 1, 256, true) X(16, 1, 256, true) X(32, 1, 256, true) X(64, 1, 256, true)        \
  X(64, 2, 256, true) X(64, 4, 256, true) X(128, 1, 256, true) X(128, 2, 256, true)     \
  X(128, 4, 256, true)                                                                  \
  X(256, 1, 256, true) X(256, 2, 256, true) X(256, 4, 256, true) X(512, 1, 512, true)   \
  X(512, 2, 512, true) X(512, 4, 512, true) X(1024, 1, 1024, true)                      \
  X(1024, 2, 1024, true) X(64, 4, 256, false) X(256, 2, 256, false)                     \
  X(512, 1, 512, false) X(512, 4, 512, false) X(1024, 1, 1024, false)

// Partial counts compiled as constants (others use the runtime-K kernel).
#define RMSN_KCS(X, ...) X(0, __VA_ARGS__) X(1, __VA_ARGS__) X(8, __VA_ARGS__) X(-1, __VA_ARGS__)

// Shapes of the streaming kernel: (bytes per chunk (0: one element),
// threads/WG, LDS stage?, nontemporal, chunks in flight per thread).
// LDS-staged variants stream; re-reading ones keep the residual cacheable for
// the second pass.  4-byte chunks are built for 16-bit types only (for fp32
// they are the element-wise kernel).
#define RMSN_STREAM_SHAPES(X)                                                             \
  X(16, 256, true, true, 2) X(16, 512, true, true, 2) X(16, 1024, true, true, 2)          \
  X(16, 256, true, true, 4) X(16, 512, true, true, 4) X(16, 1024, true, true, 4)          \
  X(16, 256, false, false, 2) X(16, 512, false, false, 2) X(16, 1024, false, false, 2)    \
  X(16, 512, true, false, 2) X(16, 256, true, true, 1) X(16, 512, true, true, 1)         \
  X(8, 256, true, true, 2) X(8, 512, true, true, 2) X(8, 1024, true, true, 2)             \
  X(8, 256, true, true, 4) X(8, 512, true, true, 4) X(8, 1024, true, true, 4)             \
  X(8, 256, false, false, 4) X(8, 512, false, false, 4) X(8, 1024, false, false, 4)       \
  X(8, 256, true, true, 8)                                                                \
  X(4, 256, true, true, 4) X(4, 512, true, true, 4) X(4, 1024, true, true, 4)             \
  X(4, 256, false, false, 4) X(4, 512, false, false, 4) X(4, 1024, false, false, 4)       \
  X(0, 256, true, true, 4) X(0, 512, true, true, 4) X(0, 1024, true, true, 4)             \
  X(0, 256, false, false, 4) X(0, 512, false, false, 4) X(0, 1024, false, false, 4)

// -1: runtime K, one partial per step; -2: runtime K, two partials per step
// (built for the LDS-staged 8-byte shapes only).
#define RMSN_STREAM_KCS(X, ...) X(0, __VA_ARGS__) X(1, __VA_ARGS__) X(-1, __VA_ARGS__) X(-2, __VA_ARGS__)

// The general interface -- gamma in fp32 with 16-bit data, or an output dtype
// other than the data's -- compiles only the shapes the dispatcher picks
// (one or two chunks per thread up to 1024 threads; the streaming forms it
// uses), with plain and runtime-K fused forms.
#define RMSN_MIXED_VGPR_SHAPES(X)                                                        \
  X(8, 1, 256, true) X(16, 1, 256, true) X(32, 1, 256, true) X(64, 1, 256, true)        \
  X(128, 1, 256, true) X(256, 1, 256, true) X(512, 1, 512, true)                        \
  X(1024, 1, 1024, true) X(64, 2, 256, true) X(128, 2, 256, true) X(256, 2, 256, true)  \
  X(512, 2, 512, true) X(1024, 2, 1024, true)

#define RMSN_MIXED_STREAM_SHAPES(X)                                                       \
  X(16, 256, false, false, 2) X(16, 512, false, false, 2) X(16, 1024, false, false, 2)    \
  X(8, 256, true, true, 4) X(8, 512, true, true, 4) X(8, 1024, true, true, 4)             \
  X(8, 256, false, false, 4) X(8, 512, false, false, 4) X(8, 1024, false, false, 4)       \
  X(8, 256, true, true, 8)                                                                \
  X(4, 256, true, true, 4) X(4, 512, true, true, 4) X(4, 1024, true, true, 4)             \
  X(4, 256, false, false, 4) X(4, 512, false, false, 4) X(4, 1024, false, false, 4)       \
  X(0, 256, true, true, 4) X(0, 512, true, true, 4) X(0, 1024, true, true, 4)             \
  X(0, 256, false, false, 4) X(0, 512, false, false, 4) X(0, 1024, false, false, 4)

#define RMSN_MIXED_KCS(X, ...) X(0, __VA_ARGS__) X(-1, __VA_ARGS__)

// The fused form with an all-gather epilogue (add_rmsnorm_ag_fwd, one dtype)
// compiles the shapes the dispatcher picks for fused calls: the register
// kernel with one chunk per thread, with K = 1, 8 or any, and the streaming
// shapes of the general interface with runtime K (one partial per step, or
// two for the LDS-staged 8-byte shapes).
#define RMSN_AG_VGPR_SHAPES(X)                                                          \
  X(8, 1, 256, true) X(16, 1, 256, true) X(32, 1, 256, true) X(64, 1, 256, true)        \
  X(128, 1, 256, true) X(256, 1, 256, true) X(512, 1, 512, true) X(1024, 1, 1024, true)

#define RMSN_AG_VGPR_KCS(X, ...) X(1, __VA_ARGS__) X(8, __VA_ARGS__) X(-1, __VA_ARGS__)
#define RMSN_AG_STREAM_KCS(X, ...) X(-1, __VA_ARGS__) X(-2, __VA_ARGS__)

}  // namespace rmsn
