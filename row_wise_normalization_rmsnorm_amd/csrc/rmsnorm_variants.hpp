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
  char name[96];
  int dtype;      // 0 f32, 1 f16, 2 bf16
  int kind;       // kVgpr or kStream
  int vec;        // 1: 16-byte chunks, 0: element-wise
  int tpr;        // threads per row
  int npt;        // chunks per thread held in registers (vgpr)
  int wgs;        // threads per workgroup
  int kc;         // 0 plain, >0 fixed partial count, -1 runtime partial count
  int lds_stage;  // stream: stage the row in LDS (1) or re-read it (0)
  int unroll;     // stream: chunks in flight per thread per step
  const void* fn; // host stub for hipLaunchKernel
};

// Shapes of the register-resident kernel: (threads/row, chunks/thread, threads/WG).
#define RMSN_VGPR_SHAPES(X)                                                  \
  X(8, 1, 256) X(16, 1, 256) X(32, 1, 256) X(64, 1, 256) X(64, 2, 256)      \
  X(64, 4, 256) X(128, 2, 256) X(128, 4, 256) X(256, 1, 256) X(256, 2, 256) \
  X(256, 4, 256) X(512, 1, 512) X(512, 2, 512) X(512, 4, 512)               \
  X(1024, 1, 1024) X(1024, 2, 1024)

// Partial counts compiled as constants (others use the runtime-K kernel).
#define RMSN_KCS(X, ...) X(0, __VA_ARGS__) X(1, __VA_ARGS__) X(8, __VA_ARGS__) X(-1, __VA_ARGS__)

// Shapes of the streaming kernel: (16-byte chunks?, threads/WG, LDS stage?).
#define RMSN_STREAM_SHAPES(X)                                                          \
  X(true, 256, true) X(true, 512, true) X(true, 1024, true) X(true, 256, false)        \
  X(true, 512, false) X(true, 1024, false) X(false, 256, true) X(false, 512, true)     \
  X(false, 1024, true) X(false, 256, false) X(false, 512, false) X(false, 1024, false)

#define RMSN_STREAM_KCS(X, ...) X(0, __VA_ARGS__) X(1, __VA_ARGS__) X(-1, __VA_ARGS__)

}  // namespace rmsn
