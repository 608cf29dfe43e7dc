// rmsnorm_table.hpp -- instantiates the kernel variants for one combination
// of data, gamma and output dtypes and builds its descriptor table (included
// by the per-dtype translation units).
#pragma once

#include <stdio.h>

#include <vector>

#include "rmsnorm_kernels.hpp"
#include "rmsnorm_variants.hpp"

namespace rmsn {

inline const char* width_name(int vb) {
  switch (vb) {
    case 16: return "vec";
    case 8: return "v8";
    case 4: return "v4";
    default: return "elem";
  }
}

inline const char* dtype_name(int code) {
  switch (code) {
    case 0: return "f32";
    case 1: return "f16";
    default: return "bf16";
  }
}

struct Types {
  int d, g, o;  // data, gamma, output dtype codes
};

inline void add_variant(std::vector<Variant>& v, Types t, int kind, int vb, int tpr, int npt,
                        int wgs, int kc, int lds, int unr, int nt, const void* fn, int ag = 0) {
  Variant d{};
  // Single-dtype variants are named by the data dtype alone; the general
  // interface's add gamma's and the output's dtypes.
  char types[48];
  if (t.g == t.d && t.o == t.d)
    snprintf(types, sizeof(types), "%s", dtype_name(t.d));
  else
    snprintf(types, sizeof(types), "%s,g=%s,o=%s", dtype_name(t.d), dtype_name(t.g),
             dtype_name(t.o));
  if (kind == kVgpr)
    snprintf(d.name, sizeof(d.name), "vgpr<%s,tpr=%d,npt=%d,wg=%d,k=%d%s%s>", types, tpr, npt,
             wgs, kc, nt ? ",nt" : "", ag ? ",ag" : "");
  else
    snprintf(d.name, sizeof(d.name), "stream<%s,%s,wg=%d,%s,k=%d,unr=%d%s%s>", types,
             width_name(vb), wgs, lds ? "lds" : "reread", kc, unr, nt ? ",nt" : "",
             ag ? ",ag" : "");
  d.nt = nt;
  d.ag = ag;
  d.dtype = t.d;
  d.gdtype = t.g;
  d.odtype = t.o;
  d.kind = kind;
  d.vb = vb;
  d.tpr = tpr;
  d.npt = npt;
  d.wgs = wgs;
  d.kc = kc;
  d.lds_stage = lds;
  d.unroll = unr;
  d.fn = fn;
  v.push_back(d);
}

// Every variant of the single-dtype interface (full shape lists, for the
// dispatcher and for sweeps).
// Shapes left out because they spill registers to scratch memory: the
// K = 8 register kernel holding 2048 chunk slots per row (nine chunk sets per
// thread), and the 16-byte runtime-K streaming kernel with four chunks in
// flight on 1024 lanes.  The dispatcher never picks them.
template <int KC, int TPR, int NPT>
constexpr bool vgpr_spills() { return KC == 8 && TPR * NPT >= 2048; }
template <int VB, int WGS, int KC, int UNR>
constexpr bool stream_spills() { return VB == 16 && WGS == 1024 && KC < 0 && UNR >= 4; }

template <typename T>
void add_full(std::vector<Variant>& v, Types t) {
#define RMSN_ADD_VGPR_K(KC, TPR, NPT, WGS, NT)                                          \
  if constexpr (!vgpr_spills<KC, TPR, NPT>())                                           \
    add_variant(v, t, kVgpr, 16, TPR, NPT, WGS, KC, 0, 0, NT ? 1 : 0,                    \
                reinterpret_cast<const void*>(&row_vgpr_kernel<T, T, T, TPR, NPT, WGS, KC, NT>));
#define RMSN_ADD_VGPR(TPR, NPT, WGS, NT) RMSN_KCS(RMSN_ADD_VGPR_K, TPR, NPT, WGS, NT)
  RMSN_VGPR_SHAPES(RMSN_ADD_VGPR)
#define RMSN_ADD_STREAM_K(KC, VB, WGS, LDS, NT, UNR)                                    \
  if constexpr ((VB == 0 || VB > (int)sizeof(typename DT<T>::scalar_t)) &&               \
                !stream_spills<VB, WGS, KC, UNR>() && (KC != -2 || (VB == 8 && LDS)))    \
    add_variant(v, t, kStream, VB, WGS, 0, WGS, KC, LDS ? 1 : 0, UNR, NT ? 1 : 0,         \
                reinterpret_cast<const void*>(                                           \
                    &row_stream_kernel<T, T, T, VB, WGS, LDS, KC, UNR, NT>));
#define RMSN_ADD_STREAM(VB, WGS, LDS, NT, UNR) \
  RMSN_STREAM_KCS(RMSN_ADD_STREAM_K, VB, WGS, LDS, NT, UNR)
  RMSN_STREAM_SHAPES(RMSN_ADD_STREAM)
#undef RMSN_ADD_VGPR_K
#undef RMSN_ADD_VGPR
#undef RMSN_ADD_STREAM_K
#undef RMSN_ADD_STREAM
}

// The variants of one general combination (data T, gamma GT, output OT).
template <typename T, typename GT, typename OT>
void add_mixed(std::vector<Variant>& v, Types t) {
#define RMSN_ADD_VGPR_K(KC, TPR, NPT, WGS, NT)                                          \
  add_variant(v, t, kVgpr, 16, TPR, NPT, WGS, KC, 0, 0, NT ? 1 : 0,                      \
              reinterpret_cast<const void*>(&row_vgpr_kernel<T, GT, OT, TPR, NPT, WGS, KC, NT>));
#define RMSN_ADD_VGPR(TPR, NPT, WGS, NT) RMSN_MIXED_KCS(RMSN_ADD_VGPR_K, TPR, NPT, WGS, NT)
  RMSN_MIXED_VGPR_SHAPES(RMSN_ADD_VGPR)
#define RMSN_ADD_STREAM_K(KC, VB, WGS, LDS, NT, UNR)                                    \
  if constexpr (VB == 0 || VB > (int)sizeof(typename DT<T>::scalar_t))                   \
    add_variant(v, t, kStream, VB, WGS, 0, WGS, KC, LDS ? 1 : 0, UNR, NT ? 1 : 0,         \
                reinterpret_cast<const void*>(                                           \
                    &row_stream_kernel<T, GT, OT, VB, WGS, LDS, KC, UNR, NT>));
#define RMSN_ADD_STREAM(VB, WGS, LDS, NT, UNR) \
  RMSN_MIXED_KCS(RMSN_ADD_STREAM_K, VB, WGS, LDS, NT, UNR)
  RMSN_MIXED_STREAM_SHAPES(RMSN_ADD_STREAM)
#undef RMSN_ADD_VGPR_K
#undef RMSN_ADD_VGPR
#undef RMSN_ADD_STREAM_K
#undef RMSN_ADD_STREAM
}

// The all-gather variants of one dtype (add_rmsnorm_ag_fwd).
template <typename T>
void add_ag(std::vector<Variant>& v, Types t) {
#define RMSN_ADD_VGPR_K(KC, TPR, NPT, WGS, NT)                                          \
  add_variant(v, t, kVgpr, 16, TPR, NPT, WGS, KC, 0, 0, NT ? 1 : 0,                      \
              reinterpret_cast<const void*>(&row_vgpr_kernel<T, T, T, TPR, NPT, WGS, KC, NT, true>), 1);
#define RMSN_ADD_VGPR(TPR, NPT, WGS, NT) RMSN_AG_VGPR_KCS(RMSN_ADD_VGPR_K, TPR, NPT, WGS, NT)
  RMSN_AG_VGPR_SHAPES(RMSN_ADD_VGPR)
#define RMSN_ADD_STREAM_K(KC, VB, WGS, LDS, NT, UNR)                                    \
  if constexpr ((VB == 0 || VB > (int)sizeof(typename DT<T>::scalar_t)) &&               \
                (KC != -2 || (VB == 8 && LDS)))                                          \
    add_variant(v, t, kStream, VB, WGS, 0, WGS, KC, LDS ? 1 : 0, UNR, NT ? 1 : 0,         \
                reinterpret_cast<const void*>(                                           \
                    &row_stream_kernel<T, T, T, VB, WGS, LDS, KC, UNR, NT, true>), 1);
#define RMSN_ADD_STREAM(VB, WGS, LDS, NT, UNR) \
  RMSN_AG_STREAM_KCS(RMSN_ADD_STREAM_K, VB, WGS, LDS, NT, UNR)
  RMSN_MIXED_STREAM_SHAPES(RMSN_ADD_STREAM)
#undef RMSN_ADD_VGPR_K
#undef RMSN_ADD_VGPR
#undef RMSN_ADD_STREAM_K
#undef RMSN_ADD_STREAM
}

}  // namespace rmsn

// One exported table per translation unit: rmsn_table_<NAME>(&n); the
// statements after NAME fill the vector v.
#define RMSN_DEFINE_TABLE(NAME, ...)                                        \
  const rmsn::Variant* rmsn_table_##NAME(int* n) {                          \
    static const std::vector<rmsn::Variant> table = [] {                    \
      std::vector<rmsn::Variant> v;                                         \
      __VA_ARGS__;                                                          \
      return v;                                                             \
    }();                                                                    \
    *n = (int)table.size();                                                 \
    return table.data();                                                    \
  }
