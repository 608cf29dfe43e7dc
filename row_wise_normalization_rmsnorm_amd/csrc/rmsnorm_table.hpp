// rmsnorm_table.hpp -- instantiates every kernel variant for one dtype and
// builds its descriptor table (included once per dtype translation unit).
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

inline void add_variant(std::vector<Variant>& v, int dtype, const char* dname, int kind, int vb,
                        int tpr, int npt, int wgs, int kc, int lds, int unr, int nt,
                        const void* fn) {
  Variant d{};
  if (kind == kVgpr)
    snprintf(d.name, sizeof(d.name), "vgpr<%s,tpr=%d,npt=%d,wg=%d,k=%d%s>", dname, tpr, npt, wgs,
             kc, nt ? ",nt" : "");
  else
    snprintf(d.name, sizeof(d.name), "stream<%s,%s,wg=%d,%s,k=%d,unr=%d%s>", dname,
             width_name(vb), wgs, lds ? "lds" : "reread", kc, unr, nt ? ",nt" : "");
  d.nt = nt;
  d.dtype = dtype;
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

template <typename T>
std::vector<Variant> build_table(int dtype, const char* dname) {
  std::vector<Variant> v;
#define RMSN_ADD_VGPR_K(KC, TPR, NPT, WGS, NT)                                        \
  add_variant(v, dtype, dname, kVgpr, 16, TPR, NPT, WGS, KC, 0, 0, NT ? 1 : 0,        \
              reinterpret_cast<const void*>(&row_vgpr_kernel<T, TPR, NPT, WGS, KC, NT>));
#define RMSN_ADD_VGPR(TPR, NPT, WGS, NT) RMSN_KCS(RMSN_ADD_VGPR_K, TPR, NPT, WGS, NT)
  RMSN_VGPR_SHAPES(RMSN_ADD_VGPR)
#define RMSN_ADD_STREAM_K(KC, VB, WGS, LDS, NT, UNR)                                  \
  if constexpr (VB == 0 || VB > (int)sizeof(typename DT<T>::scalar_t))                 \
    add_variant(v, dtype, dname, kStream, VB, WGS, 0, WGS, KC, LDS ? 1 : 0, UNR,        \
                NT ? 1 : 0,                                                             \
                reinterpret_cast<const void*>(                                         \
                    &row_stream_kernel<T, VB, WGS, LDS, KC, UNR, NT>));
#define RMSN_ADD_STREAM(VB, WGS, LDS, NT, UNR) \
  RMSN_STREAM_KCS(RMSN_ADD_STREAM_K, VB, WGS, LDS, NT, UNR)
  RMSN_STREAM_SHAPES(RMSN_ADD_STREAM)
#undef RMSN_ADD_VGPR_K
#undef RMSN_ADD_VGPR
#undef RMSN_ADD_STREAM_K
#undef RMSN_ADD_STREAM
  return v;
}

}  // namespace rmsn

#define RMSN_DEFINE_TABLE(T, CODE, DNAME)                                   \
  const rmsn::Variant* rmsn_table_##DNAME(int* n) {                         \
    static const std::vector<rmsn::Variant> table =                         \
        rmsn::build_table<T>(CODE, #DNAME);                                 \
    *n = (int)table.size();                                                 \
    return table.data();                                                    \
  }
