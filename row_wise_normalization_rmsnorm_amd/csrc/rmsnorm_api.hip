// rmsnorm_api.hip -- the C ABI of librmsnorm.so (include/rmsnorm.h):
// argument validation, aliasing rules, kernel choice, and the launch on the
// caller's stream.  Host code only; the kernels live in kernels_<dtype>.hip.
//
// Argument conventions follow the pages' problem statement: x[rows, hidden]
// with gamma[hidden] of the same dtype, a float eps and an out-of-place
// output (page "RMSNorm kernel", section 2, naive kernel signature), and for
// the fused form an input, a residual updated in place and a weight over
// num_tokens x hidden_size (page "Tokenweave fused-RMSNorm-AR kernel", "Code
// walkthrough").  Sizes are validated before any launch, as the torch
// bindings on page "Block All Reduce CUDA代码学习" check dtype and size before
// dispatching.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/rmsnorm.h"
#include "rmsnorm_kernels.hpp"
#include "rmsnorm_variants.hpp"

const rmsn::Variant* rmsn_table_f32(int* n);
const rmsn::Variant* rmsn_table_f16(int* n);
const rmsn::Variant* rmsn_table_bf16(int* n);

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int dtype_size(int dtype) { return dtype == RMSN_F32 ? 4 : 2; }

// LDS budget for staging one row in the streaming kernel.  64 KiB keeps at
// least two workgroups resident per CU (160 KiB of LDS per CU on gfx950).
constexpr int64_t kLdsStageMax = 64 * 1024;
// Upper bound on workgroups per launch; longer problems loop over rows.
constexpr int64_t kGridCapDefault = 1 << 20;
// Rows up to this many elements are held in registers.
constexpr int64_t kVgprMaxHidden = 8192;
// With two or more partials, rows of at least this many bytes use the
// streaming kernel (fewer registers per thread than holding K+1 chunk sets).
constexpr int64_t kStreamMinBytesForK = 8192;

const rmsn::Variant* table_for(int dtype, int* n) {
  switch (dtype) {
    case RMSN_F32: return rmsn_table_f32(n);
    case RMSN_F16: return rmsn_table_f16(n);
    case RMSN_BF16: return rmsn_table_bf16(n);
    default: *n = 0; return nullptr;
  }
}

// npt: chunks per thread (register kernel) or chunks in flight per step
// (streaming kernel).
const rmsn::Variant* find(int dtype, int kind, int vb, int tpr, int npt, int wgs, int kc, int lds,
                          int nt) {
  int n = 0;
  const rmsn::Variant* t = table_for(dtype, &n);
  for (int i = 0; i < n; ++i) {
    const rmsn::Variant& v = t[i];
    if (v.kind == kind && v.vb == vb && v.tpr == tpr && v.wgs == wgs && v.kc == kc &&
        v.nt == nt &&
        (kind == rmsn::kVgpr ? v.npt == npt : (v.lds_stage == lds && v.unroll == npt)))
      return &v;
  }
  return nullptr;
}

int vgpr_kc(int k) { return k == 0 ? 0 : (k == 1 || k == 8) ? k : -1; }
int stream_kc(int k) { return k == 0 ? 0 : k == 1 ? 1 : -1; }

struct Plan {
  const rmsn::Variant* v;
  int chunks;        // chunks per row for this variant
  size_t lds_bytes;  // dynamic LDS
};

// The widest chunk (16, 8 or 4 bytes; 0 = element) that divides both the
// row's byte length and the alignment every base pointer shares.
int widest_chunk(int dtype, int64_t hidden, int align) {
  const int s = dtype_size(dtype);
  for (int vb = 16; vb > s; vb /= 2)
    if (align >= vb && (hidden * s) % vb == 0) return vb;
  return 0;
}

int64_t chunks_of(const rmsn::Variant& v, int dtype, int64_t hidden) {
  return v.vb ? hidden * dtype_size(dtype) / v.vb : hidden;
}

// Can variant v run a call with these sizes and this base alignment?
bool fits(const rmsn::Variant& v, int dtype, int64_t hidden, int k, int align) {
  const int s = dtype_size(dtype);
  if (v.dtype != dtype) return false;
  if (v.vb && (align < v.vb || (hidden * s) % v.vb != 0)) return false;
  if (v.kind == rmsn::kVgpr) {
    if (v.kc != vgpr_kc(k) && !(v.kc == -1 && k > 0)) return false;
    return chunks_of(v, dtype, hidden) <= (int64_t)v.tpr * v.npt;
  }
  if (v.kc != stream_kc(k) && !(v.kc == -1 && k > 0)) return false;
  if (v.lds_stage && hidden * s > kLdsStageMax) return false;
  return true;
}

// The dispatcher.  Register-resident rows up to 8192 elements, packing rows
// into waves when they are short; streaming two-pass kernels above that
// (LDS-staged while the row fits the stage budget), for K >= 2 on long rows,
// and whenever 16-byte accesses do not fit the alignment or row length.
// align: the largest power of two (capped at 16) dividing every base pointer.
int choose(int dtype, int64_t hidden, int k, int align, Plan* plan) {
  const int s = dtype_size(dtype);
  const int vb = widest_chunk(dtype, hidden, align);
  const rmsn::Variant* v = nullptr;

  const char* forced = getenv("RMSNORM_VARIANT");
  if (forced && *forced) {
    int n = 0;
    const rmsn::Variant* t = table_for(dtype, &n);
    for (int i = 0; i < n && !v; ++i)
      if (strcmp(t[i].name, forced) == 0) v = &t[i];
    if (!v) return fail(RMSN_ERR_SHAPE, "RMSNORM_VARIANT=%s names no variant of this dtype", forced);
    if (!fits(*v, dtype, hidden, k, align))
      return fail(RMSN_ERR_SHAPE, "RMSNORM_VARIANT=%s cannot run hidden=%lld k=%d align=%d",
                  forced, (long long)hidden, k, align);
  } else if (vb == 16 && hidden <= kVgprMaxHidden &&
             !(k >= 2 && hidden * s >= kStreamMinBytesForK)) {
    // One 16-byte chunk per thread wherever a workgroup can cover the row:
    // threads per row = the next power of two >= chunks (several rows per
    // wave below 64 chunks), up to 1024 threads, then 2 or 4 chunks each.
    const int64_t C = hidden * s / 16;
    int tpr = 8;
    while (tpr < C && tpr < 1024) tpr *= 2;
    int npt = (int)((C + tpr - 1) / tpr);
    npt = npt <= 1 ? 1 : npt <= 2 ? 2 : 4;
    int wgs = tpr < 256 ? 256 : tpr;
    if (npt == 4 && tpr == 1024) {  // 16 waves x 4 chunks exceeds the register budget
      tpr = 512;
      wgs = 512;
    }
    v = find(dtype, rmsn::kVgpr, 16, tpr, npt, wgs, vgpr_kc(k), 0, 1);
  } else {
    // Streaming two-pass, LDS-staged while the row fits the stage budget.
    // Fused calls use the runtime-K form, which sums the partials one at a
    // time with few registers (measured faster than holding all K+1 chunk
    // sets in registers at K = 8).  The LDS-staged form moves 8-byte chunks,
    // four per thread, with just enough threads to put the whole row in
    // flight in one step: measured 3% faster than 16-byte chunks at K = 8
    // and 2% on 16384-wide rows.
    const bool lds = hidden * s <= kLdsStageMax;
    const int svb = (lds && vb == 16) ? 8 : vb;
    const int64_t C = svb ? hidden * s / svb : hidden;
    const int unr = svb == 16 ? 2 : 4;
    int wgs = 256;
    while (wgs < 1024 && (int64_t)wgs * unr < C) wgs *= 2;
    v = find(dtype, rmsn::kStream, svb, wgs, unr, wgs, k == 0 ? 0 : -1, lds ? 1 : 0,
             lds ? 1 : 0);
  }
  if (!v) return fail(RMSN_ERR_SHAPE, "no kernel variant for hidden=%lld k=%d", (long long)hidden, k);
  plan->v = v;
  plan->chunks = (int)chunks_of(*v, dtype, hidden);
  plan->lds_bytes = (v->kind == rmsn::kStream && v->lds_stage) ? (size_t)hidden * s : 0;
  return RMSN_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Largest power of two, capped at 16, dividing the address.
int align_of(const void* p) {
  const uintptr_t u = (uintptr_t)p;
  int a = 16;
  while (a > 1 && (u & (uintptr_t)(a - 1))) a /= 2;
  return a;
}

int min_align(int a, const void* p) {
  const int b = align_of(p);
  return a < b ? a : b;
}

int common_checks(int dtype, int64_t rows, int64_t hidden, float eps) {
  if (dtype != RMSN_F32 && dtype != RMSN_F16 && dtype != RMSN_BF16)
    return fail(RMSN_ERR_DTYPE, "unknown dtype %d", dtype);
  if (rows < 0 || hidden < 1 || hidden > RMSN_MAX_HIDDEN)
    return fail(RMSN_ERR_SHAPE, "rows=%lld hidden=%lld out of range", (long long)rows,
                (long long)hidden);
  if (!(eps >= 0.0f) || isinf(eps)) return fail(RMSN_ERR_EPS, "eps=%g must be finite and >= 0", eps);
  return RMSN_OK;
}

int launch(const Plan& plan, rmsn::RowArgs a, void* stream) {
  const rmsn::Variant& v = *plan.v;
  a.chunks = plan.chunks;
  const int64_t rows_per_wg = v.kind == rmsn::kVgpr ? v.wgs / v.tpr : 1;
  int64_t groups = (a.rows + rows_per_wg - 1) / rows_per_wg;
  int64_t cap = kGridCapDefault;
  if (const char* e = getenv("RMSNORM_GRID_CAP")) {
    const long long c = atoll(e);
    if (c > 0) cap = c;
  }
  const unsigned grid = (unsigned)(groups < cap ? groups : cap);
  void* args[] = {&a};
  hipError_t err = hipLaunchKernel(v.fn, dim3(grid), dim3(v.wgs), args, plan.lds_bytes,
                                   (hipStream_t)stream);
  if (err != hipSuccess)
    return fail(RMSN_ERR_HIP, "launch of %s failed: %s", v.name, hipGetErrorString(err));
  return RMSN_OK;
}

}  // namespace

// The last-error slot, shared with the other entry points of the library.
int rmsn_set_error(int code, const char* msg) { return fail(code, "%s", msg); }

extern "C" {

int rmsnorm_fwd(void* out, const void* x, const void* gamma, int64_t rows, int64_t hidden,
                float eps, int dtype, void* stream) {
  int rc = common_checks(dtype, rows, hidden, eps);
  if (rc) return rc;
  if (rows == 0) return RMSN_OK;
  if (!out || !x || !gamma) return fail(RMSN_ERR_NULL, "out, x and gamma must be non-NULL");
  const size_t nbytes = (size_t)rows * (size_t)hidden * dtype_size(dtype);
  const size_t gbytes = (size_t)hidden * dtype_size(dtype);
  if (out != x && overlap(out, nbytes, x, nbytes))
    return fail(RMSN_ERR_ALIAS, "out partially overlaps x");
  if (overlap(out, nbytes, gamma, gbytes)) return fail(RMSN_ERR_ALIAS, "out overlaps gamma");
  Plan plan;
  rc = choose(dtype, hidden, 0, min_align(min_align(align_of(out), x), gamma), &plan);
  if (rc) return rc;
  rmsn::RowArgs a{};
  a.out = out;
  a.residual = nullptr;
  a.partials.p[0] = x;
  a.gamma = gamma;
  a.rows = rows;
  a.hidden = (int)hidden;
  a.k = 1;
  a.eps = eps;
  return launch(plan, a, stream);
}

int add_rmsnorm_fwd(void* out, void* residual, const void* const* partials, int k,
                    const void* gamma, int64_t rows, int64_t hidden, float eps, int dtype,
                    void* stream) {
  int rc = common_checks(dtype, rows, hidden, eps);
  if (rc) return rc;
  if (k < 1 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [1, %d]", k, RMSN_KMAX);
  if (rows == 0) return RMSN_OK;
  if (!out || !residual || !gamma || !partials)
    return fail(RMSN_ERR_NULL, "out, residual, partials and gamma must be non-NULL");
  const size_t nbytes = (size_t)rows * (size_t)hidden * dtype_size(dtype);
  const size_t gbytes = (size_t)hidden * dtype_size(dtype);
  int align = min_align(min_align(align_of(out), residual), gamma);
  for (int j = 0; j < k; ++j) {
    if (!partials[j]) return fail(RMSN_ERR_NULL, "partials[%d] is NULL", j);
    if (overlap(residual, nbytes, partials[j], nbytes))
      return fail(RMSN_ERR_ALIAS, "residual overlaps partials[%d]", j);
    if (out != partials[j] && overlap(out, nbytes, partials[j], nbytes))
      return fail(RMSN_ERR_ALIAS, "out partially overlaps partials[%d]", j);
    align = min_align(align, partials[j]);
  }
  if (overlap(out, nbytes, residual, nbytes)) return fail(RMSN_ERR_ALIAS, "out overlaps residual");
  if (overlap(out, nbytes, gamma, gbytes)) return fail(RMSN_ERR_ALIAS, "out overlaps gamma");
  if (overlap(residual, nbytes, gamma, gbytes))
    return fail(RMSN_ERR_ALIAS, "residual overlaps gamma");
  Plan plan;
  rc = choose(dtype, hidden, k, align, &plan);
  if (rc) return rc;
  rmsn::RowArgs a{};
  a.out = out;
  a.residual = residual;
  for (int j = 0; j < k; ++j) a.partials.p[j] = partials[j];
  a.gamma = gamma;
  a.rows = rows;
  a.hidden = (int)hidden;
  a.k = k;
  a.eps = eps;
  return launch(plan, a, stream);
}

const char* rmsnorm_strerror(int code) {
  switch (code) {
    case RMSN_OK: return "success";
    case RMSN_ERR_NULL: return "a required pointer is NULL";
    case RMSN_ERR_SHAPE: return "rows/hidden out of range or no kernel for the shape";
    case RMSN_ERR_DTYPE: return "unknown dtype";
    case RMSN_ERR_K: return "number of partials outside [1, RMSN_KMAX]";
    case RMSN_ERR_ALIAS: return "forbidden overlap between buffers";
    case RMSN_ERR_EPS: return "eps must be finite and >= 0";
    case RMSN_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown error code";
  }
}

const char* rmsnorm_last_error(void) { return g_last_error; }

int rmsnorm_plan(int64_t rows, int64_t hidden, int k, int dtype, int align, char* buf,
                 int buflen) {
  int rc = common_checks(dtype, rows, hidden, 0.0f);
  if (rc) return rc;
  if (k < 0 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [0, %d]", k, RMSN_KMAX);
  if (!buf || buflen < 1) return fail(RMSN_ERR_NULL, "buf must be non-NULL");
  Plan plan;
  int a = 1;
  while (a < 16 && a * 2 <= align) a *= 2;
  rc = choose(dtype, hidden, k, a, &plan);
  if (rc) return rc;
  snprintf(buf, (size_t)buflen, "%s", plan.v->name);
  return RMSN_OK;
}

int rmsnorm_variants(int dtype, char* buf, int buflen) {
  if (dtype != RMSN_F32 && dtype != RMSN_F16 && dtype != RMSN_BF16)
    return fail(RMSN_ERR_DTYPE, "unknown dtype %d", dtype);
  if (!buf || buflen < 1) return fail(RMSN_ERR_NULL, "buf must be non-NULL");
  int n = 0;
  const rmsn::Variant* t = table_for(dtype, &n);
  size_t used = 0;
  buf[0] = 0;
  for (int i = 0; i < n; ++i) {
    const size_t len = strlen(t[i].name);
    if (used + len + 2 > (size_t)buflen) return fail(RMSN_ERR_SHAPE, "buffer too small");
    memcpy(buf + used, t[i].name, len);
    used += len;
    buf[used++] = '\n';
    buf[used] = 0;
  }
  return n;
}

}  // extern "C"
