// rmsnorm_api.hip -- the C ABI of librmsnorm.so (include/rmsnorm.h):
// argument validation, aliasing rules, kernel choice, and the launch on the
// caller's stream.  Host code only; the kernels live in kernels_<dtype>.hip
// (single dtype) and kernels_mixed_<dtype>.hip (the general interface).
//
// Argument conventions follow the pages' problem statement: x[rows, hidden]
// with gamma[hidden] of the same dtype, a float eps and an out-of-place
// output (page "RMSNorm kernel", section 2, naive kernel signature), and for
// the fused form an input, a residual updated in place and a weight over
// num_tokens x hidden_size (page "Tokenweave fused-RMSNorm-AR kernel", "Code
// walkthrough").  The *_ex entry points take the same page's [..., hidden_dim]
// reading further: per-tensor row strides, an fp32 gamma and an output dtype
// of its own.  Sizes are validated before any launch, as the torch bindings
// on page "Block All Reduce CUDA代码学习" check dtype and size before
// dispatching.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/rmsnorm.h"
#include "rmsnorm_kernels.hpp"
#include "rmsnorm_span.hpp"
#include "rmsnorm_variants.hpp"

const rmsn::Variant* rmsn_table_f32(int* n);
const rmsn::Variant* rmsn_table_f16(int* n);
const rmsn::Variant* rmsn_table_bf16(int* n);
const rmsn::Variant* rmsn_table_mixed_f32(int* n);
const rmsn::Variant* rmsn_table_mixed_f16(int* n);
const rmsn::Variant* rmsn_table_mixed_bf16(int* n);
const rmsn::Variant* rmsn_table_ag_f32(int* n);
const rmsn::Variant* rmsn_table_ag_f16(int* n);
const rmsn::Variant* rmsn_table_ag_bf16(int* n);

namespace {

using rmsn_host::align_of;
using rmsn_host::align_of_int;
using rmsn_host::overlap;
using rmsn_host::same_span;
using rmsn_host::Span;

thread_local char g_last_error[512] = "";

// Process-wide tuning overrides, set only through rmsnorm_tune (never from
// the environment): a forced variant name and a cap on workgroups per
// launch.  A call reads them once, without a lock; rmsnorm_tune is meant to
// run before the calls it should affect, not concurrently with them.
std::mutex g_tune_mutex;
char g_forced[128] = "";
std::atomic<bool> g_forced_on{false};
std::atomic<int64_t> g_grid_cap{0};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int dtype_size(int dtype) { return dtype == RMSN_F32 ? 4 : 2; }
bool known(int dtype) { return dtype == RMSN_F32 || dtype == RMSN_F16 || dtype == RMSN_BF16; }

// LDS budget for staging one row in the streaming kernel.  64 KiB keeps at
// least two workgroups resident per CU (160 KiB of LDS per CU on gfx950).
constexpr int64_t kLdsStageMax = 64 * 1024;
// Upper bound on workgroups per launch; longer problems loop over rows.
constexpr int64_t kGridCapDefault = 1 << 20;
// Rows up to this many bytes are held in registers.
constexpr int64_t kVgprMaxBytes = 16384;
// LDS-staged rows longer than this many bytes stream in eight 8-byte chunks
// per lane with 256-lane workgroups.
constexpr int64_t kLongRowBytes = 16384;
// With two or more partials, rows of at least this many bytes use the
// streaming kernel (fewer registers per thread than holding K+1 chunk sets).
constexpr int64_t kStreamMinBytesForK = 8192;
// The plain form takes two chunks per thread when the launch, so shaped,
// still has this many threads: twice what the 256 CUs hold at once, so it is
// bandwidth-bound rather than short of threads.
constexpr int64_t kPlainTwoChunkThreads = 1 << 20;

// dtypes of one call: data (partials, residual, x), gamma, output
struct Types {
  int d, g, o;
  bool single() const { return g == d && o == d; }
};

// Alignment (largest power of two, capped at 16) shared by the base and the
// row pitch of every tensor in a role: data, gamma, output.
struct Aligns {
  int in, g, out;
};

// ag: the all-gather variants (single dtype only).
const rmsn::Variant* table_for(Types t, int* n, bool ag = false) {
  if (ag) {
    if (t.single()) {
      switch (t.d) {
        case RMSN_F32: return rmsn_table_ag_f32(n);
        case RMSN_F16: return rmsn_table_ag_f16(n);
        case RMSN_BF16: return rmsn_table_ag_bf16(n);
      }
    }
    *n = 0;
    return nullptr;
  }
  if (t.single()) {
    switch (t.d) {
      case RMSN_F32: return rmsn_table_f32(n);
      case RMSN_F16: return rmsn_table_f16(n);
      case RMSN_BF16: return rmsn_table_bf16(n);
    }
  } else {
    switch (t.d) {
      case RMSN_F32: return rmsn_table_mixed_f32(n);
      case RMSN_F16: return rmsn_table_mixed_f16(n);
      case RMSN_BF16: return rmsn_table_mixed_bf16(n);
    }
  }
  *n = 0;
  return nullptr;
}

bool same_types(const rmsn::Variant& v, Types t) {
  return v.dtype == t.d && v.gdtype == t.g && v.odtype == t.o;
}

// npt: chunks per thread (register kernel) or chunks in flight per step
// (streaming kernel).
const rmsn::Variant* find(Types t, int kind, int vb, int tpr, int npt, int wgs, int kc, int lds,
                          int nt, bool ag) {
  int n = 0;
  const rmsn::Variant* tab = table_for(t, &n, ag);
  for (int i = 0; i < n; ++i) {
    const rmsn::Variant& v = tab[i];
    if (same_types(v, t) && v.kind == kind && v.vb == vb && v.tpr == tpr && v.wgs == wgs &&
        v.kc == kc && v.nt == nt &&
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

// Elements per chunk of a variant with access width vb over data dtype d.
int64_t elems_per_chunk(int vb, int d) { return vb ? vb / dtype_size(d) : 1; }

// Can chunks of vb bytes of data (E elements; E elements of gamma and of the
// output) be used: the row splits into whole chunks, and every tensor's base
// and row pitch are aligned to its own access width (16 bytes, or the chunk
// when it is narrower)?
bool width_ok(int vb, Types t, int64_t hidden, Aligns al) {
  if (vb == 0) return true;
  const int64_t e = elems_per_chunk(vb, t.d);
  if (hidden % e != 0) return false;
  auto need = [&](int dtype) { return (int)std::min<int64_t>(16, e * dtype_size(dtype)); };
  return al.in >= vb && al.g >= need(t.g) && al.out >= need(t.o);
}

// The widest chunk (16, 8 or 4 bytes of data; 0 = element) that fits.
int widest_chunk(Types t, int64_t hidden, Aligns al) {
  for (int vb = 16; vb > dtype_size(t.d); vb /= 2)
    if (width_ok(vb, t, hidden, al)) return vb;
  return 0;
}

int64_t chunks_of(const rmsn::Variant& v, int64_t hidden) {
  return hidden / elems_per_chunk(v.vb, v.dtype);
}

// Can variant v run a call with these sizes, dtypes and alignments?
bool fits(const rmsn::Variant& v, Types t, int64_t hidden, int k, Aligns al) {
  const int s = dtype_size(t.d);
  if (!same_types(v, t)) return false;
  if (!width_ok(v.vb, t, hidden, al)) return false;
  if (v.kind == rmsn::kVgpr) {
    if (v.kc != vgpr_kc(k) && !(v.kc == -1 && k > 0)) return false;
    return chunks_of(v, hidden) <= (int64_t)v.tpr * v.npt;
  }
  if (v.kc != stream_kc(k) && !(v.kc < 0 && k > 0)) return false;
  if (v.lds_stage && hidden * s > kLdsStageMax) return false;
  return true;
}

// The dispatcher.  Register-resident rows up to 16 KiB, packing rows into
// waves when they are short; streaming two-pass kernels above that
// (LDS-staged while the row fits the stage budget), for K >= 2 on rows of
// 8 KiB and more, and whenever 16-byte accesses do not fit the alignment or
// row length.
// The general interface (other gamma or output dtypes) makes the same
// choice among the shapes compiled for it, with runtime-K fused kernels.
// ag: the same choice among the all-gather variants.
int choose(Types t, int64_t rows, int64_t hidden, int k, Aligns al, Plan* plan, bool ag = false) {
  const int s = dtype_size(t.d);
  const int vb = widest_chunk(t, hidden, al);
  const rmsn::Variant* v = nullptr;

  const char* forced = g_forced_on.load(std::memory_order_acquire) ? g_forced : nullptr;
  if (forced) {
    int n = 0;
    const rmsn::Variant* tab = table_for(t, &n, ag);
    for (int i = 0; i < n && !v; ++i)
      if (same_types(tab[i], t) && strcmp(tab[i].name, forced) == 0) v = &tab[i];
    if (!v)
      return fail(RMSN_ERR_SHAPE, "forced variant %s names no variant of these dtypes", forced);
    if (!fits(*v, t, hidden, k, al))
      return fail(RMSN_ERR_SHAPE, "forced variant %s cannot run hidden=%lld k=%d", forced,
                  (long long)hidden, k);
  } else if (vb == 16 && hidden * s <= kVgprMaxBytes &&
             !(k >= 2 && hidden * s >= kStreamMinBytesForK)) {
    // One 16-byte chunk per thread: threads per row = the next power of two
    // >= chunks (several rows per wave below 64 chunks); a 16 KiB row is
    // 1024 chunks, one workgroup's worth.  Large plain launches give each thread two chunks from 128 chunks up,
    // so that a thread has two loads in flight as the fused form's x and
    // residual give it, and twice the rows fit on a CU: measured 9-11%
    // faster on 2-16 KiB bf16 rows (e.g. 8192x4096: 23.9 vs 26.3 us), even
    // on fp32.  Small launches (512 rows) keep one chunk per thread: they
    // need every thread they can get (3.24 vs 3.40 us per graph-replayed
    // launch for 512x2048 fp32).
    const int64_t C = hidden * s / 16;
    int64_t half = 8;
    while (half * 2 < C) half *= 2;
    const int per = (k == 0 && C >= 128 && rows * half >= kPlainTwoChunkThreads) ? 2 : 1;
    int tpr = 8;
    while ((int64_t)tpr * per < C && tpr < 1024) tpr *= 2;
    const int npt = C <= tpr ? 1 : 2;
    const int wgs = tpr < 256 ? 256 : tpr;
    v = find(t, rmsn::kVgpr, 16, tpr, npt, wgs, vgpr_kc(k), 0, 1, ag);
    if (!v && k > 0) v = find(t, rmsn::kVgpr, 16, tpr, npt, wgs, -1, 0, 1, ag);
  } else {
    // Streaming two-pass, LDS-staged while the row fits the stage budget.
    // Fused calls use the runtime-K form, which sums the partials one at a
    // time with few registers (measured faster than holding all K+1 chunk
    // sets in registers at K = 8).  The LDS-staged form moves 8-byte chunks,
    // four per thread, with just enough threads to put the whole row in
    // flight in one step: measured 3% faster than 16-byte chunks at K = 8
    // and 2% on 16384-wide rows.  Rows over 16 KiB take 256-lane
    // workgroups with eight chunks in flight per lane instead (several
    // steps per row): 2-10% faster from 10240- to 32768-wide bf16 rows and
    // on 8192-wide fp32 ones (65536x16384 bf16: 1439 vs 1499 us).
    const bool lds = hidden * s <= kLdsStageMax;
    const int svb = (lds && vb == 16) ? 8 : vb;
    const int64_t C = hidden / elems_per_chunk(svb, t.d);
    const bool long_row = lds && svb == 8 && hidden * s > kLongRowBytes;
    const int unr = long_row ? 8 : svb == 16 ? 2 : 4;
    int wgs = 256;
    while (!long_row && wgs < 1024 && (int64_t)wgs * unr < C) wgs *= 2;
    // K = 8 sums the partials two per step: measured 1.3% faster at K = 8
    // (4096x8192 bf16: 114.6 vs 116.1 us; 8192x16384: 477 vs 483 us), and
    // 1-2% slower at K = 2, 3, 4 and 16, which keep one per step.
    const int kc = k == 0 ? 0 : k == 8 ? -2 : -1;
    v = find(t, rmsn::kStream, svb, wgs, unr, wgs, kc, lds ? 1 : 0, lds ? 1 : 0, ag);
    if (!v && kc == -2)
      v = find(t, rmsn::kStream, svb, wgs, unr, wgs, -1, lds ? 1 : 0, lds ? 1 : 0, ag);
  }
  if (!v) return fail(RMSN_ERR_SHAPE, "no kernel variant for hidden=%lld k=%d", (long long)hidden, k);
  plan->v = v;
  plan->chunks = (int)chunks_of(*v, hidden);
  plan->lds_bytes = (v->kind == rmsn::kStream && v->lds_stage) ? (size_t)hidden * s : 0;
  return RMSN_OK;
}

int common_checks(int dtype, int64_t rows, int64_t hidden, float eps) {
  if (!known(dtype)) return fail(RMSN_ERR_DTYPE, "unknown dtype %d", dtype);
  if (rows < 0 || hidden < 1 || hidden > RMSN_MAX_HIDDEN)
    return fail(RMSN_ERR_SHAPE, "rows=%lld hidden=%lld out of range", (long long)rows,
                (long long)hidden);
  if (!(eps >= 0.0f) || isinf(eps)) return fail(RMSN_ERR_EPS, "eps=%g must be finite and >= 0", eps);
  return RMSN_OK;
}

int type_checks(Types t) {
  if (!known(t.d) || !known(t.o)) return fail(RMSN_ERR_DTYPE, "unknown dtype %d / %d", t.d, t.o);
  if (t.g != t.d && t.g != RMSN_F32)
    return fail(RMSN_ERR_DTYPE, "gamma dtype %d must be the data dtype %d or RMSN_F32", t.g, t.d);
  return RMSN_OK;
}

// Row stride (elements) of a tensor: at least hidden when rows > 1, and the
// last row's end must be addressable.
int stride_check(const char* what, int64_t stride, int64_t rows, int64_t hidden, int size) {
  if (rows <= 1) return RMSN_OK;
  if (stride < hidden)
    return fail(RMSN_ERR_SHAPE, "%s row stride %lld < hidden %lld", what, (long long)stride,
                (long long)hidden);
  if (stride > (INT64_MAX / size - hidden) / (rows - 1))
    return fail(RMSN_ERR_SHAPE, "%s row stride %lld overflows the address range", what,
                (long long)stride);
  return RMSN_OK;
}

template <typename Args>
int launch(const Plan& plan, Args a, void* stream) {
  const rmsn::Variant& v = *plan.v;
  a.chunks = plan.chunks;
  const int64_t rows_per_wg = v.kind == rmsn::kVgpr ? v.wgs / v.tpr : 1;
  int64_t groups = (a.rows + rows_per_wg - 1) / rows_per_wg;
  const int64_t tuned = g_grid_cap.load(std::memory_order_relaxed);
  const int64_t cap = tuned > 0 ? tuned : kGridCapDefault;
  const unsigned grid = (unsigned)(groups < cap ? groups : cap);
  void* args[] = {&a};
  hipError_t err = hipLaunchKernel(v.fn, dim3(grid), dim3(v.wgs), args, plan.lds_bytes,
                                   (hipStream_t)stream);
  if (err != hipSuccess)
    return fail(RMSN_ERR_HIP, "launch of %s failed: %s", v.name, hipGetErrorString(err));
  return RMSN_OK;
}

// Both forms, every dtype combination and stride: validate, choose, launch.
// residual == nullptr is plain RMSNorm (k == 1, partials[0] is x).  Strides
// are in elements of each tensor's own dtype.  With dry != nullptr nothing is
// launched: *dry receives the chosen variant (nullptr when rows == 0).
// gather (fused, single dtype only): ngather buffers that each receive the
// output rows instead of out (the all-gather epilogue); out is then unused.
int run(Types t, void* out, int64_t out_stride, void* residual, int64_t res_stride,
        const void* const* partials, const int64_t* part_strides, int k, const void* gamma,
        int64_t rows, int64_t hidden, float eps, void* stream,
        const rmsn::Variant** dry = nullptr, void* const* gather = nullptr, int ngather = 0) {
  if (dry) *dry = nullptr;
  int rc = common_checks(t.d, rows, hidden, eps);
  if (rc) return rc;
  if ((rc = type_checks(t))) return rc;
  const bool fused = residual != nullptr;
  if (k < 1 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [1, %d]", k, RMSN_KMAX);
  if (rows == 0) return RMSN_OK;
  if (!out || !gamma || !partials) return fail(RMSN_ERR_NULL, "out, inputs and gamma must be non-NULL");
  const int sd = dtype_size(t.d), so = dtype_size(t.o), sg = dtype_size(t.g);
  if ((rc = stride_check("out", out_stride, rows, hidden, so))) return rc;
  if (fused && (rc = stride_check("residual", res_stride, rows, hidden, sd))) return rc;
  // a single row has no stride: whatever was passed is never used
  if (rows == 1) out_stride = res_stride = hidden;
  const Span o{out, out_stride * so, hidden * so, rows};
  const Span g{gamma, hidden * sg, hidden * sg, 1};
  const Span r{residual, res_stride * sd, hidden * sd, rows};
  Aligns al{16, align_of(gamma), o.align()};
  if (fused) al.in = r.align();
  rmsn::RowArgs a{};
  for (int j = 0; j < k; ++j) {
    char nm[32] = "x";
    if (fused) snprintf(nm, sizeof(nm), "partials[%d]", j);
    if (!partials[j]) return fail(RMSN_ERR_NULL, "%s is NULL", nm);
    const int64_t st = part_strides && rows > 1 ? part_strides[j] : hidden;
    if ((rc = stride_check(nm, st, rows, hidden, sd))) return rc;
    const Span p{partials[j], st * sd, hidden * sd, rows};
    if (fused && overlap(r, p)) return fail(RMSN_ERR_ALIAS, "residual overlaps %s", nm);
    // out may be exactly an input (in place) when it has the input's dtype
    // and layout; any other overlap would let one thread's store reach
    // elements another thread has not read yet.
    if (overlap(o, p) && !(t.o == t.d && same_span(o, p)))
      return fail(RMSN_ERR_ALIAS, "out partially overlaps %s", nm);
    al.in = std::min(al.in, p.align());
    a.partials.p[j] = partials[j];
    a.partials.s[j] = p.pitch;
  }
  if (fused && overlap(o, r)) return fail(RMSN_ERR_ALIAS, "out overlaps residual");
  if (overlap(o, g)) return fail(RMSN_ERR_ALIAS, "out overlaps gamma");
  if (fused && overlap(r, g)) return fail(RMSN_ERR_ALIAS, "residual overlaps gamma");
  rmsn::GatherPtrs gp{};
  if (gather) {
    // out is gather[0]; every gather buffer is checked like out, and none
    // may touch an input, gamma, the residual or another gather buffer, not
    // even exactly: the buffers stand for distinct ranks' gather buffers, so
    // the in-place exception of the single-output form is not carried over.
    gp.n = ngather;
    for (int j = 0; j < ngather; ++j) {
      const Span oj{gather[j], o.pitch, o.len, rows};
      for (int q = 0; q < k; ++q)
        if (overlap(oj, Span{partials[q], a.partials.s[q], hidden * sd, rows}))
          return fail(RMSN_ERR_ALIAS, "gather[%d] overlaps partials[%d]", j, q);
      if (overlap(oj, r)) return fail(RMSN_ERR_ALIAS, "gather[%d] overlaps residual", j);
      if (overlap(oj, g)) return fail(RMSN_ERR_ALIAS, "gather[%d] overlaps gamma", j);
      for (int q = 0; q < j; ++q)
        if (overlap(oj, Span{gather[q], o.pitch, o.len, rows}))
          return fail(RMSN_ERR_ALIAS, "gather[%d] overlaps gather[%d]", j, q);
      al.out = std::min(al.out, oj.align());
      gp.p[j] = gather[j];
    }
  }
  Plan plan;
  rc = choose(t, rows, hidden, fused ? k : 0, al, &plan, gather != nullptr);
  if (rc) return rc;
  if (dry) {
    *dry = plan.v;
    return RMSN_OK;
  }
  a.out = out;
  a.out_stride = o.pitch;
  a.residual = residual;
  a.res_stride = fused ? r.pitch : 0;
  a.gamma = gamma;
  a.rows = rows;
  a.hidden = (int)hidden;
  a.k = k;
  a.eps = eps;
  if (gather) {
    rmsn::RowArgsAG ag{};
    static_cast<rmsn::RowArgs&>(ag) = a;
    ag.gather = gp;
    return launch(plan, ag, stream);
  }
  return launch(plan, a, stream);
}

int list_variants(Types t, char* buf, int buflen, bool ag = false) {
  if (!buf || buflen < 1) return fail(RMSN_ERR_NULL, "buf must be non-NULL");
  int n = 0, count = 0;
  const rmsn::Variant* tab = table_for(t, &n, ag);
  size_t used = 0;
  buf[0] = 0;
  for (int i = 0; i < n; ++i) {
    if (!same_types(tab[i], t)) continue;
    const size_t len = strlen(tab[i].name);
    if (used + len + 2 > (size_t)buflen) return fail(RMSN_ERR_SHAPE, "buffer too small");
    memcpy(buf + used, tab[i].name, len);
    used += len;
    buf[used++] = '\n';
    buf[used] = 0;
    ++count;
  }
  return count;
}

int plan_name(Types t, int64_t rows, int64_t hidden, int k, int align, char* buf, int buflen,
              bool ag = false) {
  int rc = common_checks(t.d, rows, hidden, 0.0f);
  if (rc) return rc;
  if ((rc = type_checks(t))) return rc;
  if (k < 0 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [0, %d]", k, RMSN_KMAX);
  if (!buf || buflen < 1) return fail(RMSN_ERR_NULL, "buf must be non-NULL");
  Plan plan;
  int a = 1;
  while (a < 16 && a * 2 <= align) a *= 2;
  // contiguous rows: each tensor's pitch is hidden elements of its dtype
  const Aligns al{std::min(a, align_of_int((uint64_t)hidden * dtype_size(t.d))),
                  a, std::min(a, align_of_int((uint64_t)hidden * dtype_size(t.o)))};
  rc = choose(t, rows, hidden, k, rows > 1 ? al : Aligns{a, a, a}, &plan, ag);
  if (rc) return rc;
  snprintf(buf, (size_t)buflen, "%s", plan.v->name);
  return RMSN_OK;
}

}  // namespace

// The last-error slot, shared with the other entry points of the library.
int rmsn_set_error(int code, const char* msg) { return fail(code, "%s", msg); }

extern "C" {

int rmsnorm_fwd(void* out, const void* x, const void* gamma, int64_t rows, int64_t hidden,
                float eps, int dtype, void* stream) {
  const void* parts[1] = {x};
  return run(Types{dtype, dtype, dtype}, out, hidden, nullptr, 0, parts, nullptr, 1, gamma, rows,
             hidden, eps, stream);
}

int add_rmsnorm_fwd(void* out, void* residual, const void* const* partials, int k,
                    const void* gamma, int64_t rows, int64_t hidden, float eps, int dtype,
                    void* stream) {
  if (!residual) {
    int rc = common_checks(dtype, rows, hidden, eps);
    if (rc) return rc;
    if (k < 1 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [1, %d]", k, RMSN_KMAX);
    if (rows == 0) return RMSN_OK;
    return fail(RMSN_ERR_NULL, "residual must be non-NULL");
  }
  return run(Types{dtype, dtype, dtype}, out, hidden, residual, hidden, partials, nullptr, k,
             gamma, rows, hidden, eps, stream);
}

int add_rmsnorm_ag_fwd(void* const* outs, int nout, void* residual, const void* const* partials,
                       int k, const void* gamma, int64_t rows, int64_t hidden, float eps,
                       int dtype, void* stream) {
  int rc = common_checks(dtype, rows, hidden, eps);
  if (rc) return rc;
  if (k < 1 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [1, %d]", k, RMSN_KMAX);
  if (nout < 1 || nout > RMSN_GATHER_MAX)
    return fail(RMSN_ERR_SHAPE, "nout=%d outside [1, %d]", nout, RMSN_GATHER_MAX);
  if (rows == 0) return RMSN_OK;
  if (!outs) return fail(RMSN_ERR_NULL, "outs must be non-NULL");
  for (int j = 0; j < nout; ++j)
    if (!outs[j]) return fail(RMSN_ERR_NULL, "outs[%d] is NULL", j);
  if (!residual) return fail(RMSN_ERR_NULL, "residual must be non-NULL");
  return run(Types{dtype, dtype, dtype}, outs[0], hidden, residual, hidden, partials, nullptr, k,
             gamma, rows, hidden, eps, stream, nullptr, outs, nout);
}

int rmsnorm_fwd_ex(void* out, int64_t out_stride, int out_dtype, const void* x, int64_t x_stride,
                   int dtype, const void* gamma, int gamma_dtype, int64_t rows, int64_t hidden,
                   float eps, void* stream) {
  const void* parts[1] = {x};
  const int64_t strides[1] = {x_stride};
  return run(Types{dtype, gamma_dtype, out_dtype}, out, out_stride, nullptr, 0, parts, strides, 1,
             gamma, rows, hidden, eps, stream);
}

int add_rmsnorm_fwd_ex(void* out, int64_t out_stride, int out_dtype, void* residual,
                       int64_t residual_stride, const void* const* partials,
                       const int64_t* partial_strides, int k, int dtype, const void* gamma,
                       int gamma_dtype, int64_t rows, int64_t hidden, float eps, void* stream) {
  if (!residual) {
    int rc = common_checks(dtype, rows, hidden, eps);
    if (rc) return rc;
    if ((rc = type_checks(Types{dtype, gamma_dtype, out_dtype}))) return rc;
    if (k < 1 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [1, %d]", k, RMSN_KMAX);
    if (rows == 0) return RMSN_OK;
    return fail(RMSN_ERR_NULL, "residual must be non-NULL");
  }
  return run(Types{dtype, gamma_dtype, out_dtype}, out, out_stride, residual, residual_stride,
             partials, partial_strides, k, gamma, rows, hidden, eps, stream);
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

int rmsnorm_tune(const char* variant, int64_t grid_cap) {
  if (variant && strlen(variant) >= sizeof(g_forced))
    return fail(RMSN_ERR_SHAPE, "variant name longer than %d bytes", (int)sizeof(g_forced) - 1);
  std::lock_guard<std::mutex> lock(g_tune_mutex);
  g_forced_on.store(false, std::memory_order_release);
  if (variant && *variant) {
    snprintf(g_forced, sizeof(g_forced), "%s", variant);
    g_forced_on.store(true, std::memory_order_release);
  }
  g_grid_cap.store(grid_cap > 0 ? grid_cap : 0, std::memory_order_relaxed);
  return RMSN_OK;
}

int rmsnorm_plan(int64_t rows, int64_t hidden, int k, int dtype, int align, char* buf,
                 int buflen) {
  return plan_name(Types{dtype, dtype, dtype}, rows, hidden, k, align, buf, buflen);
}

int rmsnorm_plan_ag(int64_t rows, int64_t hidden, int k, int dtype, int align, char* buf,
                    int buflen) {
  if (k < 1 || k > RMSN_KMAX) return fail(RMSN_ERR_K, "k=%d outside [1, %d]", k, RMSN_KMAX);
  return plan_name(Types{dtype, dtype, dtype}, rows, hidden, k, align, buf, buflen, true);
}

int rmsnorm_plan_ex(int64_t rows, int64_t hidden, int k, int dtype, int gamma_dtype,
                    int out_dtype, int align, char* buf, int buflen) {
  return plan_name(Types{dtype, gamma_dtype, out_dtype}, rows, hidden, k, align, buf, buflen);
}

int rmsnorm_plan_call(void* out, int64_t out_stride, int out_dtype, void* residual,
                      int64_t residual_stride, const void* const* partials,
                      const int64_t* partial_strides, int k, int dtype, const void* gamma,
                      int gamma_dtype, int64_t rows, int64_t hidden, float eps, char* buf,
                      int buflen) {
  if (!buf || buflen < 1) return fail(RMSN_ERR_NULL, "buf must be non-NULL");
  buf[0] = 0;
  const rmsn::Variant* v = nullptr;
  const int rc = run(Types{dtype, gamma_dtype, out_dtype}, out, out_stride, residual,
                     residual_stride, partials, partial_strides, k, gamma, rows, hidden, eps,
                     nullptr, &v);
  if (rc) return rc;
  snprintf(buf, (size_t)buflen, "%s", v ? v->name : "none");
  return RMSN_OK;
}

int rmsnorm_variants(int dtype, char* buf, int buflen) {
  if (!known(dtype)) return fail(RMSN_ERR_DTYPE, "unknown dtype %d", dtype);
  return list_variants(Types{dtype, dtype, dtype}, buf, buflen);
}

int rmsnorm_variants_ag(int dtype, char* buf, int buflen) {
  if (!known(dtype)) return fail(RMSN_ERR_DTYPE, "unknown dtype %d", dtype);
  return list_variants(Types{dtype, dtype, dtype}, buf, buflen, true);
}

int rmsnorm_variants_ex(int dtype, int gamma_dtype, int out_dtype, char* buf, int buflen) {
  const Types t{dtype, gamma_dtype, out_dtype};
  const int rc = type_checks(t);
  if (rc) return rc;
  return list_variants(t, buf, buflen);
}

}  // extern "C"
