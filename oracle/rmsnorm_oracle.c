/*
 * rmsnorm_oracle.c -- plain CPU oracle for row-wise RMSNorm and the fused
 * "K partials + residual -> residual in place -> RMSNorm" form.
 *
 * TEST INFRASTRUCTURE, not product code.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the GPU library; the two are built by
 * different compilers from different sources.
 *
 * The oracle is the definition written out, slowly and in the obvious order:
 *   - RMSNorm: page "RMSNorm kernel", section 1 Background (PyTorch RMSNorm
 *     definition over the last dimension, x as [rows, hidden_dim]) and
 *     section 2 Analytics & Implementation, "Abstraction" (per-row sum of
 *     squares, take the mean, add eps, square root; then x_i*gamma_i/RMS).
 *   - Fused form: page "Tokenweave fused-RMSNorm-AR kernel", section "Code
 *     walkthrough" (per token: reduced partials, + residual, residual stored
 *     back in place, sum of squares of the stored values in fp32, then
 *     rsqrt(variance/hidden + eps) and residual*scale*weight).
 * Readings taken where the pages are silent:
 *   - the partials and the residual are summed in binary32, in the order
 *     p_0, ..., p_{k-1}, r, with the accumulator seeded by p_0 (not by +0.0,
 *     which would turn an all -0.0 sum into +0.0);
 *   - the stored residual is that fp32 sum rounded once to the storage dtype,
 *     and the row that is normalised is the stored (rounded) residual;
 *   - everything after the residual is computed in double and y is rounded
 *     once, to nearest with ties to even, to the output dtype;
 *   - eps enters as the float argument widened to double, added after the
 *     mean and inside the square root; the order is (v * inv) * gamma;
 *   - in the general form (rmsnorm_oracle_ex) gamma may have its own dtype
 *     (read exactly) and y is rounded once to its own output dtype; the rows
 *     are still [..., hidden] with the hidden dimension contiguous, as page
 *     "RMSNorm kernel" section 2 states the input shape.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -fno-fast-math (no FMA
 * contraction, no reassociation, binary32 adds stay binary32 on x86-64 SSE).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "rmsnorm_oracle.h" /* include/, the oracle's own header */

/* ---- storage formats (IEEE 754 binary32, binary16, and bfloat16) ---------
 * p = significand bits including the implicit one; emin = exponent of the
 * smallest normal; emax = exponent of the largest finite; bias as stored.   */
typedef struct {
    int p, emin, emax, bias, mant_bits;
} fmt_t;

static const fmt_t FMT_F32 = {24, -126, 127, 127, 23};
static const fmt_t FMT_F16 = {11, -14, 15, 15, 10};
static const fmt_t FMT_BF16 = {8, -126, 127, 127, 7};

static const fmt_t* fmt_of(int dtype) {
    switch (dtype) {
        case RMSNORM_ORACLE_F32: return &FMT_F32;
        case RMSNORM_ORACLE_F16: return &FMT_F16;
        case RMSNORM_ORACLE_BF16: return &FMT_BF16;
        default: return NULL;
    }
}

/* Round v to the nearest value of format f, ties to even, by the textbook
 * recipe: find v's binade (clamped to the subnormal binade), express v as a
 * multiple of that binade's quantum 2^(e-p+1), round the multiple to the
 * nearest integer (the default FE_TONEAREST mode of nearbyint is
 * ties-to-even), and scale back.  All steps are exact in double except the
 * one rounding.  A result above the largest finite value is an overflow and
 * becomes infinity, as IEEE 754 round-to-nearest prescribes. */
static double round_to(double v, const fmt_t* f) {
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    double a = fabs(v);
    int E;
    (void)frexp(a, &E);            /* a in [2^(E-1), 2^E) */
    int e = E - 1;
    if (e < f->emin) e = f->emin;  /* subnormal: fixed quantum 2^(emin-p+1) */
    int qexp = e - (f->p - 1);
    double n = nearbyint(ldexp(a, -qexp));
    double r = ldexp(n, qexp);
    double maxfin = ldexp(ldexp(1.0, f->p) - 1.0, f->emax - (f->p - 1));
    if (r > maxfin) r = INFINITY;
    return copysign(r, v);
}

/* Bit pattern of a value already representable in a 16-bit format. */
static uint16_t encode16(double r, const fmt_t* f) {
    uint16_t sign = signbit(r) ? 0x8000u : 0u;
    uint16_t exp_all = (uint16_t)(((1u << (15 - f->mant_bits)) - 1u) << f->mant_bits);
    if (isnan(r)) return (uint16_t)(sign | exp_all | (1u << (f->mant_bits - 1)));
    if (isinf(r)) return (uint16_t)(sign | exp_all);
    if (r == 0.0) return sign;
    double a = fabs(r);
    int E;
    (void)frexp(a, &E);
    int e = E - 1;
    if (e < f->emin) { /* subnormal: a = m * 2^(emin - mant_bits) */
        uint32_t m = (uint32_t)ldexp(a, f->mant_bits - f->emin);
        return (uint16_t)(sign | m);
    }
    uint32_t m = (uint32_t)ldexp(a, f->mant_bits - e) - (1u << f->mant_bits);
    return (uint16_t)(sign | ((uint32_t)(e + f->bias) << f->mant_bits) | m);
}

/* Exact value of a 16-bit pattern. */
static double decode16(uint16_t h, const fmt_t* f) {
    int sign = h >> 15;
    int ebits = 15 - f->mant_bits;
    uint32_t e = (h >> f->mant_bits) & ((1u << ebits) - 1u);
    uint32_t m = h & ((1u << f->mant_bits) - 1u);
    double v;
    if (e == (1u << ebits) - 1u)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, f->emin - f->mant_bits);
    else
        v = ldexp((double)((1u << f->mant_bits) + m), (int)e - f->bias - f->mant_bits);
    return sign ? -v : v;
}

static double load(const void* base, int64_t idx, int dtype) {
    if (dtype == RMSNORM_ORACLE_F32) {
        float x;
        memcpy(&x, (const char*)base + idx * 4, 4);
        return (double)x;
    }
    uint16_t h;
    memcpy(&h, (const char*)base + idx * 2, 2);
    return decode16(h, fmt_of(dtype));
}

/* Store a double that is already representable in dtype. */
static void store_exact(void* base, int64_t idx, double r, int dtype) {
    if (dtype == RMSNORM_ORACLE_F32) {
        float x = (float)r; /* exact: r is a binary32 value (or inf/NaN) */
        memcpy((char*)base + idx * 4, &x, 4);
        return;
    }
    uint16_t h = encode16(r, fmt_of(dtype));
    memcpy((char*)base + idx * 2, &h, 2);
}

static void store_rounded(void* base, int64_t idx, double v, int dtype) {
    store_exact(base, idx, round_to(v, fmt_of(dtype)), dtype);
}

int rmsnorm_oracle_round(void* dst, const double* src, int64_t n, int dtype) {
    if (!fmt_of(dtype)) return RMSNORM_ORACLE_ERR_DTYPE;
    if (n < 0) return RMSNORM_ORACLE_ERR_SHAPE;
    if (n > 0 && (!dst || !src)) return RMSNORM_ORACLE_ERR_NULL;
    for (int64_t i = 0; i < n; ++i) store_rounded(dst, i, src[i], dtype);
    return RMSNORM_ORACLE_OK;
}

int rmsnorm_oracle_decode(double* dst, const void* src, int64_t n, int dtype) {
    if (!fmt_of(dtype)) return RMSNORM_ORACLE_ERR_DTYPE;
    if (n < 0) return RMSNORM_ORACLE_ERR_SHAPE;
    if (n > 0 && (!dst || !src)) return RMSNORM_ORACLE_ERR_NULL;
    for (int64_t i = 0; i < n; ++i) dst[i] = load(src, i, dtype);
    return RMSNORM_ORACLE_OK;
}

int rmsnorm_oracle_ex(void* out, int out_dtype, double* y_f64, void* residual,
                      const void* const* partials, int k, int dtype,
                      const void* gamma, int gamma_dtype, int64_t rows, int64_t hidden,
                      float eps, double* rstd_out) {
    if (!fmt_of(dtype) || !fmt_of(out_dtype) || !fmt_of(gamma_dtype))
        return RMSNORM_ORACLE_ERR_DTYPE;
    if (rows < 0 || hidden < 1) return RMSNORM_ORACLE_ERR_SHAPE;
    if (k < 1 || k > RMSNORM_ORACLE_KMAX) return RMSNORM_ORACLE_ERR_K;
    if (!residual && k != 1) return RMSNORM_ORACLE_ERR_K;
    if (!(eps >= 0.0f) || isinf(eps)) return RMSNORM_ORACLE_ERR_EPS;
    if (rows == 0) return RMSNORM_ORACLE_OK;
    if (!partials || !gamma) return RMSNORM_ORACLE_ERR_NULL;
    for (int j = 0; j < k; ++j)
        if (!partials[j]) return RMSNORM_ORACLE_ERR_NULL;

    const fmt_t* f = fmt_of(dtype);
    double* v = (double*)malloc((size_t)hidden * sizeof(double));
    if (!v) return RMSNORM_ORACLE_ERR_NOMEM;

    for (int64_t i = 0; i < rows; ++i) {
        const int64_t base = i * hidden;

        /* Step 1: the row to normalise. */
        for (int64_t j = 0; j < hidden; ++j) {
            if (!residual) {
                v[j] = load(partials[0], base + j, dtype);
                continue;
            }
            /* binary32 sum in the order p_0, ..., p_{k-1}, r; every dtype
             * value converts to float exactly.  The residual keeps the data
             * dtype whatever the output dtype is. */
            float acc = (float)load(partials[0], base + j, dtype);
            for (int q = 1; q < k; ++q) acc = acc + (float)load(partials[q], base + j, dtype);
            acc = acc + (float)load(residual, base + j, dtype);
            double r_new = round_to((double)acc, f);
            store_exact(residual, base + j, r_new, dtype);
            v[j] = r_new;
        }

        /* Step 2: mean of squares, accumulated in double. */
        double ss = 0.0;
        for (int64_t j = 0; j < hidden; ++j) ss += v[j] * v[j];
        double ms = ss / (double)hidden;

        /* Step 3: eps inside the square root, after the mean. */
        double inv = 1.0 / sqrt(ms + (double)eps);
        if (rstd_out) rstd_out[i] = inv;

        /* Step 4: y = (v * inv) * gamma (gamma read exactly in its own
         * dtype), rounded once to the output dtype. */
        for (int64_t j = 0; j < hidden; ++j) {
            double y = (v[j] * inv) * load(gamma, j, gamma_dtype);
            if (y_f64) y_f64[base + j] = y;
            if (out) store_rounded(out, base + j, y, out_dtype);
        }
    }
    free(v);
    return RMSNORM_ORACLE_OK;
}

int rmsnorm_oracle_f64(void* out, double* y_f64, void* residual,
                       const void* const* partials, int k, const void* gamma,
                       int64_t rows, int64_t hidden, float eps, int dtype,
                       double* rstd_out) {
    return rmsnorm_oracle_ex(out, dtype, y_f64, residual, partials, k, dtype, gamma, dtype,
                             rows, hidden, eps, rstd_out);
}

int rmsnorm_oracle(void* out, void* residual, const void* const* partials, int k,
                   const void* gamma, int64_t rows, int64_t hidden, float eps,
                   int dtype, double* rstd_out) {
    if (!out && rows > 0) return RMSNORM_ORACLE_ERR_NULL;
    return rmsnorm_oracle_f64(out, NULL, residual, partials, k, gamma, rows, hidden,
                              eps, dtype, rstd_out);
}
