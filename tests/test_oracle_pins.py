"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's formula: each compares the oracle
with a closed form, an invariant, an exact brute-force computation
(fractions / 60-digit decimal), a library routine (torch's RMSNorm in float64,
numpy's and torch's converters), or a special case.  Each pin is a function of
the oracle build so that ``test_oracle_mutants.py`` can show the battery
rejects plausible mistakes planted in a copy of the oracle.

The method: page "RMSNorm kernel", section 1 Background (RMSNorm over the last
dimension) and section 2 "Abstraction" (sum of squares -> mean -> + eps ->
square root; then x_i * gamma_i / RMS); fused form: page "Tokenweave
fused-RMSNorm-AR kernel", "Code walkthrough" (partials + residual, residual
stored in place, then the stored row is normalised).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import independent as ind

DTYPES = ["f32", "f16", "bf16"]
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_storage_vals(vals: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values that are exactly representable in dtype -> storage."""
    t = torch.from_numpy(np.asarray(vals, dtype=np.float64)).to(torch.float32)
    if dtype == "f32":
        return t.numpy()
    s = t.to(TORCH[dtype])
    assert torch.equal(s.to(torch.float32), t), "value not representable"
    return s.view(torch.int16).numpy().view(np.uint16)


def rand_storage(rng, shape, dtype, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    t = torch.from_numpy(a)
    if dtype == "f32":
        return a
    return t.to(TORCH[dtype]).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# P1: constant row.  x_j = c for all j gives ms = c^2 exactly, so
# y_j = c / sqrt(c^2 + eps) * gamma_j (closed form, 60-digit decimal).

def pin_constant_row(lib=None, dtypes=DTYPES, cs=(1e-4, 0.3, 1.0, 3e3), epss=(1e-6, 1e-5),
                     hs=(1, 7, 1592, 4096)):
    rng = np.random.default_rng(1)
    for dtype in dtypes:
        for c0 in cs:
            for sgn in (1, -1):
                # c rounded to bf16 so that it has <= 8 significant bits in
                # every dtype: H * c^2 is then exact in double.
                c = float(torch.tensor(sgn * c0).to(torch.bfloat16).to(torch.float64))
                for eps in epss:
                    for H in hs:
                        x = to_storage_vals(np.full((2, H), c), dtype)
                        g = rand_storage(rng, (H,), dtype) if dtype == "f32" else \
                            to_storage_vals(np.round(rng.uniform(0.5, 1.5, H) * 64) / 64, dtype)
                        out, rstd, y64 = oracle.rmsnorm(x, g, eps, dtype, want_f64=True, lib=lib)
                        gv = ind.decode_np(g, dtype)
                        cq = Fraction(c)
                        epsq = Fraction(float(np.float32(eps)))
                        inv = 1 / ind.sqrt_dec(cq * cq + epsq)
                        assert ind.isclose_rel(rstd[0], float(inv), 4e-16), (dtype, c, eps, H)
                        for j in range(0, H, max(1, H // 37)):
                            exact = ind.dec(cq) * inv * ind.dec(Fraction(float(gv[j])))
                            assert ind.isclose_rel(y64[0, j], float(exact), 2e-15), (dtype, c, eps, H, j)
                            r, tie = ind.exact_round(Fraction(exact), dtype)
                            want = ind.storage_of(r, dtype)
                            if out[1, j] != want:
                                # only a value sitting on a rounding tie may differ
                                assert tie < Fraction(1, 10 ** 9), (dtype, c, eps, H, j)


# P2: gamma = 1 gives mean_j(y_j^2) = ms / (ms + eps).

def pin_gamma_one_invariant(lib=None, dtypes=DTYPES):
    rng = np.random.default_rng(2)
    for dtype in dtypes:
        for H in (1, 3, 64, 1592, 4096):
            for eps in (1e-6, 1e-2, 0.0):
                x = rand_storage(rng, (4, H), dtype, scale=rng.uniform(0.01, 10))
                g = to_storage_vals(np.ones(H), dtype)
                _, _, y64 = oracle.rmsnorm(x, g, eps, dtype, want_f64=True, lib=lib)
                xv = ind.decode_np(x, dtype)
                for i in range(4):
                    ms = sum(Fraction(float(v)) ** 2 for v in xv[i]) / H
                    want = ms / (ms + Fraction(float(np.float32(eps))))
                    got = float(np.mean(y64[i] ** 2))
                    assert ind.isclose_rel(got, float(want), 1e-13), (dtype, H, eps, i)


# P3: scale.  With eps = 0 and s = 2^k every double step scales exactly, so
# y(s x) is bit-identical to y(x); y(-x) = -y(x); and with eps scaled by s^2,
# y(s x; eps s^2) = y(x; eps) exactly.  As eps -> 0, y(s x) -> y(x).

def pin_scale(lib=None, dtypes=DTYPES):
    rng = np.random.default_rng(3)
    for dtype in dtypes:
        H = 257
        x = rand_storage(rng, (3, H), dtype)
        g = rand_storage(rng, (H,), dtype)
        xv = ind.decode_np(x, dtype)
        _, _, y0 = oracle.rmsnorm(x, g, 0.0, dtype, want_f64=True, lib=lib)
        ks = (-8, 4, 10) if dtype != "f16" else (-4, 3)
        for k in ks:
            xs = to_storage_vals(xv * 2.0 ** k, dtype)
            _, _, ys = oracle.rmsnorm(xs, g, 0.0, dtype, want_f64=True, lib=lib)
            assert np.array_equal(ys, y0), (dtype, k)
            eps = 1e-6 if dtype != "f16" else 1e-4
            e2 = float(np.float32(eps) * np.float32(4.0 ** k))
            assert float(np.float32(e2)) == float(np.float32(eps)) * 4.0 ** k
            _, _, ya = oracle.rmsnorm(x, g, eps, dtype, want_f64=True, lib=lib)
            _, _, yb = oracle.rmsnorm(xs, g, e2, dtype, want_f64=True, lib=lib)
            assert np.array_equal(ya, yb), (dtype, k)
        xn = to_storage_vals(-xv, dtype)
        _, _, yn = oracle.rmsnorm(xn, g, 1e-6, dtype, want_f64=True, lib=lib)
        _, _, yp = oracle.rmsnorm(x, g, 1e-6, dtype, want_f64=True, lib=lib)
        assert np.array_equal(yn, -yp)
        _, _, ye = oracle.rmsnorm(x, g, 1e-9, dtype, want_f64=True, lib=lib)
        assert np.allclose(ye, y0, rtol=1e-8, atol=0)


# P4: brute force on tiny rows, including the residual (exact arithmetic).

def _tiny_values(rng, n, dtype):
    """Finite values of dtype, mixing normals, +-0, subnormals and big values."""
    kind = rng.integers(0, 6, n)
    v = rng.standard_normal(n)
    v = np.where(kind == 1, 0.0, v)
    v = np.where(kind == 2, -0.0, v)
    tiny = {"f32": 1e-40, "f16": 3e-6, "bf16": 1e-39}[dtype]
    big = {"f32": 1e18, "f16": 3e3, "bf16": 1e18}[dtype]
    v = np.where(kind == 3, rng.standard_normal(n) * tiny, v)
    v = np.where(kind == 4, rng.standard_normal(n) * big, v)
    t = torch.from_numpy(v.astype(np.float32))
    if dtype == "f32":
        return t.numpy()
    return t.to(TORCH[dtype]).view(torch.int16).numpy().view(np.uint16)


def pin_brute_force(lib=None, dtypes=DTYPES, trials=12):
    rng = np.random.default_rng(4)
    near_ties = 0
    for dtype in dtypes:
        for trial in range(trials):
            H = int(rng.choice([1, 2, 3, 7, 8, 9]))
            R = int(rng.integers(1, 4))
            K = int(rng.integers(0, 4))  # 0: plain RMSNorm
            eps = float(rng.choice([1e-6, 1e-5, 0.5]))
            g = _tiny_values(rng, H, dtype)
            gv = ind.decode_np(g, dtype)
            if K == 0:
                x = _tiny_values(rng, R * H, dtype).reshape(R, H)
                out, _ = oracle.rmsnorm(x, g, eps, dtype, lib=lib)
                rows_v = ind.decode_np(x, dtype)
            else:
                ps = [_tiny_values(rng, R * H, dtype).reshape(R, H) for _ in range(K)]
                r = _tiny_values(rng, R * H, dtype).reshape(R, H)
                out, rnew, _ = oracle.add_rmsnorm(ps, r, g, eps, dtype, lib=lib)
                pv = [ind.decode_np(p, dtype) for p in ps]
                rv = ind.decode_np(r, dtype)
                rows_v = np.empty((R, H))
                for i in range(R):
                    for j in range(H):
                        acc = ind.fused_residual_f32([pv[q][i, j] for q in range(K)] + [rv[i, j]])
                        want, _ = ind.round_signed(Fraction(float(acc)), float(acc), dtype)
                        assert int(ind.storage_bits(rnew, dtype)[i, j]) == ind.bits(want, dtype), \
                            (dtype, trial, i, j)
                        rows_v[i, j] = want
            for i in range(R):
                bf = ind.brute_force_row(rows_v[i], gv, eps, dtype)
                for j, (want, tie) in enumerate(bf):
                    got = int(ind.storage_bits(out, dtype)[i, j])
                    if got != ind.bits(want, dtype):
                        near_ties += 1
                        assert tie < Fraction(1, 10 ** 9), (dtype, trial, i, j, got, want)
    assert near_ties <= 2


# P5: special cases.

def pin_special_cases(lib=None, dtypes=DTYPES):
    for dtype in dtypes:
        # H = 1: y = x / sqrt(x^2 + eps) * gamma
        for xv, gv, eps in ((3.0, 1.5, 1e-6), (-0.5, 0.75, 0.25), (2.0 ** -10, 1.0, 1e-6)):
            x = to_storage_vals(np.array([[xv]]), dtype)
            g = to_storage_vals(np.array([gv]), dtype)
            _, _, y = oracle.rmsnorm(x, g, eps, dtype, want_f64=True, lib=lib)
            e = Fraction(float(np.float32(eps)))
            want = ind.dec(Fraction(xv)) / ind.sqrt_dec(Fraction(xv) ** 2 + e) * ind.dec(Fraction(gv))
            assert ind.isclose_rel(y[0, 0], float(want), 2e-15)
        # zero row with eps > 0: y = 0 and the fused residual stays zero
        H = 33
        z = to_storage_vals(np.zeros((2, H)), dtype)
        g = to_storage_vals(np.ones(H), dtype)
        out, rnew, rstd = oracle.add_rmsnorm([z], z.copy(), g, 1e-6, dtype, lib=lib)
        assert np.all(ind.decode_np(out, dtype) == 0) and np.all(ind.decode_np(rnew, dtype) == 0)
        assert ind.isclose_rel(rstd[0], 1 / math.sqrt(float(np.float32(1e-6))), 1e-15)
        # all -0.0 partials and residual: the binary32 sum is -0.0
        nz = to_storage_vals(np.full((1, H), -0.0), dtype)
        _, rnew, _ = oracle.add_rmsnorm([nz, nz.copy()], nz.copy(), g, 1e-6, dtype, lib=lib)
        assert np.all(np.signbit(ind.decode_np(rnew, dtype))), dtype
        # one non-zero element e at index j: y_j = e / sqrt(e^2 / H + eps) * gamma_j
        H = 100
        row = np.zeros((1, H))
        row[0, 17] = 6.0
        x = to_storage_vals(row, dtype)
        gs = to_storage_vals(np.linspace(0.5, 1.5, H).round(3) if dtype == "f32" else
                             np.round(np.linspace(0.5, 1.5, H) * 64) / 64, dtype)
        _, _, y = oracle.rmsnorm(x, gs, 1e-5, dtype, want_f64=True, lib=lib)
        gq = Fraction(float(ind.decode_np(gs, dtype)[17]))
        want = 6 / ind.sqrt_dec(Fraction(36, H) + Fraction(float(np.float32(1e-5)))) * ind.dec(gq)
        assert ind.isclose_rel(y[0, 17], float(want), 2e-15)
        assert np.count_nonzero(y) == 1


# P6: torch's RMSNorm (the definition page "RMSNorm kernel" links) in float64.

def pin_torch_rms_norm(lib=None, dtypes=DTYPES):
    rng = np.random.default_rng(6)
    for dtype in dtypes:
        for (R, H, K) in ((5, 1592, 0), (3, 2048, 1), (2, 4096, 3), (2, 9, 8)):
            g = rand_storage(rng, (H,), dtype)
            if K == 0:
                x = rand_storage(rng, (R, H), dtype, 3.0)
                _, _, y = oracle.rmsnorm(x, g, 1e-6, dtype, want_f64=True, lib=lib)
                v = ind.decode_np(x, dtype)
            else:
                ps = [rand_storage(rng, (R, H), dtype) for _ in range(K)]
                r = rand_storage(rng, (R, H), dtype)
                _, rnew, _, y = oracle.add_rmsnorm(ps, r, g, 1e-5, dtype, want_f64=True, lib=lib)
                v = ind.decode_np(rnew, dtype)
            eps = float(np.float32(1e-6 if K == 0 else 1e-5))
            want = torch.nn.functional.rms_norm(torch.from_numpy(v), [H],
                                                torch.from_numpy(ind.decode_np(g, dtype)), eps)
            np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=0)


# P7: residual.  K = 1: the binary32 sum of two dtype values rounded to dtype
# equals the exactly rounded exact sum (checked with fractions); any K: the
# residual equals numpy's binary32 sequential sum rounded by torch.

def pin_residual(lib=None, dtypes=("bf16", "f16"), n=3000):
    rng = np.random.default_rng(7)
    for dtype in dtypes:
        x = rand_storage(rng, (1, n), dtype)
        r = rand_storage(rng, (1, n), dtype, rng.uniform(0.01, 100))
        g = rand_storage(rng, (n,), dtype)
        _, rnew, _ = oracle.add_rmsnorm([x], r, g, 1e-6, dtype, lib=lib)
        xv, rv = ind.decode_np(x, dtype)[0], ind.decode_np(r, dtype)[0]
        for j in range(n):
            want, _ = ind.exact_round(Fraction(float(xv[j])) + Fraction(float(rv[j])), dtype)
            assert ind.decode_np(rnew[:, j:j + 1], dtype)[0, 0] == float(want), (dtype, j)
    for dtype in ("bf16", "f16", "f32"):
        for K in (1, 3, 8):
            ps = [rand_storage(rng, (4, 1000), dtype, 0.35) for _ in range(K)]
            r = rand_storage(rng, (4, 1000), dtype)
            g = rand_storage(rng, (1000,), dtype)
            _, rnew, _ = oracle.add_rmsnorm(ps, r, g, 1e-5, dtype, lib=lib)
            acc = ind.decode_np(ps[0], dtype).astype(np.float32)
            for p in ps[1:]:
                acc = acc + ind.decode_np(p, dtype).astype(np.float32)
            acc = acc + ind.decode_np(r, dtype).astype(np.float32)
            t = torch.from_numpy(acc)
            want = t.numpy() if dtype == "f32" else \
                t.to(TORCH[dtype]).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(rnew.view(np.uint32 if dtype == "f32" else np.uint16),
                                  want.view(np.uint32 if dtype == "f32" else np.uint16)), (dtype, K)


# P8: converters.  float32 -> bf16 against torch; float32 / float64 -> f16
# against numpy; float64 -> f32 against numpy; float64 -> bf16 against exact
# rational rounding; decoders against numpy views (all 65536 patterns).

def _stratified_f32(rng):
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF], dtype=np.uint32)
    a = (hi[:, None] | lows[None, :]).ravel()
    a = np.concatenate([a, rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)])
    f = a.view(np.float32)
    return f[~np.isnan(f)]


def pin_converters(lib=None):
    rng = np.random.default_rng(8)
    f = _stratified_f32(rng)
    got = oracle.round_to(f.astype(np.float64), "bf16", lib=lib)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # f16 from float32: low 13 bits around the rounding position, all binades
    # that reach fp16 (including its subnormals and overflow)
    exps = np.arange(127 - 26, 127 + 17, dtype=np.uint32)
    tops = np.arange(1 << 10, dtype=np.uint32)
    lows = np.array([0, 1, 0x7FF, 0xFFF, 0x1000, 0x1001, 0x17FF, 0x1FFF], dtype=np.uint32)
    a = ((exps[:, None, None] << 23) | (tops[None, :, None] << 13) | lows[None, None, :]).ravel()
    a = np.concatenate([a, a | 0x80000000])
    f16in = a.view(np.float32)
    got = oracle.round_to(f16in.astype(np.float64), "f16", lib=lib)
    assert np.array_equal(got, f16in.astype(np.float16).view(np.uint16))
    # f16 / f32 from float64, including exact ties and their double neighbours
    d = rng.standard_normal(200000) * np.exp2(rng.integers(-30, 18, 200000))
    q = np.exp2(np.floor(np.log2(np.abs(d))) - 10)
    ties16 = (np.floor(d / q) + 0.5) * q
    d16 = np.concatenate([d, ties16, np.nextafter(ties16, 0), np.nextafter(ties16, np.inf)])
    d16 = d16[np.abs(d16) < 1e6]
    assert np.array_equal(oracle.round_to(d16, "f16", lib=lib), d16.astype(np.float16).view(np.uint16))
    q32 = np.exp2(np.floor(np.log2(np.abs(d))) - 23)
    ties32 = (np.floor(d / q32) + 0.5) * q32
    d32 = np.concatenate([d, ties32, np.nextafter(ties32, 0), np.nextafter(ties32, np.inf),
                          np.array([1e-45, 7e-46, 3.4028235677973366e38, 3.5e38])])
    assert np.array_equal(oracle.round_to(d32, "f32", lib=lib).view(np.uint32),
                          d32.astype(np.float32).view(np.uint32))
    # bf16 from float64 near ties: a float32 detour would round twice
    qb = np.exp2(np.floor(np.log2(np.abs(d[:3000]))) - 7)
    tb = (np.floor(d[:3000] / qb) + 0.5) * qb
    db = np.concatenate([tb, np.nextafter(tb, 0), np.nextafter(tb, np.inf), d[:3000]])
    got = oracle.round_to(db, "bf16", lib=lib)
    for j in range(len(db)):
        want, _ = ind.exact_round(Fraction(float(db[j])), "bf16")
        assert ind.decode_np(got[j:j + 1], "bf16")[0] == float(want), (j, db[j])
    # decoders
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dtype in ("bf16", "f16"):
        got = oracle.decode(allbits, dtype, lib=lib)
        want = ind.decode_np(allbits, dtype)
        ok = (got == want) | (np.isnan(got) & np.isnan(want))
        assert ok.all() and np.array_equal(np.signbit(got), np.signbit(want))


# P9: the general form -- gamma and the output each in their own dtype.  A
# constant row against the closed form, with gamma values that need fp32's
# full significand, and the rounded output against exact rational rounding to
# the output dtype; torch's RMSNorm in float64 with the wider gamma; every
# output element against an independent converter (numpy for f32 and f16,
# exact rationals for bf16); the residual, which keeps the data dtype,
# against numpy's binary32 sequential sum rounded by torch.

GENERAL = [(d, g, o) for d in DTYPES for g in sorted({d, "f32"}) for o in DTYPES
           if (g, o) != (d, d)]


def _round_indep(y: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return y.astype(np.float32)
    if dtype == "f16":
        return y.astype(np.float16).view(np.uint16)
    out = np.empty(y.shape, np.uint16)
    for idx, v in np.ndenumerate(y):
        r, _ = ind.exact_round(Fraction(float(v)), "bf16")
        out[idx] = ind.storage_of(math.copysign(float(r), v) if r == 0 else float(r), "bf16")
    return out


def pin_general_dtypes(lib=None, combos=GENERAL):
    rng = np.random.default_rng(9)
    for dtype, gd, od in combos:
        H = 97
        for c0 in (0.3, -3e3):
            c = float(torch.tensor(c0).to(torch.bfloat16).to(torch.float64))
            x = to_storage_vals(np.full((2, H), c), dtype)
            g = rand_storage(rng, (H,), gd)
            out, rstd, y64 = oracle.rmsnorm(x, g, 1e-6, dtype, gamma_dtype=gd, out_dtype=od,
                                            want_f64=True, lib=lib)
            assert out.dtype == (np.float32 if od == "f32" else np.uint16), (dtype, gd, od)
            gv = ind.decode_np(g, gd)
            cq = Fraction(c)
            inv = 1 / ind.sqrt_dec(cq * cq + Fraction(float(np.float32(1e-6))))
            for j in range(H):
                exact = ind.dec(cq) * inv * ind.dec(Fraction(float(gv[j])))
                assert ind.isclose_rel(y64[0, j], float(exact), 2e-15), (dtype, gd, od, c, j)
                r, tie = ind.exact_round(Fraction(exact), od)
                if ind.storage_of(r, od) != out[1, j]:
                    assert tie < Fraction(1, 10 ** 9), (dtype, gd, od, c, j)
        R, H = 3, 300
        ps = [rand_storage(rng, (R, H), dtype) for _ in range(2)]
        r = rand_storage(rng, (R, H), dtype)
        g = rand_storage(rng, (H,), gd)
        out, rnew, _, y = oracle.add_rmsnorm(ps, r, g, 1e-5, dtype, gamma_dtype=gd,
                                             out_dtype=od, want_f64=True, lib=lib)
        want = torch.nn.functional.rms_norm(torch.from_numpy(ind.decode_np(rnew, dtype)), [H],
                                            torch.from_numpy(ind.decode_np(g, gd)),
                                            float(np.float32(1e-5)))
        np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=0)
        assert np.array_equal(ind.storage_bits(out, od), ind.storage_bits(_round_indep(y, od), od)), \
            (dtype, gd, od)
        acc = ind.decode_np(ps[0], dtype).astype(np.float32) + \
            ind.decode_np(ps[1], dtype).astype(np.float32)
        acc = acc + ind.decode_np(r, dtype).astype(np.float32)
        t = torch.from_numpy(acc)
        wr = t.numpy() if dtype == "f32" else \
            t.to(TORCH[dtype]).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ind.storage_bits(rnew, dtype), ind.storage_bits(wr, dtype)), \
            (dtype, gd, od)


PINS = {
    "constant_row": pin_constant_row,
    "gamma_one": pin_gamma_one_invariant,
    "scale": pin_scale,
    "brute_force": pin_brute_force,
    "special_cases": pin_special_cases,
    "torch_rms_norm": pin_torch_rms_norm,
    "residual": pin_residual,
    "converters": pin_converters,
    "general_dtypes": pin_general_dtypes,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    with np.errstate(over="ignore", invalid="ignore"):
        PINS[name]()


def test_oracle_error_codes():
    x = np.zeros((2, 4), np.float32)
    g = np.ones(4, np.float32)
    assert oracle.raw_call(x.copy(), None, [x], g, 2, 4, 1e-6, 0) == 0
    assert oracle.raw_call(x.copy(), None, [x], g, 2, 0, 1e-6, 0) == -2
    assert oracle.raw_call(x.copy(), None, [x], g, -1, 4, 1e-6, 0) == -2
    assert oracle.raw_call(x.copy(), None, [x], g, 2, 4, 1e-6, 7) == -3
    assert oracle.raw_call(x.copy(), None, [x, x], g, 2, 4, 1e-6, 0) == -4
    assert oracle.raw_call(x.copy(), x.copy(), [x] * 17, g, 2, 4, 1e-6, 0) == -4
    assert oracle.raw_call(x.copy(), None, [x], g, 2, 4, -1.0, 0) == -6
    assert oracle.raw_call(x.copy(), None, [x], g, 2, 4, float("nan"), 0) == -6
    assert oracle.raw_call(x.copy(), None, [x], None, 2, 4, 1e-6, 0) == -1
    assert oracle.raw_call(None, None, [x], g, 2, 4, 1e-6, 0) == -1
    assert oracle.raw_call(None, None, [None], None, 0, 4, 1e-6, 0) == 0  # rows == 0: no-op


def test_oracle_aliasing_out_over_input():
    """out may be the very buffer it reads (plain x, or a partial)."""
    rng = np.random.default_rng(9)
    x = rand_storage(rng, (3, 50), "bf16")
    g = rand_storage(rng, (50,), "bf16")
    ref, _ = oracle.rmsnorm(x, g, 1e-6, "bf16")
    lib = oracle._load()
    import ctypes
    buf = x.copy()
    parts = (ctypes.c_void_p * 1)(buf.ctypes.data)
    rc = lib.rmsnorm_oracle(ctypes.c_void_p(buf.ctypes.data), None, parts, 1,
                            ctypes.c_void_p(g.ctypes.data), 3, 50, ctypes.c_float(1e-6), 2,
                            ctypes.cast(None, ctypes.POINTER(ctypes.c_double)))
    assert rc == 0 and np.array_equal(buf, ref)


def test_oracle_nan_propagates():
    x = to_storage_vals(np.array([[1.0, 2.0, 3.0]]), "bf16")
    x[0, 1] = 0x7FC0  # NaN
    g = to_storage_vals(np.ones(3), "bf16")
    out, _ = oracle.rmsnorm(x, g, 1e-6, "bf16")
    assert np.all(np.isnan(ind.decode_np(out, "bf16")))


# ---- property-based: the brute force on rows hypothesis chooses -------------

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=150, deadline=None)
@given(dtype=st.sampled_from(DTYPES),
       vals=st.lists(st.floats(min_value=-1e6, max_value=1e6, allow_nan=False, width=32),
                     min_size=1, max_size=9),
       eps=st.sampled_from([1e-6, 1e-5, 0.25]),
       k=st.integers(min_value=0, max_value=3),
       seed=st.integers(min_value=0, max_value=2 ** 31))
def test_brute_force_property(dtype, vals, eps, k, seed):
    """One row of hypothesis-chosen values (rounded to dtype), plain or with k
    partials derived from it: the oracle equals exact arithmetic, the
    residual bit for bit and y up to a value on a rounding tie."""
    rng = np.random.default_rng(seed)
    H = len(vals)
    with np.errstate(over="ignore"):
        x = np.asarray(vals, dtype=np.float32)
        if dtype == "f16":
            x = np.clip(x, -6e4, 6e4)
        xs = torch.from_numpy(x)
        store = (lambda t: t.numpy()) if dtype == "f32" else \
            (lambda t: t.to(TORCH[dtype]).view(torch.int16).numpy().view(np.uint16))
        g = store(torch.from_numpy(rng.uniform(0.5, 1.5, H).astype(np.float32)))
        row = store(xs).reshape(1, H)
    gv = ind.decode_np(g, dtype)
    if k == 0:
        out, _ = oracle.rmsnorm(row, g, eps, dtype)
        v = ind.decode_np(row, dtype)[0]
    else:
        ps = [store(torch.from_numpy((rng.standard_normal(H) * 0.3).astype(np.float32))).reshape(1, H)
              for _ in range(k)]
        out, rnew, _ = oracle.add_rmsnorm(ps, row, g, eps, dtype)
        pv = [ind.decode_np(p, dtype)[0] for p in ps]
        rv = ind.decode_np(row, dtype)[0]
        v = np.empty(H)
        for j in range(H):
            acc = ind.fused_residual_f32([p[j] for p in pv] + [rv[j]])
            want, _ = ind.round_signed(Fraction(float(acc)), float(acc), dtype)
            assert int(ind.storage_bits(rnew, dtype)[0, j]) == ind.bits(want, dtype)
            v[j] = want
    for j, (want, tie) in enumerate(ind.brute_force_row(v, gv, eps, dtype)):
        if int(ind.storage_bits(out, dtype)[0, j]) != ind.bits(want, dtype):
            assert tie < Fraction(1, 10 ** 9)
