"""Pins of the GEMM + reduce-scatter epilogue oracle (page "LLM System:
通信计算融合算子实现 01 - sm80GEMM + ReduceScatter": the product of the FFN's
second GEMM, scaled by alpha plus beta times C in the epilogue, stored in one
chunk per rank).

The oracle is checked against: exact rational arithmetic (``Fraction``) on
tiny products, rounded by the independent converter of ``tests/independent``;
closed forms (constant operands, an identity weight, alpha = 0); a worked 2x2
example that tells A B^T from A B; numpy's float64 matmul within the double
accumulation bound; the invariance of the values under the chunk split and
the row range; IEEE special values; and its argument checks.  Planted
mistakes in a copy of the oracle are caught.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import independent as ind

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gemm_scatter_oracle.c")
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def store(a, dtype: str) -> np.ndarray:
    """float values -> uint16 storage (round to nearest even, by torch)."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).to(TORCH[dtype])
    return t.view(torch.int16).numpy().view(np.uint16)


def value_grid(rng, shape, dtype: str) -> np.ndarray:
    """Storage of values with a spread of exponents and signs, some zeros of
    either sign, all exactly representable."""
    mag = rng.uniform(1.0, 2.0, shape) * np.exp2(rng.integers(-6, 7, shape))
    v = np.where(rng.random(shape) < 0.5, -mag, mag)
    v = np.where(rng.random(shape) < 0.08, 0.0, v)
    v = np.where(rng.random(shape) < 0.04, -0.0, v)
    return store(v, dtype)


def exact_product(a, b, c, alpha, beta, dtype):
    """Fraction-exact alpha * a @ b.T + beta * c and the error scale."""
    av, bv = ind.decode_np(a, dtype), ind.decode_np(b, dtype)
    cv = ind.decode_np(c, dtype) if c is not None else None
    m, k = a.shape
    n = b.shape[0]
    fa, fb = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    out, mags = [], []
    for i in range(m):
        row, mrow = [], []
        for j in range(n):
            terms = [Fraction(float(av[i, p])) * Fraction(float(bv[j, p])) for p in range(k)]
            q = fa * sum(terms, Fraction(0))
            mg = abs(fa) * sum((abs(t) for t in terms), Fraction(0))
            if cv is not None:
                q += fb * Fraction(float(cv[i, j]))
                mg += abs(fb * Fraction(float(cv[i, j])))
            row.append(q)
            mrow.append(mg)
        out.append(row)
        mags.append(mrow)
    return out, mags


def assemble(chunks) -> np.ndarray:
    return np.concatenate(chunks, axis=0)


# ---- pins -------------------------------------------------------------------

def pin_brute_force(lib=None):
    """Every element of tiny products against exact rationals: the unrounded
    double within (k + 2) * 2^-53 of its scale, the stored value equal to the
    exact value rounded (one ulp allowed only next to a rounding boundary)."""
    rng = np.random.default_rng(11)
    for dtype in ("bf16", "f16"):
        for (m, n, k, world, with_c) in ((2, 3, 5, 1, False), (4, 2, 7, 2, True),
                                         (6, 5, 3, 3, True), (3, 4, 1, 3, False),
                                         (2, 2, 0, 2, True), (4, 3, 9, 4, True)):
            a = value_grid(rng, (m, k), dtype)
            b = value_grid(rng, (n, k), dtype)
            c = value_grid(rng, (m, n), dtype) if with_c else None
            alpha = float(np.float32(rng.choice([1.0, -0.75, 0.3, 2.5])))
            beta = float(np.float32(rng.choice([1.0, 0.5, -1.25])))
            chunks, y, _ = oracle.gemm_scatter(a, b, c, alpha, beta, world, dtype,
                                               want_f64=True, lib=lib)
            got = assemble(chunks)
            exact, mags = exact_product(a, b, c, alpha, beta, dtype)
            for i in range(m):
                for j in range(n):
                    q, mg = exact[i][j], mags[i][j]
                    bound = (k + 2) * Fraction(1, 2 ** 53) * mg
                    assert abs(Fraction(float(y[i, j])) - q) <= bound, (dtype, m, n, k, i, j)
                    r, tie = ind.exact_round(q, dtype)
                    want = int(ind.storage_of(float(r), dtype)) if r != 0 else None
                    g = int(got[i, j])
                    if want is None:
                        assert g & 0x7FFF == 0, (dtype, i, j, hex(g))
                        continue
                    if g != want:
                        near = tie * Fraction(2) ** -60 <= bound or tie == 0
                        d = ind.ulp_distance(np.array([g], np.uint16), np.array([want], np.uint16),
                                             dtype)[0]
                        assert near and d <= 1, (dtype, m, n, k, i, j, hex(g), hex(want))


def pin_closed_forms(lib=None):
    rng = np.random.default_rng(5)
    for dtype in ("bf16", "f16"):
        # constant operands: every element is k * v * alpha
        a = store(np.ones((4, 100)), dtype)
        b = store(np.full((6, 100), 0.375), dtype)
        got = assemble(oracle.gemm_scatter(a, b, None, 1.0, 0.0, 2, dtype, lib=lib))
        assert np.all(got == store(np.full((4, 6), 37.5), dtype))
        got = assemble(oracle.gemm_scatter(a, b, None, -0.5, 0.0, 4, dtype, lib=lib))
        assert np.all(got == store(np.full((4, 6), -18.75), dtype))
        # identity weight: D = A exactly
        k = 24
        a = value_grid(rng, (6, k), dtype)
        eye = store(np.eye(k), dtype)
        got = assemble(oracle.gemm_scatter(a, eye, None, 1.0, 0.0, 3, dtype, lib=lib))
        assert np.array_equal(got & 0x7FFF, a & 0x7FFF) and \
            np.array_equal(got[(a & 0x7FFF) != 0], a[(a & 0x7FFF) != 0])
        # alpha = 0, beta = 1: D = C exactly
        c = value_grid(rng, (6, 5), dtype)
        b = value_grid(rng, (5, k), dtype)
        got = assemble(oracle.gemm_scatter(a, b, c, 0.0, 1.0, 2, dtype, lib=lib))
        nz = (c & 0x7FFF) != 0
        assert np.array_equal(got[nz], c[nz]) and np.all(got[~nz] & 0x7FFF == 0)
        # rounded once from the exact value: 1 + half an ulp + a little rounds
        # up (through binary32 first it would land on the tie and round down)
        tiny = 2.0 ** -30 if dtype == "bf16" else 2.0 ** -24
        half = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
        a1 = store([[1.0, half, tiny]], dtype)
        b1 = store([[1.0, 1.0, 1.0]], dtype)
        got = oracle.gemm_scatter(a1, b1, None, 1.0, 0.0, 1, dtype, lib=lib)[0]
        assert got[0, 0] == store([1.0 + 2 * half], dtype)[0]
        # beta scales C; with A = 0 only beta * C remains
        z = store(np.zeros((6, k)), dtype)
        got = assemble(oracle.gemm_scatter(z, b, c, 1.0, 2.0, 1, dtype, lib=lib))
        assert np.array_equal(got[nz], store(2.0 * ind.decode_np(c, dtype), dtype)[nz])


def pin_worked_example(lib=None):
    """A = [[1,2],[3,4]], B (rows are the weight's output rows) = [[5,6],[7,8]]:
    A B^T = [[17,23],[39,53]] (A B would give [[19,22],[43,50]]).  With C =
    [[1,1],[1,1]], alpha = 2, beta = -1: [[33,45],[77,105]].  Chunk 0 holds
    row 0 and chunk 1 row 1."""
    for dtype in ("bf16", "f16"):
        a = store([[1, 2], [3, 4]], dtype)
        b = store([[5, 6], [7, 8]], dtype)
        c = store([[1, 1], [1, 1]], dtype)
        ch = oracle.gemm_scatter(a, b, None, 1.0, 0.0, 2, dtype, lib=lib)
        assert np.array_equal(ch[0], store([[17, 23]], dtype))
        assert np.array_equal(ch[1], store([[39, 53]], dtype))
        ch = oracle.gemm_scatter(a, b, c, 2.0, -1.0, 1, dtype, lib=lib)
        assert np.array_equal(ch[0], store([[33, 45], [77, 105]], dtype))


def pin_numpy_matmul(lib=None):
    """Medium random products against numpy's float64 matmul (a different
    summation order) within the double bound, with strided operands."""
    rng = np.random.default_rng(9)
    for dtype in ("bf16", "f16"):
        m, n, k = 48, 40, 200
        a_full = store(rng.standard_normal((m, k + 8)), dtype)
        a = a_full[:, 3:3 + k]                     # row stride k + 8
        b = store(rng.standard_normal((n, k)), dtype)
        c = store(rng.standard_normal((m, n)), dtype)
        alpha, beta = 0.8125, -0.5
        _, y, mag = oracle.gemm_scatter(a, b, c, alpha, beta, 4, dtype, want_f64=True, lib=lib)
        av, bv, cv = (ind.decode_np(np.ascontiguousarray(x), dtype) for x in (a, b, c))
        ref = alpha * (av @ bv.T) + beta * cv
        assert np.all(np.abs(y - ref) <= (k + 4) * 2.0 ** -52 * mag + 1e-300)
        # the stored values are y rounded to nearest even (torch rounds the
        # float64 values through float32: compare where that cannot matter)
        got = assemble(oracle.gemm_scatter(a, b, c, alpha, beta, 4, dtype, lib=lib))
        via_torch = torch.from_numpy(ref).to(TORCH[dtype]).view(torch.int16).numpy() \
            .view(np.uint16)
        d = ind.ulp_distance(got, via_torch, dtype)
        assert d.max() <= 1 and (d == 0).mean() > 0.99


def pin_chunks_and_rows(lib=None):
    """The values do not depend on the chunk split or on the row range."""
    rng = np.random.default_rng(3)
    dtype = "bf16"
    m, n, k = 24, 10, 33
    a = value_grid(rng, (m, k), dtype)
    b = value_grid(rng, (n, k), dtype)
    c = value_grid(rng, (m, n), dtype)
    ref = assemble(oracle.gemm_scatter(a, b, c, 1.5, 0.25, 1, dtype, lib=lib))
    for world in (2, 3, 4, 6, 8, 12):
        ch = oracle.gemm_scatter(a, b, c, 1.5, 0.25, world, dtype, lib=lib)
        assert len(ch) == world and all(x.shape == (m // world, n) for x in ch)
        assert np.array_equal(assemble(ch), ref), world
    for r0, r1 in ((0, 5), (5, 13), (13, 24), (7, 7)):
        ch = oracle.gemm_scatter(a, b, c, 1.5, 0.25, 4, dtype, rows=(r0, r1), lib=lib)
        got = assemble(ch)
        assert np.array_equal(got[r0:r1], ref[r0:r1])
        assert not got[:r0].any() and not got[r1:].any()
        rows_only = oracle.gemm_scatter(a, b, c, 1.5, 0.25, 4, dtype, rows=(r0, r1),
                                        scatter=False, lib=lib)
        assert np.array_equal(rows_only, ref[r0:r1])


def pin_specials(lib=None):
    """IEEE: inf times a positive weight is inf, times zero is NaN, opposite
    infinities give NaN; a NaN in C makes that element NaN; overflow of the
    rounded value gives inf."""
    for dtype in ("bf16", "f16"):
        inf, nan = float("inf"), float("nan")
        a = store([[inf, 1.0, 1.0], [1.0, 2.0, 3.0]], dtype)
        b = store([[1.0, 1.0, 1.0], [0.0, 1.0, 1.0], [-1.0, 0.5, 0.5], [1.0, 0.0, 0.0]], dtype)
        c = store([[0.0, 0.0, 0.0, 0.0], [0.0, nan, 0.0, 0.0]], dtype)
        _, y, _ = oracle.gemm_scatter(a, b, c, 1.0, 1.0, 2, dtype, want_f64=True, lib=lib)
        assert y[0, 0] == inf and math.isnan(y[0, 1]) and y[0, 2] == -inf and y[0, 3] == inf
        assert y[1, 0] == 6.0 and math.isnan(y[1, 1]) and y[1, 2] == 1.5 and y[1, 3] == 1.0
        a2 = store([[inf, 1.0]], dtype)
        b2 = store([[1.0, 0.0], [-1.0, 0.0]], dtype)
        a3 = np.concatenate([a2, store([[inf, 0.0]], dtype)])  # two rows, opposite sums
        b3 = store([[1.0, 0.0]], dtype)
        _, y3, _ = oracle.gemm_scatter(a3, b3, None, 1.0, 0.0, 1, dtype, want_f64=True, lib=lib)
        assert y3[0, 0] == inf and y3[1, 0] == inf
        _, y2, _ = oracle.gemm_scatter(a2, b2, None, 1.0, 0.0, 1, dtype, want_f64=True, lib=lib)
        assert y2[0, 0] == inf and y2[0, 1] == -inf
        # overflow on rounding
        big = 60000.0 if dtype == "f16" else 3.0e38
        a4 = store([[big, big]], dtype)
        b4 = store([[1.0, 1.0]], dtype)
        got = oracle.gemm_scatter(a4, b4, None, 1.0, 0.0, 1, dtype, lib=lib)[0]
        assert int(got[0, 0]) == (0x7C00 if dtype == "f16" else 0x7F80)


def pin_chunk_order(lib=None):
    """Other ranks' chunks first, each once, the local chunk last, starting
    with the next rank."""
    for world in (1, 2, 3, 8, 16):
        for rank in range(world):
            order = oracle.gemm_scatter_chunk_order(world, rank, lib=lib)
            assert sorted(order) == list(range(world))
            assert order[-1] == rank and order[0] == (rank + 1) % world
            assert all((order[s + 1] - order[s]) % world == 1 for s in range(world - 1))


def pin_power_of_two_scaling(lib=None):
    """Scaling A, or alpha, by 2^e scales every unrounded value by exactly
    2^e (in the normal range both are exact), so the stored values of the
    scaled product equal those of the product rounded after scaling."""
    rng = np.random.default_rng(21)
    for dtype in ("bf16", "f16"):
        a = value_grid(rng, (8, 40), dtype)
        b = value_grid(rng, (6, 40), dtype)
        c = value_grid(rng, (8, 6), dtype)
        _, y, _ = oracle.gemm_scatter(a, b, c, 0.75, 0.5, 2, dtype, want_f64=True, lib=lib)
        for e in (-3, 2):
            a2 = store(ind.decode_np(a, dtype) * 2.0 ** e, dtype)
            _, ya, _ = oracle.gemm_scatter(a2, b, None, 0.75, 0.0, 2, dtype, want_f64=True,
                                           lib=lib)
            _, y0, _ = oracle.gemm_scatter(a, b, None, 0.75, 0.0, 2, dtype, want_f64=True,
                                           lib=lib)
            assert np.array_equal(ya, y0 * 2.0 ** e)
            _, yb, _ = oracle.gemm_scatter(a, b, None, 0.75 * 2.0 ** e, 0.0, 2, dtype,
                                           want_f64=True, lib=lib)
            assert np.array_equal(yb, y0 * 2.0 ** e)
        # C enters once, scaled by beta: y(beta) - y(0) = beta * C exactly here
        _, yc0, _ = oracle.gemm_scatter(a, b, c, 0.75, 0.0, 2, dtype, want_f64=True, lib=lib)
        assert np.array_equal(y - yc0, 0.5 * ind.decode_np(c, dtype))


PINS = {"worked_example": pin_worked_example, "power_of_two_scaling": pin_power_of_two_scaling, "closed_forms": pin_closed_forms,
        "chunks_and_rows": pin_chunks_and_rows, "specials": pin_specials,
        "chunk_order": pin_chunk_order, "numpy_matmul": pin_numpy_matmul,
        "brute_force": pin_brute_force}


@pytest.mark.parametrize("name", list(PINS))
def test_gemm_scatter_pin(name):
    PINS[name]()


def test_gemm_scatter_oracle_errors():
    import ctypes
    lib = oracle._load()
    vp = ctypes.c_void_p
    buf = (ctypes.c_uint16 * 64)()
    p = ctypes.cast(buf, vp)
    dst = (vp * 2)(p, p)
    F = ctypes.c_float

    def call(world=2, m=4, n=2, k=2, dtype=2, r0=0, r1=4, lda=2, ldb=2, ldd=2, a=p, b=p,
             d=dst):
        return lib.gemm_scatter_oracle(d, ldd, world, a, lda, b, ldb, None, 0, F(1), F(0),
                                       m, n, k, dtype, r0, r1, None, None)

    assert call() == 0
    assert call(dtype=0) == -3 and call(dtype=7) == -3
    assert call(m=5) == -2 and call(world=0) == -2 and call(world=17) == -2
    assert call(r1=5) == -2 and call(r0=3, r1=2) == -2
    assert call(lda=1) == -2 and call(ldd=1) == -2
    assert call(a=None) == -1
    assert call(d=(vp * 2)(p, None)) == -1
    order = (ctypes.c_int * 4)()
    assert lib.gemm_scatter_oracle_chunk_order(4, 4, order) == -2
    assert lib.gemm_scatter_oracle_chunk_order(0, 0, order) == -2


MUTANTS = {
    "b_transposed": [("value[B[j * ldb + p]]", "value[B[p * ldb + j]]")],
    "beta_dropped": [("y += (double)beta * cv;", "y += cv;")],
    "alpha_dropped": [("double y = (double)alpha * dot;", "double y = dot;")],
    "float_accumulator": [("double dot = 0.0, dot_abs = 0.0;",
                           "float dot = 0.0f; double dot_abs = 0.0;")],
    "last_k_dropped": [("for (int64_t p = 0; p < k; ++p) {", "for (int64_t p = 0; p + 1 < k; ++p) {")],
    "chunk_off_by_one": [("uint16_t* out = (uint16_t*)dst[q] + (i - q * chunk) * ldd;",
                          "uint16_t* out = (uint16_t*)dst[(q + 1) % world] + (i - q * chunk) * ldd;")],
    "chunk_rows_interleaved": [("const int64_t q = i / chunk;", "const int64_t q = i % world;"),
                               ("(i - q * chunk) * ldd", "(i / world) * ldd")],
    "order_local_first": [("order[s] = (rank + 1 + s) % world;", "order[s] = (rank + s) % world;")],
    "rounded_through_float": [("row[j] = y;", "row[j] = (double)(float)y;")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gemm_scatter_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, old
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    rms = os.path.join(ROOT, "oracle", "rmsnorm_oracle.c")
    lib = oracle.load_library(oracle.compile_library([rms, str(path)], str(tmp_path / "libm.so")))
    caught = None
    with np.errstate(all="ignore"):
        for pin_name, pin in PINS.items():
            try:
                pin(lib=lib)
            except (AssertionError, RuntimeError):
                caught = pin_name
                break
    assert caught, name
