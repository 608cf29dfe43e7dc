"""CPU oracle for row-wise RMSNorm and the fused K-partial + residual form.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never calls it; the product path has no CPU fallback.

This module is a thin ctypes wrapper over ``oracle/rmsnorm_oracle.c`` (plain C,
double accumulation, single-threaded), whose C ABI is declared in
``include/rmsnorm_oracle.h``.  Arrays are numpy: float32 data for "f32",
uint16 bit patterns for "f16" and "bf16".

What the oracle computes follows page "RMSNorm kernel" (section 1 Background
and section 2 "Abstraction") for the plain form and page "Tokenweave
fused-RMSNorm-AR kernel" (section "Code walkthrough") for the fused form; the
readings taken where they are silent are listed in the C source header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "rmsnorm_oracle.c"), os.path.join(_HERE, "block_sum_oracle.c"),
         os.path.join(_HERE, "gemm_scatter_oracle.c")]
_INCLUDE = os.path.join(os.path.dirname(_HERE), "include")
LIB_PATH = os.path.join(_HERE, "librmsnorm_oracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
KMAX = 16

_ERRORS = {
    -1: "null pointer",
    -2: "bad shape",
    -3: "bad dtype",
    -4: "bad k",
    -6: "bad eps",
    -8: "out of memory",
}

_default = None
_lock = threading.Lock()


def compile_library(src, out: str) -> str:
    """Compile oracle source file(s) with the oracle's flags: no FMA
    contraction, no fast-math, no excess precision (binary32 adds stay
    binary32)."""
    srcs = [src] if isinstance(src, str) else list(src)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
           "-I", _INCLUDE, "-o", tmp, *srcs, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle library in-tree."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_library(_SRCS, LIB_PATH)


class Library:
    """ctypes handle on one build of the oracle (the default build, or a
    deliberately mutated copy compiled by the oracle's mutation tests)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, dp, i64 = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_int64
        lib.rmsnorm_oracle.argtypes = [vp, vp, ctypes.POINTER(vp), ctypes.c_int, vp,
                                       i64, i64, ctypes.c_float, ctypes.c_int, dp]
        lib.rmsnorm_oracle.restype = ctypes.c_int
        lib.rmsnorm_oracle_f64.argtypes = [vp, dp, vp, ctypes.POINTER(vp), ctypes.c_int, vp,
                                           i64, i64, ctypes.c_float, ctypes.c_int, dp]
        lib.rmsnorm_oracle_f64.restype = ctypes.c_int
        if hasattr(lib, "rmsnorm_oracle_ex"):
            ci = ctypes.c_int
            lib.rmsnorm_oracle_ex.argtypes = [vp, ci, dp, vp, ctypes.POINTER(vp), ci, ci, vp, ci,
                                              i64, i64, ctypes.c_float, dp]
            lib.rmsnorm_oracle_ex.restype = ctypes.c_int
        lib.rmsnorm_oracle_round.argtypes = [vp, dp, i64, ctypes.c_int]
        lib.rmsnorm_oracle_round.restype = ctypes.c_int
        lib.rmsnorm_oracle_decode.argtypes = [dp, vp, i64, ctypes.c_int]
        lib.rmsnorm_oracle_decode.restype = ctypes.c_int
        if hasattr(lib, "block_sum_oracle"):
            lib.block_sum_oracle.argtypes = [dp, dp, ctypes.POINTER(ctypes.c_int32), vp, i64,
                                             ctypes.c_int]
            lib.block_sum_oracle.restype = ctypes.c_int
            lib.block_sum_oracle_decode.argtypes = [dp, vp, i64, ctypes.c_int]
            lib.block_sum_oracle_decode.restype = ctypes.c_int
        if hasattr(lib, "gemm_scatter_oracle"):
            lib.gemm_scatter_oracle.argtypes = [ctypes.POINTER(vp), i64, ctypes.c_int, vp, i64,
                                                vp, i64, vp, i64, ctypes.c_float, ctypes.c_float,
                                                i64, i64, i64, ctypes.c_int, i64, i64, dp, dp]
            lib.gemm_scatter_oracle.restype = ctypes.c_int
            lib.gemm_scatter_oracle_chunk_order.argtypes = [ctypes.c_int, ctypes.c_int,
                                                            ctypes.POINTER(ctypes.c_int)]
            lib.gemm_scatter_oracle_chunk_order.restype = ctypes.c_int
        self.lib = lib
        self.path = path


def load_library(path: str) -> Library:
    """Open another build of the oracle (the mutation tests use this)."""
    return Library(path)


def _load(lib: "Library | None" = None):
    global _default
    if lib is not None:
        return lib.lib
    with _lock:
        if _default is None:
            if not os.path.exists(LIB_PATH):
                build()
            _default = Library(LIB_PATH)
        return _default.lib


def _storage(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _check(arr: np.ndarray, dtype: str, shape=None) -> np.ndarray:
    want = _storage(dtype)
    if arr.dtype != want:
        raise TypeError(f"oracle expects {np.dtype(want)} storage for {dtype}, got {arr.dtype}")
    if not arr.flags.c_contiguous:
        raise ValueError("oracle expects C-contiguous arrays")
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError(f"shape {arr.shape} != {tuple(shape)}")
    return arr


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _dptr(a):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctypes.c_double))
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _raise(rc: int):
    if rc != 0:
        raise RuntimeError(f"rmsnorm_oracle failed: {rc} ({_ERRORS.get(rc, 'unknown')})")


def _general(out, y64, res, parts, gamma, rows, hidden, eps, dtype, gamma_dtype, out_dtype,
             rstd, lib):
    k = len(parts)
    arr = (ctypes.c_void_p * max(k, 1))(*[p.ctypes.data for p in parts])
    rc = _load(lib).rmsnorm_oracle_ex(_ptr(out), DTYPE_CODE[out_dtype], _dptr(y64),
                                      None if res is None else _ptr(res), arr, k,
                                      DTYPE_CODE[dtype], _ptr(gamma), DTYPE_CODE[gamma_dtype],
                                      rows, hidden, ctypes.c_float(eps), _dptr(rstd))
    _raise(rc)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, dtype: str, *,
            gamma_dtype: str = None, out_dtype: str = None,
            want_f64: bool = False, lib: "Library | None" = None):
    """Plain RMSNorm of x[rows, hidden].  Returns (out, rstd[rows]) and, with
    ``want_f64``, the unrounded double y as a third item.  gamma_dtype and
    out_dtype default to dtype."""
    gamma_dtype = gamma_dtype or dtype
    out_dtype = out_dtype or dtype
    rows, hidden = x.shape
    _check(x, dtype)
    _check(gamma, gamma_dtype, (hidden,))
    out = np.empty((rows, hidden), dtype=_storage(out_dtype))
    rstd = np.empty(rows, dtype=np.float64)
    y64 = np.empty((rows, hidden), dtype=np.float64) if want_f64 else None
    if gamma_dtype == dtype and out_dtype == dtype:
        parts = (ctypes.c_void_p * 1)(x.ctypes.data)
        rc = _load(lib).rmsnorm_oracle_f64(_ptr(out), _dptr(y64), None, parts, 1, _ptr(gamma),
                                           rows, hidden, ctypes.c_float(eps), DTYPE_CODE[dtype],
                                           _dptr(rstd))
        _raise(rc)
    else:
        _general(out, y64, None, [x], gamma, rows, hidden, eps, dtype, gamma_dtype, out_dtype,
                 rstd, lib)
    return (out, rstd, y64) if want_f64 else (out, rstd)


def add_rmsnorm(partials, residual: np.ndarray, gamma: np.ndarray, eps: float, dtype: str,
                *, gamma_dtype: str = None, out_dtype: str = None,
                want_f64: bool = False, lib: "Library | None" = None):
    """Fused form.  ``residual`` is NOT modified; the oracle works on a copy.
    Returns (out, new_residual, rstd) and, with ``want_f64``, the unrounded y.
    gamma_dtype and out_dtype default to dtype."""
    gamma_dtype = gamma_dtype or dtype
    out_dtype = out_dtype or dtype
    rows, hidden = residual.shape
    _check(residual, dtype)
    _check(gamma, gamma_dtype, (hidden,))
    parts = [_check(p, dtype, (rows, hidden)) for p in partials]
    k = len(parts)
    out = np.empty((rows, hidden), dtype=_storage(out_dtype))
    res = residual.copy()
    rstd = np.empty(rows, dtype=np.float64)
    y64 = np.empty((rows, hidden), dtype=np.float64) if want_f64 else None
    if gamma_dtype == dtype and out_dtype == dtype:
        arr = (ctypes.c_void_p * max(k, 1))(*[p.ctypes.data for p in parts])
        rc = _load(lib).rmsnorm_oracle_f64(_ptr(out), _dptr(y64), _ptr(res), arr, k,
                                           _ptr(gamma), rows, hidden, ctypes.c_float(eps),
                                           DTYPE_CODE[dtype], _dptr(rstd))
        _raise(rc)
    else:
        _general(out, y64, res, parts, gamma, rows, hidden, eps, dtype, gamma_dtype, out_dtype,
                 rstd, lib)
    return (out, res, rstd, y64) if want_f64 else (out, res, rstd)


def raw_call(out, residual, partials, gamma, rows, hidden, eps, dtype_code,
             lib: "Library | None" = None) -> int:
    """Direct call with arbitrary (possibly invalid) arguments; returns the code."""
    k = len(partials)
    arr = (ctypes.c_void_p * max(k, 1))(*[(p.ctypes.data if p is not None else None)
                                          for p in partials])
    return _load(lib).rmsnorm_oracle(
        None if out is None else _ptr(out), None if residual is None else _ptr(residual),
        arr, k, None if gamma is None else _ptr(gamma), rows, hidden,
        ctypes.c_float(eps), dtype_code, _dptr(None))


def round_to(values: np.ndarray, dtype: str, lib: "Library | None" = None) -> np.ndarray:
    """Round float64 values to dtype with the oracle's converter."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    dst = np.empty(v.shape, dtype=_storage(dtype))
    _raise(_load(lib).rmsnorm_oracle_round(_ptr(dst), _dptr(v), v.size, DTYPE_CODE[dtype]))
    return dst


def decode(bits: np.ndarray, dtype: str, lib: "Library | None" = None) -> np.ndarray:
    """Exact float64 values of dtype storage."""
    b = _check(np.ascontiguousarray(bits), dtype)
    dst = np.empty(b.shape, dtype=np.float64)
    _raise(_load(lib).rmsnorm_oracle_decode(_dptr(dst), _ptr(b), b.size, DTYPE_CODE[dtype]))
    return dst


# ---- block all-reduce sum family -------------------------------------------

SUM_DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8_e4m3": 3, "fp8_e5m2": 4, "i8": 5}


def _sum_storage(dtype: str):
    return {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}.get(
        dtype, np.int8 if dtype == "i8" else np.uint8)


def block_sum(x: np.ndarray, dtype: str, lib: "Library | None" = None):
    """Sum of all elements of x (numpy storage: float32, uint16 bit patterns,
    uint8 fp8 codes, or int8).  Floating dtypes: (sum, sum of |x|) as
    floats; i8: (int32 sum modulo 2^32, exact sum)."""
    a = np.ascontiguousarray(x)
    if a.dtype != _sum_storage(dtype):
        raise TypeError(f"block_sum oracle expects {np.dtype(_sum_storage(dtype))} for {dtype}")
    s = np.zeros(1, np.float64)
    ab = np.zeros(1, np.float64)
    i32 = ctypes.c_int32(0)
    rc = _load(lib).block_sum_oracle(_dptr(s), _dptr(ab), ctypes.byref(i32),
                                     ctypes.c_void_p(a.ctypes.data) if a.size else None, a.size,
                                     SUM_DTYPE_CODE[dtype])
    _raise(rc)
    if dtype == "i8":
        return int(i32.value), float(s[0])
    return float(s[0]), float(ab[0])


def block_sum_decode(x: np.ndarray, dtype: str, lib: "Library | None" = None) -> np.ndarray:
    a = np.ascontiguousarray(x)
    dst = np.empty(a.shape, np.float64)
    _raise(_load(lib).block_sum_oracle_decode(_dptr(dst), ctypes.c_void_p(a.ctypes.data), a.size,
                                              SUM_DTYPE_CODE[dtype]))
    return dst


# ---- GEMM with a reduce-scatter epilogue ------------------------------------

def gemm_scatter(a: np.ndarray, b: np.ndarray, c, alpha: float, beta: float, world: int,
                 dtype: str, rows=None, want_f64: bool = False, scatter: bool = True,
                 lib: "Library | None" = None):
    """``alpha * a @ b.T + beta * c`` split into ``world`` row chunks.

    a [m, k], b [n, k] and c [m, n] (or None) are uint16 bit patterns of
    dtype ("f16" or "bf16"); row strides are taken from the arrays, which must
    have unit element stride.  ``rows`` = (row0, row1) restricts the rows
    computed (default: all).  Returns the list of ``world`` chunks ([m/world,
    n] uint16; for a row range only the rows inside it are filled, the others
    are zero) and, with ``want_f64``, (y, mag) for the computed rows: the
    unrounded values and the magnitude scale of their rounding error bound.
    With ``scatter=False`` nothing is scattered: the first item is instead
    the computed rows ([row1 - row0, n] uint16), rounded by the oracle's
    converter.
    """
    m, k = a.shape
    n = b.shape[0]
    for arr, what in ((a, "a"), (b, "b")) + (((c, "c"),) if c is not None else ()):
        if arr.dtype != np.uint16 or arr.ndim != 2 or (arr.shape[1] > 1 and arr.strides[1] != 2):
            raise ValueError(f"{what}: expected a 2-D uint16 array with unit element stride")
    if b.shape[1] != k or (c is not None and c.shape != (m, n)):
        raise ValueError("shape mismatch")
    if world < 1 or m % world:
        raise ValueError("m must split into world equal chunks")
    r0, r1 = rows if rows is not None else (0, m)
    chunks = [np.zeros((m // world, n), np.uint16) for _ in range(world)] if scatter else None
    ptrs = (ctypes.c_void_p * world)(*[ch.ctypes.data for ch in chunks]) if scatter else None
    y = np.empty((r1 - r0, n), np.float64) if (want_f64 or not scatter) else None
    mag = np.empty((r1 - r0, n), np.float64) if want_f64 else None
    rc = _load(lib).gemm_scatter_oracle(
        ptrs, n, world, _ptr(a), _ld(a), _ptr(b), _ld(b),
        None if c is None else _ptr(c), 0 if c is None else _ld(c),
        ctypes.c_float(alpha), ctypes.c_float(beta), m, n, k, DTYPE_CODE[dtype], r0, r1,
        _dptr(y), _dptr(mag))
    _raise(rc)
    first = chunks if scatter else round_to(y, dtype, lib=lib)
    return (first, y, mag) if want_f64 else first


def _ld(arr: np.ndarray) -> int:
    """Row stride in elements (at least the row length, also for one row)."""
    return max(arr.strides[0] // 2, arr.shape[1]) if arr.shape[0] > 1 else arr.shape[1]


def gemm_scatter_chunk_order(world: int, rank: int, lib: "Library | None" = None) -> list:
    """The order in which one rank's chunks are produced: the other ranks'
    chunks first, the rank's own last."""
    order = (ctypes.c_int * max(world, 1))()
    _raise(_load(lib).gemm_scatter_oracle_chunk_order(world, rank, order))
    return list(order[:world])
