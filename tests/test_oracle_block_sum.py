"""Pins of the block all-reduce sum oracle (page "Block All Reduce
CUDA代码学习": the sum of every element, narrow storage widened before
accumulation, fp8 decoded first, int8 accumulated in int32).

The oracle is checked against: torch's own fp8 / fp16 / bf16 decoders for
every code; math.fsum (the correctly rounded exact sum) within the double
accumulation bound; closed forms; Python integers for int8 (modulo 2^32);
and IEEE special cases.  Planted mistakes in a copy of the oracle are caught.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "block_sum_oracle.c")
FLOAT_DTYPES = ["f32", "f16", "bf16", "fp8_e4m3", "fp8_e5m2"]
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn,
         "fp8_e5m2": torch.float8_e5m2}


def storage_from_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(a.astype(np.float32))
    if dtype == "f32":
        return t.numpy()
    c = t.to(TORCH[dtype])
    return c.view(torch.uint8).numpy() if c.element_size() == 1 else \
        c.view(torch.int16).numpy().view(np.uint16)


def pin_decoders(lib=None):
    for dtype in ("fp8_e4m3", "fp8_e5m2"):
        codes = np.arange(256, dtype=np.uint8)
        got = oracle.block_sum_decode(codes, dtype, lib=lib)
        want = torch.from_numpy(codes).view(TORCH[dtype]).double().numpy()
        same = (got == want) | (np.isnan(got) & np.isnan(want))
        assert same.all(), (dtype, codes[~same][:8], got[~same][:8], want[~same][:8])
        assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(want[~np.isnan(want)]))
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dtype in ("f16", "bf16"):
        got = oracle.block_sum_decode(allbits, dtype, lib=lib)
        want = torch.from_numpy(allbits.view(np.int16)).view(TORCH[dtype]).double().numpy()
        assert ((got == want) | (np.isnan(got) & np.isnan(want))).all(), dtype


def pin_fsum(lib=None):
    rng = np.random.default_rng(3)
    for dtype in FLOAT_DTYPES:
        for n in (1, 7, 1000, 100_003):
            x = storage_from_f32(rng.standard_normal(n) * rng.uniform(0.1, 100), dtype)
            s, a = oracle.block_sum(x, dtype, lib=lib)
            vals = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x)
            if dtype != "f32":
                vals = vals.view(TORCH[dtype])
            v = vals.double().numpy()
            exact = math.fsum(v.tolist())
            assert abs(s - exact) <= n * 2.0 ** -53 * np.abs(v).sum() + 1e-300, (dtype, n)
            assert abs(a - math.fsum(np.abs(v).tolist())) <= n * 2.0 ** -53 * np.abs(v).sum()


def pin_closed_forms(lib=None):
    # 0, 1, ..., n-1 in f32 (exact), and +-1 alternating in every float dtype
    n = 4096
    s, _ = oracle.block_sum(np.arange(n, dtype=np.float32), "f32", lib=lib)
    assert s == n * (n - 1) / 2
    for dtype in FLOAT_DTYPES:
        x = storage_from_f32(np.tile([1.0, -1.0, 0.5], 999), dtype)
        assert oracle.block_sum(x, dtype, lib=lib)[0] == 999 * 0.5
        assert oracle.block_sum(x[:0], dtype, lib=lib)[0] == 0.0


def pin_int8(lib=None):
    rng = np.random.default_rng(5)
    x = rng.integers(-128, 128, 100_000, dtype=np.int8)
    got, exact = oracle.block_sum(x, "i8", lib=lib)
    assert exact == int(x.astype(np.int64).sum()) and got == exact
    big = np.full((1 << 25) + 3, 127, dtype=np.int8)     # exact sum 4.26e9 > 2^31
    got, exact = oracle.block_sum(big, "i8", lib=lib)
    want = 127 * ((1 << 25) + 3)
    assert exact == want
    assert got == ((want + 2 ** 31) % 2 ** 32) - 2 ** 31


def pin_specials(lib=None):
    x = storage_from_f32(np.array([1.0, np.nan, 2.0]), "bf16")
    assert math.isnan(oracle.block_sum(x, "bf16", lib=lib)[0])
    x = storage_from_f32(np.array([np.inf, 1.0, -np.inf]), "f32")
    assert math.isnan(oracle.block_sum(x, "f32", lib=lib)[0])
    x = storage_from_f32(np.array([np.inf, 1.0]), "fp8_e5m2")
    assert oracle.block_sum(x, "fp8_e5m2", lib=lib)[0] == math.inf
    nan_e4m3 = np.array([0x7F, 0x01], dtype=np.uint8)     # S.1111.111 is NaN; 0x01 = 2^-9
    assert math.isnan(oracle.block_sum(nan_e4m3, "fp8_e4m3", lib=lib)[0])
    assert oracle.block_sum(np.array([0x01, 0x7E], dtype=np.uint8), "fp8_e4m3", lib=lib)[0] == \
        2.0 ** -9 + 448.0


PINS = {"decoders": pin_decoders, "fsum": pin_fsum, "closed_forms": pin_closed_forms,
        "int8": pin_int8, "specials": pin_specials}


@pytest.mark.parametrize("name", list(PINS))
def test_block_sum_pin(name):
    PINS[name]()


def test_block_sum_oracle_errors():
    lib = oracle._load()
    import ctypes
    d = ctypes.c_double(0)
    assert lib.block_sum_oracle(ctypes.byref(d), None, None, None, 5, 0) == -1
    assert lib.block_sum_oracle(ctypes.byref(d), None, None, None, -1, 0) == -2
    assert lib.block_sum_oracle(ctypes.byref(d), None, None, None, 0, 9) == -3
    assert lib.block_sum_oracle(ctypes.byref(d), None, None, None, 0, 0) == 0


MUTANTS = {
    "e4m3_bias_8": [("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)")],
    "e4m3_inf_like_ieee": [("(e == 15 && m == 7) ? NAN", "(e == 15) ? (m ? NAN : INFINITY)")],
    "e5m2_subnormal_scale": [("ldexp((double)m, -16)", "ldexp((double)m, -15)")],
    "i8_no_wrap": [("uint32_t w = (uint32_t)(uint64_t)s;", "uint32_t w = (uint32_t)(s > 2147483647 ? 2147483647 : s);")],
    "i8_unsigned": [("s += (int8_t)((const unsigned char*)x)[i];", "s += ((const unsigned char*)x)[i];")],
    "float_accumulator": [("double s = 0.0, a = 0.0;", "float s = 0.0f; double a = 0.0;")],
    "last_element_dropped": [("for (int64_t i = 0; i < n; ++i) {\n    const double v", "for (int64_t i = 0; i + 1 < n; ++i) {\n    const double v")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_block_sum_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, old
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    rms = os.path.join(ROOT, "oracle", "rmsnorm_oracle.c")
    lib = oracle.load_library(oracle.compile_library([rms, str(path)], str(tmp_path / "libm.so")))
    caught = False
    for pin in PINS.values():
        try:
            pin(lib=lib)
        except AssertionError:
            caught = True
            break
    assert caught, name
