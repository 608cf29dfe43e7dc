"""The C ABI without a GPU: both libraries load, export every function their
headers declare, and reject invalid arguments with the documented codes
before touching the GPU (validation precedes any HIP call)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from row_wise_normalization_rmsnorm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M))


def test_gpu_library_exports_every_declared_function():
    names = declared("rmsnorm.h")
    assert {"rmsnorm_fwd", "add_rmsnorm_fwd", "rmsnorm_strerror"} <= names
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTS) == names


def test_block_sum_exports_every_declared_function():
    names = declared("block_sum.h")
    assert names == set(B.BLOCK_SUM_EXPORTS)
    for n in names:
        assert hasattr(B.lib(), n), n


def test_block_sum_error_codes():
    f = B.lib().block_all_reduce_sum
    ws = FAKE + (1 << 26)
    assert f(FAKE, FAKE + (1 << 20), 10, 9, ws, B.BRS_WORKSPACE_BYTES, None) == -3
    assert f(FAKE, FAKE + (1 << 20), -1, 0, ws, B.BRS_WORKSPACE_BYTES, None) == -2
    assert f(None, FAKE + (1 << 20), 10, 0, ws, B.BRS_WORKSPACE_BYTES, None) == -1
    assert f(FAKE, None, 10, 0, ws, B.BRS_WORKSPACE_BYTES, None) == -1
    assert f(FAKE, FAKE + (1 << 20), 10, 0, None, B.BRS_WORKSPACE_BYTES, None) == -1
    assert f(FAKE, FAKE + (1 << 20) + 2, 10, 0, ws, B.BRS_WORKSPACE_BYTES, None) == -2  # f32 at 2 mod 4
    assert f(FAKE, FAKE + (1 << 20), 10, 0, ws, B.BRS_WORKSPACE_BYTES - 4, None) == -2
    assert f(FAKE, FAKE + (1 << 20), 10, 0, ws + 8, B.BRS_WORKSPACE_BYTES, None) == -2
    assert f(FAKE + (1 << 20) + 4, FAKE + (1 << 20), 10, 0, ws, B.BRS_WORKSPACE_BYTES, None) == -5
    assert f(FAKE, FAKE + (1 << 20), 10, 0, FAKE + (1 << 20) + 16, B.BRS_WORKSPACE_BYTES, None) == -5


def test_oracle_library_exports_every_declared_function():
    import oracle
    names = declared("rmsnorm_oracle.h") | declared("block_sum_oracle.h") | \
        declared("gemm_scatter_oracle.h")
    assert {"rmsnorm_oracle", "block_sum_oracle"} <= names
    lib = oracle._load()
    for n in names:
        assert hasattr(lib, n), n


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def fwd(**kw):
    a = dict(out=FAKE, x=FAKE + (1 << 24), gamma=FAKE + (1 << 26), rows=4, hidden=64, eps=1e-6,
             dtype=2)
    a.update(kw)
    return B.lib().rmsnorm_fwd(a["out"], a["x"], a["gamma"], a["rows"], a["hidden"], a["eps"],
                               a["dtype"], None)


def add(k=1, parts=None, **kw):
    a = dict(out=FAKE, residual=FAKE + (1 << 24), gamma=FAKE + (1 << 26), rows=4, hidden=64,
             eps=1e-6, dtype=2)
    a.update(kw)
    parts = parts if parts is not None else [FAKE + (1 << 27) + i * (1 << 20) for i in range(k)]
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts)
    return B.lib().add_rmsnorm_fwd(a["out"], a["residual"], arr, k, a["gamma"], a["rows"],
                                   a["hidden"], a["eps"], a["dtype"], None)


def test_error_codes():
    assert fwd(dtype=3) == -3
    assert fwd(hidden=0) == -2
    assert fwd(hidden=(1 << 24) + 1) == -2
    assert fwd(rows=-1) == -2
    assert fwd(eps=-1.0) == -6
    assert fwd(eps=float("inf")) == -6
    assert fwd(eps=float("nan")) == -6
    assert fwd(out=0) == -1
    assert fwd(gamma=0) == -1
    assert fwd(rows=0, out=0, x=0, gamma=0) == 0          # rows == 0: no-op
    assert fwd(out=FAKE + 2, x=FAKE) == -5                 # partial overlap out/x
    assert fwd(gamma=FAKE + 64) == -5                      # out overlaps gamma
    assert add(k=0) == -4
    assert add(k=17) == -4
    assert add(k=2, parts=[FAKE + (1 << 27), 0]) == -1
    assert add(residual=FAKE + (1 << 27) + 8, k=1) == -5   # residual overlaps a partial
    assert add(out=FAKE + (1 << 24)) == -5                 # out overlaps residual
    assert add(k=1, parts=[FAKE + 16]) == -5               # out partially overlaps a partial
    assert add(gamma=FAKE + (1 << 24) + 100) == -5         # residual overlaps gamma
    assert "overlap" in B.lib().rmsnorm_last_error().decode()
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert B.lib().rmsnorm_strerror(code)


def test_plan_names_follow_the_dispatch_rule():
    plan = B.rmsnorm_plan
    assert plan(8192, 4096, 1, "bf16").startswith("vgpr<bf16")
    assert plan(4096, 8192, 8, "bf16").startswith("stream<bf16,v8")    # K >= 2, long rows
    assert plan(4096, 1024, 8, "bf16").startswith("vgpr<bf16")
    assert plan(512, 2048, 0, "f32").startswith("vgpr<f32")
    assert plan(65536, 16384, 1, "bf16").startswith("stream<bf16,v8")
    assert "lds" in plan(65536, 16384, 1, "bf16")
    assert ",wg=256,lds,k=-1,unr=8," in plan(65536, 16384, 1, "bf16")   # rows over 16 KiB
    assert plan(32768, 8192, 1, "f32").startswith("stream<f32,v8,wg=256,lds")
    assert plan(4096, 8192, 8, "bf16") == "stream<bf16,v8,wg=512,lds,k=-2,unr=4,nt>"  # pairs at K=8
    assert plan(4096, 8192, 4, "bf16") == "stream<bf16,v8,wg=512,lds,k=-1,unr=4,nt>"
    assert "k=-1" in B.rmsnorm_plan_ex(4096, 8192, 8, "bf16", "f32", "f32")      # none compiled
    assert "tpr=8," in plan(1000, 64, 1, "bf16")            # several rows per wave
    assert "tpr=64," in plan(512, 512, 0, "bf16")           # one row per wave
    # large plain launches: two chunks per thread; small ones and the fused form: one
    assert "tpr=256,npt=2," in plan(8192, 4096, 0, "bf16")
    assert "tpr=512,npt=1," in plan(512, 4096, 0, "bf16")
    assert "tpr=512,npt=1," in plan(8192, 4096, 1, "bf16")
    assert "elem" in plan(10, 1591, 0, "bf16")              # odd row length
    assert "elem" in plan(10, 4096, 1, "bf16", align=2)
    assert ",v4," in plan(10, 4096, 1, "bf16", align=4)        # 4-byte aligned bases
    assert ",v8," in plan(10, 4096, 1, "bf16", align=8)
    assert ",v4," in plan(10, 1594, 0, "bf16")                  # 3188-byte rows
    assert ",v8," in plan(10, 1596, 0, "bf16")                  # 3192-byte rows
    assert "elem" in plan(10, 1595, 0, "f32")
    assert ",v8," in plan(10, 1594, 0, "f32")
    assert "reread" in plan(10, 100000, 1, "bf16")          # row beyond the LDS stage
    for k in range(0, 17):
        assert plan(3, 777 * 8, k, "f16")


def test_variant_table_and_forcing(monkeypatch):
    names = B.rmsnorm_variants("bf16")
    assert len(names) == len(set(names)) > 50
    with B.forced("vgpr<bf16,tpr=64,npt=1,wg=256,k=1,nt>"):
        assert B.rmsnorm_plan(4, 512, 1, "bf16") == "vgpr<bf16,tpr=64,npt=1,wg=256,k=1,nt>"
        with pytest.raises(B.RmsnormError):
            B.rmsnorm_plan(4, 1024, 1, "bf16")   # too long for that variant
    assert B.rmsnorm_plan(4, 1024, 1, "bf16")    # the dispatcher decides again
    with B.forced("no-such-kernel"):
        with pytest.raises(B.RmsnormError):
            B.rmsnorm_plan(4, 512, 1, "bf16")
    with pytest.raises(B.RmsnormError):
        B.tune("x" * 128)                        # longer than the name slot


def test_environment_does_not_change_calls(monkeypatch):
    """The library reads no environment variable: variables that once forced
    a variant or capped the grid, set after load, change neither the plan of
    a call nor the check of a call's arguments."""
    base = B.rmsnorm_plan(8192, 4096, 1, "bf16")
    ex = plan_call(rows=8192, hidden=4096)
    monkeypatch.setenv("RMSNORM_VARIANT", "vgpr<bf16,tpr=64,npt=1,wg=256,k=1,nt>")
    monkeypatch.setenv("RMSNORM_GRID_CAP", "7")
    assert B.rmsnorm_plan(8192, 4096, 1, "bf16") == base
    assert plan_call(rows=8192, hidden=4096) == ex
    monkeypatch.setenv("RMSNORM_VARIANT", "no-such-kernel")
    assert B.rmsnorm_plan(8192, 4096, 1, "bf16") == base


def fwd_ex(**kw):
    a = dict(out=FAKE, out_stride=64, out_dtype=0, x=FAKE + (1 << 24), x_stride=64, dtype=2,
             gamma=FAKE + (1 << 26), gamma_dtype=0, rows=4, hidden=64, eps=1e-6)
    a.update(kw)
    return B.lib().rmsnorm_fwd_ex(a["out"], a["out_stride"], a["out_dtype"], a["x"], a["x_stride"],
                                  a["dtype"], a["gamma"], a["gamma_dtype"], a["rows"], a["hidden"],
                                  a["eps"], None)


def add_ex(k=1, parts=None, strides=None, **kw):
    a = dict(out=FAKE, out_stride=64, out_dtype=0, residual=FAKE + (1 << 24), res_stride=64,
             dtype=2, gamma=FAKE + (1 << 26), gamma_dtype=2, rows=4, hidden=64, eps=1e-6)
    a.update(kw)
    parts = parts if parts is not None else [FAKE + (1 << 27) + i * (1 << 20) for i in range(k)]
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts)
    st = None if strides is None else (ctypes.c_int64 * max(1, len(strides)))(*strides)
    return B.lib().add_rmsnorm_fwd_ex(a["out"], a["out_stride"], a["out_dtype"], a["residual"],
                                      a["res_stride"], arr, st, k, a["dtype"], a["gamma"],
                                      a["gamma_dtype"], a["rows"], a["hidden"], a["eps"], None)


def test_general_interface_error_codes():
    assert fwd_ex(gamma_dtype=1) == -3                     # fp16 gamma with bf16 data
    assert fwd_ex(out_dtype=3) == -3
    assert fwd_ex(dtype=7) == -3
    assert fwd_ex(x_stride=63) == -2                       # stride below hidden
    assert fwd_ex(out_stride=-64) == -2
    assert fwd_ex(x_stride=1 << 62) == -2                  # last row beyond the address range
    assert fwd_ex(out=0) == -1
    assert fwd_ex(rows=0, out=0, x=0, gamma=0) == 0
    assert fwd_ex(rows=1, x_stride=0, out=FAKE, x=FAKE + 2, out_dtype=2) == -5   # one row, shifted
    # out over x: refused unless same dtype and layout
    assert fwd_ex(out=FAKE, x=FAKE, out_dtype=0) == -5     # another dtype
    assert fwd_ex(out=FAKE, x=FAKE, out_dtype=2, out_stride=128, x_stride=64) == -5
    # equal pitches: rows that interleave share no byte (x at byte 0 of each
    # 256-byte row, out at byte 128), but a shift into x's bytes is caught
    assert fwd_ex(out=FAKE + 130, out_dtype=2, out_stride=128, x=FAKE, x_stride=128) == -5
    assert add_ex(k=2, strides=[64, 32]) == -2             # a partial's stride below hidden
    assert add_ex(res_stride=10) == -2
    assert add_ex(residual=0) == -1
    assert add_ex(k=0) == -4
    assert add_ex(residual=FAKE + (1 << 27) + 4, k=1) == -5  # residual overlaps the partial
    assert add_ex(gamma_dtype=1) == -3
    assert "dtype" in B.lib().rmsnorm_last_error().decode()


def test_general_interface_plans():
    plan = B.rmsnorm_plan_ex
    assert plan(8192, 4096, 1, "bf16", "f32", "f32") == \
        "vgpr<bf16,g=f32,o=f32,tpr=512,npt=1,wg=512,k=-1,nt>"
    assert plan(8192, 4096, 1, "bf16", "bf16", "bf16") == B.rmsnorm_plan(8192, 4096, 1, "bf16")
    assert plan(512, 2048, 0, "f32", "f32", "bf16").startswith("vgpr<f32,g=f32,o=bf16,tpr=512,npt=1")
    assert plan(8192, 2048, 0, "f32", "f32", "bf16").startswith("vgpr<f32,g=f32,o=bf16,tpr=256,npt=2")
    assert plan(4096, 8192, 8, "f16", "f32", "f16").startswith("stream<f16,g=f32,o=f16,v8,")
    assert "lds" in plan(100, 16384, 1, "bf16", "f32", "f32")
    assert "elem" in plan(10, 1595, 0, "f32", "f32", "f16")
    # 8-byte aligned bases: 8-byte bf16 chunks would need 16-byte fp32 ones,
    # so the data moves in 4-byte chunks (8 bytes of fp32 gamma and output)
    assert ",v4," in plan(10, 4096, 1, "bf16", "f32", "f32", align=8)
    assert "elem" in plan(10, 4096, 1, "bf16", "f32", "f32", align=4)
    assert "reread" in plan(10, 100000, 1, "bf16", "bf16", "f32")
    for k in range(0, 17):
        assert plan(3, 777 * 8, k, "bf16", "f32", "f16")
    with pytest.raises(B.RmsnormError):
        plan(3, 64, 0, "bf16", "f16", "bf16")


def test_general_interface_variant_tables():
    for d, n in (("bf16", 70), ("f16", 70), ("f32", 58)):
        for g in sorted({d, "f32"}):
            for o in ("f32", "f16", "bf16"):
                names = B.rmsnorm_variants_ex(d, g, o)
                if g == d == o:
                    assert names == B.rmsnorm_variants(d)
                    continue
                assert len(names) == len(set(names)) == n, (d, g, o, len(names))
                assert all(f"<{d},g={g},o={o}," in v for v in names)


def plan_call(out=FAKE, out_stride=64, out_dtype=2, residual=None, res_stride=64, parts=None,
              strides=None, dtype=2, gamma=FAKE + (1 << 26), gamma_dtype=2, rows=4, hidden=64,
              eps=1e-6):
    parts = parts if parts is not None else [FAKE + (1 << 24)]
    arr = (ctypes.c_void_p * len(parts))(*parts)
    st = None if strides is None else (ctypes.c_int64 * len(strides))(*strides)
    buf = ctypes.create_string_buffer(128)
    rc = B.lib().rmsnorm_plan_call(out, out_stride, out_dtype, residual, res_stride, arr, st,
                                   len(parts), dtype, gamma, gamma_dtype, rows, hidden, eps, buf, 128)
    return rc, buf.value.decode()


def test_plan_call_validates_without_launching():
    # interleaved rows of one buffer (x in the first half of each 256-byte
    # row, out in the second half): legal
    rc, name = plan_call(out=FAKE + 128, out_stride=128, parts=[FAKE], strides=[128])
    assert rc == 0 and name.startswith("vgpr<bf16,"), (rc, name)
    assert plan_call(out=FAKE + 126, out_stride=128, parts=[FAKE], strides=[128])[0] == -5
    # exact in place with the same stride: legal; with another dtype: not
    assert plan_call(out=FAKE, out_stride=128, parts=[FAKE], strides=[128])[0] == 0
    assert plan_call(out=FAKE, out_stride=128, out_dtype=1, parts=[FAKE], strides=[128])[0] == -5
    # row pitches decide the chunk width: 136-byte pitch -> 8-byte chunks,
    # 132 -> 4-byte, 130 -> elements
    for pitch_elems, width in ((68, ",v8,"), (66, ",v4,"), (65, "elem")):
        rc, name = plan_call(parts=[FAKE + (1 << 24)], strides=[pitch_elems])
        assert rc == 0 and width in name, (pitch_elems, name)
    # fp32 gamma with bf16 data and an fp32 output: 32-byte output chunks
    rc, name = plan_call(out_dtype=0, gamma_dtype=0, hidden=4096, out_stride=4096, strides=[4096])
    assert rc == 0 and name == "vgpr<bf16,g=f32,o=f32,tpr=512,npt=1,wg=512,k=0,nt>", name
    # ... whose 8-byte aligned base forces 4-byte data chunks (8 bytes of fp32)
    rc, name = plan_call(out=FAKE + 8, out_dtype=0, gamma_dtype=0, hidden=4096, out_stride=4096,
                         strides=[4096])
    assert rc == 0 and ",v4," in name, name
    # the fused form, and rows == 0
    rc, name = plan_call(residual=FAKE + (1 << 25), parts=[FAKE + (1 << 24), FAKE + (1 << 23)],
                         hidden=16384, out_stride=16384, res_stride=16384, strides=[16384, 16384])
    assert rc == 0 and name.startswith("stream<bf16,v8,") and "lds" in name, name
    assert plan_call(rows=0, out=0, gamma=0, parts=[0]) == (0, "none")


def test_row_collapse_rules():
    assert B.collapse_rows((8192, 4096), (4096, 1)) == (8192, 4096, 4096)
    assert B.collapse_rows((8192, 4096), (4224, 1)) == (8192, 4096, 4224)     # padded rows
    assert B.collapse_rows((3, 4, 1000), (4 * 1016, 1016, 1)) == (12, 1000, 1016)
    assert B.collapse_rows((1, 5, 1, 7), (99, 7, 7, 1)) == (5, 7, 7)            # size-1 dims ignored
    assert B.collapse_rows((), ()) == (1, 1, 1)
    assert B.collapse_rows((0, 16), (16, 1)) == (0, 16, 16)
    assert B.collapse_rows((6, 1), (3, 5)) == (6, 1, 3)                         # hidden 1: any stride
    with pytest.raises(B.RmsnormError):
        B.collapse_rows((4, 6, 1000), (1016, 4 * 1016, 1))                   # transposed leading dims
    with pytest.raises(B.RmsnormError):
        B.collapse_rows((16, 64), (1, 16))                                   # column-major


def test_dispatcher_covers_every_shape():
    """Every row length, K, alignment and row count finds a compiled kernel,
    for the single-dtype tables and every general combination."""
    hs = list(range(1, 70)) + [511, 512, 513, 1023, 1024, 1025, 1591, 1592, 2047, 2048, 4096,
                               4097, 8191, 8192, 8193, 12288, 16384, 16385, 20000, 32768, 32769,
                               40000, 65536, 70000]
    for d in ("bf16", "f16", "f32"):
        for h in hs:
            for k in (0, 1, 2, 8, 16):
                for al in (16, 8, 4, 2):
                    for rows in (1, 512, 65536):
                        assert B.rmsnorm_plan(rows, h, k, d, align=al)
        for g in sorted({d, "f32"}):
            for o in ("f32", "f16", "bf16"):
                for h in (1, 7, 64, 1592, 4096, 8192, 16384, 20000, 70000):
                    for k in (0, 1, 3, 8):
                        for al in (16, 8, 4, 2):
                            assert B.rmsnorm_plan_ex(65536, h, k, d, g, o, align=al)


# ---- the all-gather epilogue (add_rmsnorm_ag_fwd) ---------------------------

def add_ag(k=1, parts=None, outs=None, nout=None, **kw):
    a = dict(residual=FAKE + (1 << 24), gamma=FAKE + (1 << 26), rows=4, hidden=64, eps=1e-6,
             dtype=2)
    a.update(kw)
    parts = parts if parts is not None else [FAKE + (1 << 27) + i * (1 << 20) for i in range(k)]
    outs = outs if outs is not None else [FAKE + (1 << 29) + j * (1 << 20) for j in range(3)]
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts)
    oarr = (ctypes.c_void_p * max(1, len(outs)))(*outs)
    return B.lib().add_rmsnorm_ag_fwd(oarr, len(outs) if nout is None else nout, a["residual"],
                                      arr, k, a["gamma"], a["rows"], a["hidden"], a["eps"],
                                      a["dtype"], None)


def test_ag_error_codes():
    """add_rmsnorm_ag_fwd validates like add_rmsnorm_fwd, plus the output
    count and every output buffer (none may touch an input, gamma, the
    residual or another output, exact aliasing included)."""
    o = FAKE + (1 << 29)
    assert add_ag(nout=0) == -2 and add_ag(nout=17) == -2
    assert add_ag(k=0) == -4 and add_ag(k=17) == -4
    assert add_ag(dtype=3) == -3 and add_ag(hidden=0) == -2 and add_ag(eps=-1.0) == -6
    assert add_ag(outs=[o, 0]) == -1
    assert add_ag(residual=0) == -1 and add_ag(gamma=0) == -1
    assert add_ag(k=2, parts=[FAKE + (1 << 27), 0]) == -1
    assert add_ag(outs=[o, o + 256]) == -5                     # two outputs overlap
    assert add_ag(outs=[o, o]) == -5                           # ... even exactly
    assert add_ag(outs=[o, FAKE + (1 << 27)]) == -5            # an output is a partial
    assert add_ag(outs=[FAKE + (1 << 24) + 64]) == -5          # an output overlaps the residual
    assert add_ag(outs=[o, FAKE + (1 << 26) - 100]) == -5      # an output overlaps gamma
    assert add_ag(residual=FAKE + (1 << 27) + 8) == -5         # residual overlaps a partial
    assert "overlap" in B.lib().rmsnorm_last_error().decode()
    assert add_ag(rows=0, outs=[0], residual=0, gamma=0) == 0  # rows == 0: no-op
    with pytest.raises(B.RmsnormError):
        B.rmsnorm_plan_ag(4, 64, 0, "bf16")                    # the fused form only


def test_ag_plans_mirror_the_fused_dispatcher():
    """For every fused call the all-gather dispatcher takes the same shape as
    add_rmsnorm_fwd's, compiled with the all-gather epilogue."""
    import random
    rng = random.Random(3)
    cases = [(8192, 4096, 1, "bf16", 16), (4096, 8192, 8, "bf16", 16), (512, 8192, 8, "bf16", 16),
             (65536, 16384, 1, "bf16", 16), (100, 100000, 3, "f16", 16), (7, 17, 16, "bf16", 2)]
    for _ in range(300):
        cases.append((rng.randint(1, 5000), rng.randint(1, 70000), rng.randint(1, 16),
                      rng.choice(["bf16", "f16", "f32"]), rng.choice([1, 2, 4, 8, 16])))
    for rows, hidden, k, dtype, align in cases:
        plain = B.rmsnorm_plan(rows, hidden, k, dtype, align=align)
        assert B.rmsnorm_plan_ag(rows, hidden, k, dtype, align=align) == plain[:-1] + ",ag>", \
            (rows, hidden, k, dtype, align)
    for dtype in ("bf16", "f16", "f32"):
        names = B.rmsnorm_variants_ag(dtype)
        assert len(names) == len(set(names)) > 40 and all(n.endswith(",ag>") for n in names)


def test_ag_binding_checks_before_the_library():
    """The Python binding rejects host tensors and mismatched shapes or
    dtypes of the all-gather form before any library call."""
    import torch
    r = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(B.RmsnormError):
        B.add_rmsnorm_ag_fwd([torch.empty_like(r)], r, [r.clone()], g, 1e-6)       # host tensors
    with pytest.raises(B.RmsnormError):
        B.add_rmsnorm_ag_fwd([torch.empty(4, 32, dtype=torch.bfloat16)], r, [r], g, 1e-6)
    with pytest.raises(B.RmsnormError):
        B.add_rmsnorm_ag_fwd([torch.empty_like(r, dtype=torch.float16)], r, [r], g, 1e-6)


def test_binding_refuses_tensors_on_two_devices():
    """Every tensor of a call must be on the first tensor's GPU (a kernel on
    one GPU addresses them all directly): the device check the binding runs
    on each tensor, with stand-ins that report a device index."""
    class OnDevice:
        def __init__(self, d):
            self.d = d

        def get_device(self):
            return self.d

    assert B._device(OnDevice(0), "x") == 0 and B._device(OnDevice(3), "out", 3) == 3
    with pytest.raises(B.RmsnormError, match="out is on cuda:1, the call's other tensors on cuda:0"):
        B._device(OnDevice(1), "out", 0)
    with pytest.raises(B.RmsnormError, match="must be a device tensor"):
        B._device(OnDevice(-1), "gamma", 0)
    with pytest.raises(B.RmsnormError, match="must be a device tensor"):
        B._dev_ptr(OnDevice(-1), "x")


def test_overlap_brute_force(tmp_path):
    """The aliasing test (rmsn_host::overlap in csrc/rmsnorm_span.hpp),
    compiled on the host, against brute force over the bytes of random
    row-strided spans, unequal row counts included: it never misses a shared
    byte, and is exact for interleaving rows of one pitch."""
    src = os.path.join(ROOT, "tests", "span_bruteforce.cpp")
    inc = os.path.join(ROOT, "row_wise_normalization_rmsnorm_amd", "csrc")
    exe = str(tmp_path / "span_bruteforce")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-I", inc, "-o", exe, src], check=True)
    r = subprocess.run([exe, "300000"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr
    cases, exact = map(int, r.stdout.split()[1:3])
    assert cases == 300000 and exact > 10000


def test_block_sum_tune_range():
    """The block sum's grid override is an explicit call with a checked range
    (no environment variable is read)."""
    with pytest.raises(B.RmsnormError):
        B.block_sum_tune(-1)
    with pytest.raises(B.RmsnormError):
        B.block_sum_tune(B.BRS_MAX_GROUPS + 1)
    B.block_sum_tune(B.BRS_MAX_GROUPS)
    B.block_sum_tune(0)


def test_fastcall_marshalling_matches_ctypes():
    """The binding's CPython marshalling module for the per-step calls passes
    arguments through unchanged: on calls the library rejects before any
    launch, it returns the very codes the ctypes calls return."""
    from row_wise_normalization_rmsnorm_amd import _fastcall as F
    l = B.lib()
    assert B._fast is F
    P, G = FAKE, FAKE + (1 << 26)
    cases = [(P, P + (1 << 24), G, -1, 64, 1e-6, 2, None),       # rows < 0
             (P, P + (1 << 24), G, 4, 0, 1e-6, 2, None),         # hidden 0
             (P, P + (1 << 24), G, 4, 64, float("nan"), 2, None),  # eps NaN
             (None, P + (1 << 24), G, 4, 64, 1e-6, 2, None),     # out NULL
             (P, P + (1 << 24), G, 4, 64, 1e-6, 9, None),        # dtype
             (P + 2, P, G, 4, 64, 1e-6, 2, None),                # partial overlap
             (P, P + (1 << 24), G, 0, 64, 1e-6, 2, None)]        # rows 0: no-op
    for c in cases:
        rc = F.rmsnorm_fwd(*c)
        assert rc == l.rmsnorm_fwd(*c) and (rc != 0 or c[3] == 0), c
    arr = lambda ps: (ctypes.c_void_p * max(len(ps), 1))(*ps)  # noqa: E731
    R = FAKE + (1 << 25)
    # every call below is rejected before a launch, or has rows == 0 (a
    # no-op): the fake addresses are never dereferenced
    for ps, k, rows in (([P + (1 << 24)], 1, 0), ([], 0, 4), ([P + (1 << 24)] * 17, 17, 4),
                        ([R + 8], 1, 4), ([None], 1, 4), ([P + (1 << 24)], 1, -3)):
        want = l.add_rmsnorm_fwd(P, R, arr(ps), k, G, rows, 64, 1e-6, 2, None)
        got = F.add_rmsnorm_fwd(P, R, ps, G, rows, 64, 1e-6, 2, None)
        assert got == want and (got != 0 or rows == 0), (k, rows, got, want)
