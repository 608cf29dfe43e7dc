"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every comparison applies the bar in ``tests/parity.py``: residual byte-exact,
fp32 output within 1e-5 relative, fp16 / bf16 output within 2 ulp, NaN
positions identical.  Inputs come from the seeded generators in
``row_wise_normalization_rmsnorm_amd.inputs``; expected values only from the
oracle.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from row_wise_normalization_rmsnorm_amd import binding as B
from row_wise_normalization_rmsnorm_amd import inputs as I
from row_wise_normalization_rmsnorm_amd.workloads import WORKLOADS
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()  # raises if the HIP library is missing
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_case(w, d, *, alias_out=False, sync=True):
    """Run the HIP path on copies of the CPU inputs ``d``; return CPU results.
    Outputs start poisoned with NaN, so an element the kernel fails to write
    shows up as a NaN mismatch."""
    g = d["gamma"].to(DEV)
    if w.fused:
        ps = [p.to(DEV) for p in d["partials"]]
        r = d["residual"].to(DEV)
        out = ps[0] if alias_out else torch.full_like(r, float("nan"))
        B.add_rmsnorm_fwd(out, r, ps, g, w.eps)
        torch.cuda.synchronize()
        return out.cpu(), r.cpu()
    x = d["x"].to(DEV)
    out = x if alias_out else torch.full_like(x, float("nan"))
    B.rmsnorm_fwd(out, x, g, w.eps)
    torch.cuda.synchronize()
    return out.cpu(), None


def check(w, d, what, **kw):
    say(f"[gpu] {what}: {w.describe()}")
    out, res = run_case(w, d, **kw)
    ref = P.run_oracle(w.dtype, w.eps, x=d.get("x"), partials=d.get("partials"),
                       residual=d.get("residual"), gamma=d["gamma"])
    return P.compare(w.dtype, out, ref, res, what=what)


# ---- the workloads ----------------------------------------------------------

@pytest.mark.parametrize("name", ["rmsnorm_f32_512x2048", "rmsnorm_bf16_512x1592",
                                  "rmsnorm_f16_512x1592"])
def test_small_workloads_full(name):
    w = WORKLOADS[name]
    stats = check(w, I.make_inputs(w), name)
    say(f"[gpu] {name}: {stats}")


def _sample_rows(w, n=128):
    rng = np.random.default_rng(12345)
    pick = set(range(8)) | set(range(w.rows - 8, w.rows))
    pick |= set(rng.choice(w.rows, size=n, replace=False).tolist())
    if w.special_frac:
        scaled, zeroed = I.special_rows(w)
        pick |= set(scaled[:6].tolist()) | set(zeroed[:6].tolist())
    return sorted(pick)


@pytest.mark.parametrize("name", ["add_rmsnorm_bf16_8192x4096_k1", "add_rmsnorm_bf16_4096x8192_k8",
                                  "add_rmsnorm_bf16_65536x16384_k1"])
def test_large_workloads_full_size(name):
    """Full-size launch (the configuration the benchmark times).  Every row
    of the output and of the in-place residual is compared with the oracle,
    in row blocks over the host's threads; besides, the whole residual equals
    the fp32 sum rounded once as torch computes it on the GPU (a different
    implementation), and the zero rows give zero outputs."""
    w = WORKLOADS[name]
    say(f"[gpu] {name}: generating full-size inputs on the device")
    d = I.make_inputs(w, device=DEV)
    g, ps, r = d["gamma"], d["partials"], d["residual"]
    host_ps = [I.to_storage(p) for p in ps]       # the inputs as launched
    host_r = I.to_storage(r)
    acc = ps[0].float()
    for p in ps[1:]:
        acc += p.float()
    acc += r.float()
    want_res = acc.to(r.dtype)
    del acc
    out = torch.empty_like(r)
    say(f"[gpu] {name}: plan {B.rmsnorm_plan(w.rows, w.hidden, w.k, w.dtype)}")
    B.add_rmsnorm_fwd(out, r, ps, g, w.eps)
    torch.cuda.synchronize()
    assert torch.equal(r.view(torch.int16), want_res.view(torch.int16)), "residual mismatch"
    del want_res
    if w.special_frac:
        _, zeroed = I.special_rows(w)
        zi = torch.from_numpy(zeroed).to(DEV)
        assert torch.all(out.index_select(0, zi) == 0) and torch.all(r.index_select(0, zi) == 0)
    gpu_out, gpu_res = I.to_storage(out), I.to_storage(r)
    del out, d, ps, r
    say(f"[gpu] {name}: every row against the oracle")
    stats = P.compare_whole(w.dtype, w.eps, gpu_out, gpu_res, I.to_storage(g), partials=host_ps,
                            residual=host_r, what=name)
    assert stats["rows_checked"] == w.rows and stats["residual_bit_exact"]
    if w.special_frac:
        scaled, zeroed = I.special_rows(w)
        say(f"[gpu] {name}: {len(scaled)} rows x1e3 and {len(zeroed)} zero rows among them")
    say(f"[gpu] {name}: whole tensor {stats}")


@pytest.mark.parametrize("dtype,rows,hidden", [("bf16", 8192, 4096), ("f32", 8192, 2048),
                                               ("f16", 16384, 1592)])
def test_large_plain_launches(dtype, rows, hidden):
    """Large plain launches take the two-chunks-per-thread shape; every row
    against the oracle."""
    w = I.case(dtype, rows, hidden, 0, seed=rows + hidden)
    plan = B.rmsnorm_plan(rows, hidden, 0, dtype)
    say(f"[gpu] large plain {dtype} {rows}x{hidden}: plan {plan}")
    assert "npt=2" in plan
    d = I.make_inputs(w, device=DEV)
    out = torch.full_like(d["x"], float("nan"))
    B.rmsnorm_fwd(out, d["x"], d["gamma"], w.eps)
    torch.cuda.synchronize()
    stats = P.compare_whole(dtype, w.eps, I.to_storage(out), None, I.to_storage(d["gamma"]),
                            x=I.to_storage(d["x"]), what=f"large plain {dtype}")
    assert stats["rows_checked"] == rows
    say(f"[gpu] large plain {dtype} {rows}x{hidden}: whole tensor {stats}")


# ---- shapes, tails, partial counts ---------------------------------------------

TAIL_H = [1, 2, 7, 8, 63, 64, 65, 511, 1591, 1592, 2048, 4096, 8191, 8192, 8193, 16384, 20000]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("hidden", TAIL_H)
def test_tail_sweep(dtype, hidden):
    for k in (0, 1, 3, 8):
        rows = 37 if hidden <= 8192 else 9
        w = I.case(dtype, rows, hidden, k, seed=hidden * 10 + k, std=0.35 if k > 1 else 1.0)
        check(w, I.make_inputs(w), f"tail {dtype} H={hidden} k={k}")


@pytest.mark.parametrize("dtype,hidden", [("bf16", 32768), ("f16", 32768), ("f32", 16384),
                                          ("bf16", 32760), ("f32", 16383)])
def test_lds_stage_limit(dtype, hidden):
    """Rows at the LDS stage budget (64 KiB of row: the largest the staged
    streaming kernel takes) and just below it, plain and fused."""
    for k in (0, 1):
        w = I.case(dtype, 7, hidden, k, seed=hidden + k)
        plan = B.rmsnorm_plan(7, hidden, k, dtype)
        say(f"[gpu] lds stage limit {dtype} H={hidden} k={k}: {plan}")
        check(w, I.make_inputs(w), f"lds stage limit {dtype} H={hidden} k={k}")


@pytest.mark.parametrize("k", [2, 4, 5, 15, 16])
def test_partial_counts(k):
    for dtype, hidden in (("bf16", 4096), ("f16", 1592), ("f32", 300), ("bf16", 12000)):
        w = I.case(dtype, 19, hidden, k, seed=k, std=0.3)
        check(w, I.make_inputs(w), f"k={k} {dtype} H={hidden}")


@pytest.mark.parametrize("rows", [1, 255, 257, 65536])
def test_row_counts(rows):
    for dtype, hidden, k in (("bf16", 64, 1), ("bf16", 1592, 0), ("f32", 24, 2)):
        if rows == 65536 and hidden > 64:
            continue
        w = I.case(dtype, rows, hidden, k, seed=rows)
        check(w, I.make_inputs(w), f"rows={rows} {dtype} H={hidden} k={k}")


def test_zero_rows_is_noop():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(x)
    B.rmsnorm_fwd(out, x, g, 1e-6)
    r = torch.zeros_like(x)
    B.add_rmsnorm_fwd(out, r, [x], g, 1e-6)
    torch.cuda.synchronize()


# ---- every compiled variant -----------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_every_variant(dtype, monkeypatch):
    names = B.rmsnorm_variants(dtype)
    assert names
    for i, name in enumerate(names):
        hidden, rows, k = P.variant_case(dtype, name)
        w = I.case(dtype, rows, hidden, k, seed=i, std=0.5)
        B.tune(name)
        assert B.rmsnorm_plan(rows, hidden, k, dtype, align=16) == name
        check(w, I.make_inputs(w), f"variant {name}")
    B.tune(None)


def test_grid_stride_loop(monkeypatch):
    """A capped grid makes every workgroup loop over several rows."""
    B.tune(None, grid_cap=7)
    for dtype, hidden, k in (("bf16", 4096, 1), ("bf16", 1592, 0), ("bf16", 128, 1),
                             ("bf16", 16384, 1), ("f32", 333, 2), ("bf16", 4096, 8)):
        w = I.case(dtype, 203, hidden, k, seed=hidden)
        check(w, I.make_inputs(w), f"grid cap 7 {dtype} H={hidden} k={k}")


# ---- alignment, aliasing, special values, determinism ------------------------------

@pytest.mark.parametrize("shift,width", [(1, "elem"), (2, "v4"), (4, "v8"), (8, "vec")])
def test_misaligned_pointers_use_narrower_chunks(shift, width):
    """Bases offset by `shift` bf16 elements from a 16-byte boundary take the
    widest chunk the shared alignment allows."""
    w = I.case("bf16", 33, 1592, 1, seed=77 + shift)
    d = I.make_inputs(w)
    n = 33 * 1592
    align = min(16, 2 * shift)
    plan = B.rmsnorm_plan(33, 1592, 1, "bf16", align=align)
    assert (f",{width}," in plan) or (width == "vec" and plan.startswith("vgpr<")), plan

    def shifted(t):
        buf = torch.empty(n + 16, dtype=t.dtype, device=DEV)
        v = buf[shift:shift + n].view(33, 1592)
        v.copy_(t)
        return v

    ps = [shifted(p) for p in d["partials"]]
    r = shifted(d["residual"])
    out = shifted(torch.zeros_like(d["residual"]))
    g = torch.empty(1600, dtype=torch.bfloat16, device=DEV)[shift:shift + 1592]
    g.copy_(d["gamma"])
    B.add_rmsnorm_fwd(out, r, ps, g, w.eps)
    torch.cuda.synchronize()
    ref = P.run_oracle("bf16", w.eps, partials=d["partials"], residual=d["residual"], gamma=d["gamma"])
    P.compare("bf16", out.cpu(), ref, r.cpu(), what=f"shift {shift}")


def test_out_aliases_input():
    for dtype, hidden in (("bf16", 4096), ("f32", 2048), ("bf16", 16384), ("f16", 1001)):
        w = I.case(dtype, 21, hidden, 0, seed=3)
        check(w, I.make_inputs(w), f"out is x {dtype} H={hidden}", alias_out=True)
        w = I.case(dtype, 21, hidden, 2, seed=4)
        check(w, I.make_inputs(w), f"out is partials[0] {dtype} H={hidden}", alias_out=True)


def _special_inputs(dtype, hidden):
    w = I.case(dtype, 6, hidden, 1, seed=5)
    d = I.make_inputs(w)
    p, r = d["partials"][0], d["residual"]
    p[0].zero_()
    r[0].zero_()                        # zero row (eps-dominated)
    p[1] = -0.0
    r[1] = -0.0                         # all negative zeros: sum stays -0.0
    # huge row: its fp32 sum of squares overflows (f32 / bf16), so the
    # kernels take their rescaled path
    big = {"f32": 1e30, "f16": 3e3, "bf16": 1e30}[dtype]
    p[2] *= big
    r[2] *= big
    tiny = {"f32": 1e-41, "f16": 1e-7, "bf16": 1e-40}[dtype]
    p[3] = tiny
    r[3] = -tiny / 2                    # denormal row
    p[4, ::3] = float("inf")            # inf elements: NaN there, 0 elsewhere
    return w, d


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_special_values(dtype):
    for hidden in (64, 4096, 16384):
        w, d = _special_inputs(dtype, hidden)
        check(w, d, f"special values {dtype} H={hidden}")


def test_nan_propagates():
    w = I.case("bf16", 4, 4096, 1, seed=9)
    d = I.make_inputs(w)
    d["partials"][0][2, 100] = float("nan")
    check(w, d, "nan row")


def test_deterministic():
    w = WORKLOADS["add_rmsnorm_bf16_4096x8192_k8"]
    rows = list(range(512))
    d = I.make_inputs(w, rows=rows)
    w2 = I.case("bf16", 512, w.hidden, 8, seed=0)
    a = run_case(w2, d)
    b = run_case(w2, d)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))


def test_alias_errors_launch_nothing():
    x = torch.randn(8, 64, device=DEV).to(torch.bfloat16)
    g = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    r = torch.randn(8, 64, device=DEV).to(torch.bfloat16)
    before = r.clone()
    out = torch.full_like(r, 7.0)
    with pytest.raises(B.RmsnormError) as e:
        B.add_rmsnorm_fwd(out, r, [r], g, 1e-6)   # residual is a partial
    assert e.value.code == -5
    with pytest.raises(B.RmsnormError) as e:
        B.add_rmsnorm_fwd(r, r, [x], g, 1e-6)     # out is the residual
    assert e.value.code == -5
    flat = torch.empty(8 * 64 + 32, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.RmsnormError) as e:
        B.rmsnorm_fwd(flat[16:16 + 512].view(8, 64), flat[:512].view(8, 64), g, 1e-6)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert torch.equal(r, before) and torch.all(out == 7.0)
