"""More GPU parity: seeded random shapes, streams, graph capture, N-D
inputs, rows beyond the LDS stage, and the largest sizes (row offsets past
4 GiB, hidden at its maximum).  Same bar as tests/parity.py."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from row_wise_normalization_rmsnorm_amd import binding as B
from row_wise_normalization_rmsnorm_amd import inputs as I
from tests import parity as P
from tests.test_gpu_parity import DEV, check, run_case, say

pytestmark = pytest.mark.gpu


def test_random_shapes():
    rng = np.random.default_rng(2024)
    for t in range(80):
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        hidden = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 9000)),
                                 int(rng.integers(9000, 40000))], p=[0.4, 0.45, 0.15]))
        if rng.random() < 0.5:
            hidden = max(8, hidden // 8 * 8)  # vector-eligible lengths half the time
        k = int(rng.choice([0, 1, 2, 3, 8, 16]))
        rows = int(rng.integers(1, 70))
        rows = max(1, min(rows, (4 << 20) // (hidden * (k + 1))))
        eps = float(rng.choice([1e-6, 1e-5, 1e-2]))
        w = I.case(dtype, rows, hidden, k, seed=t, std=float(rng.choice([0.25, 1.0, 30.0])), eps=eps)
        check(w, I.make_inputs(w), f"random #{t}")


def test_side_stream_and_ordering():
    w = I.case("bf16", 300, 4096, 1, seed=31)
    d = I.make_inputs(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ps = [p.to(DEV) for p in d["partials"]]
        r = d["residual"].to(DEV)
        g = d["gamma"].to(DEV)
        out = torch.empty_like(r)
        B.add_rmsnorm_fwd(out, r, ps, g, w.eps)         # enqueued on s
        r2 = r.clone()                                   # ordered after it on s
    s.synchronize()
    ref = P.run_oracle("bf16", w.eps, partials=d["partials"], residual=d["residual"], gamma=d["gamma"])
    P.compare("bf16", out.cpu(), ref, r2.cpu(), what="side stream")


def test_graph_capture_replays_match_eager():
    """Captured launches (no memset nodes), replayed several times with eager
    work in between; every replay equals the eager result."""
    w = I.case("bf16", 512, 4096, 2, seed=41)
    d = I.make_inputs(w)
    ps = [p.to(DEV) for p in d["partials"]]
    r0 = d["residual"].to(DEV)
    g = d["gamma"].to(DEV)
    x = I.make_inputs(I.case("bf16", 64, 1592, 0, seed=42))
    xs, gx = x["x"].to(DEV), x["gamma"].to(DEV)
    # eager reference of one step from the pristine residual
    r_e = r0.clone()
    out_e = torch.empty_like(r_e)
    B.add_rmsnorm_fwd(out_e, r_e, ps, g, w.eps)
    y_e = torch.empty_like(xs)
    B.rmsnorm_fwd(y_e, xs, gx, 1e-6)
    torch.cuda.synchronize()
    r = torch.empty_like(r0)
    out = torch.empty_like(r0)
    y = torch.empty_like(xs)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r.copy_(r0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            B.add_rmsnorm_fwd(out, r, ps, g, w.eps)
            B.rmsnorm_fwd(y, xs, gx, 1e-6)
    torch.cuda.synchronize()
    for rep in range(4):
        r.copy_(r0)                      # eager work between replays
        out.fill_(float("nan"))
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(r.view(torch.int16), r_e.view(torch.int16)), rep
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), rep
        assert torch.equal(y.view(torch.int16), y_e.view(torch.int16)), rep


def test_nd_inputs():
    w = I.case("bf16", 24, 2048, 1, seed=51)
    d = I.make_inputs(w)
    ps = [p.to(DEV).view(2, 3, 4, 2048) for p in d["partials"]]
    r = d["residual"].to(DEV).view(2, 3, 4, 2048)
    out = torch.empty_like(r)
    B.add_rmsnorm_fwd(out, r, ps, d["gamma"].to(DEV), w.eps)
    torch.cuda.synchronize()
    ref = P.run_oracle("bf16", w.eps, partials=d["partials"], residual=d["residual"], gamma=d["gamma"])
    P.compare("bf16", out.view(24, 2048).cpu(), ref, r.view(24, 2048).cpu(), what="N-D")


@pytest.mark.parametrize("dtype,hidden", [("bf16", 70000), ("f32", 40000), ("f16", 65537)])
def test_rows_beyond_the_lds_stage(dtype, hidden):
    for k in (0, 1, 4):
        w = I.case(dtype, 5, hidden, k, seed=hidden + k, std=0.4)
        plan = B.rmsnorm_plan(5, hidden, k, dtype)
        assert "reread" in plan, plan
        check(w, I.make_inputs(w), f"beyond LDS {dtype} H={hidden} k={k} ({plan})")


def test_maximum_hidden():
    hidden = 1 << 24
    for k in (0, 1):
        w = I.case("bf16", 2, hidden, k, seed=61 + k)
        check(w, I.make_inputs(w), f"hidden = 2^24, k={k}")


def test_offsets_beyond_4gib():
    """131080 rows x 16384 bf16: each tensor is 4.0002 GiB, so the last rows
    sit past byte offset 2^32.  Inputs drawn on the device; whole-tensor
    residual check against torch's fp32 sum, sampled rows against the oracle."""
    w = I.case("bf16", 131080, 16384, 1, seed=71)
    say("[gpu] >4 GiB tensors: drawing inputs on the device")
    p = I.device_tensor(w, 0, DEV)
    r = I.device_tensor(w, I.RESIDUAL_ID, DEV)
    g = I.gamma(w, DEV)
    rows = [0, 1, 65535, 131071, 131072, 131073, 131079]
    p_s, r_s = p[rows].cpu(), r[rows].cpu()
    want = (p.float() + r.float()).to(torch.bfloat16)
    out = torch.empty_like(r)
    B.add_rmsnorm_fwd(out, r, [p], g, w.eps)
    torch.cuda.synchronize()
    assert torch.equal(r.view(torch.int16), want.view(torch.int16))
    del want
    ref = P.run_oracle("bf16", w.eps, partials=[p_s], residual=r_s, gamma=g.cpu())
    P.compare("bf16", out[rows].cpu(), ref, r[rows].cpu(), what=">4 GiB offsets")


CANARY = 4096  # elements of guard on each side of every tensor


def _guarded(t):
    """A device copy of t placed between two guard regions filled with a
    pattern; returns (view, whole buffer)."""
    n = t.numel()
    buf = torch.empty(n + 2 * CANARY, dtype=t.dtype, device=DEV)
    buf.view(torch.int16 if t.element_size() == 2 else torch.int32).fill_(0x5A5A)
    v = buf[CANARY:CANARY + n].view(t.shape)
    v.copy_(t)
    return v, buf


@pytest.mark.parametrize("dtype,hidden,k", [("bf16", 4096, 1), ("bf16", 1591, 0), ("f32", 333, 3),
                                            ("f16", 16384, 1), ("bf16", 70000, 2), ("bf16", 24, 8),
                                            ("f32", 8192, 0), ("bf16", 1594, 1), ("bf16", 20000, 0),
                                            ("bf16", 12296, 3)])
def test_no_writes_outside_the_tensors(dtype, hidden, k):
    """Guard regions around out and the residual stay untouched (tails, odd
    lengths, every kernel family)."""
    rows = 13
    w = I.case(dtype, rows, hidden, k, seed=hidden + k)
    d = I.make_inputs(w)
    g = d["gamma"].to(DEV)
    out, obuf = _guarded(torch.zeros((rows, hidden), dtype=d["gamma"].dtype))
    guards = []
    if k:
        ps = [p.to(DEV) for p in d["partials"]]
        r, rbuf = _guarded(d["residual"])
        guards.append(rbuf)
        B.add_rmsnorm_fwd(out, r, ps, g, w.eps)
    else:
        B.rmsnorm_fwd(out, d["x"].to(DEV), g, w.eps)
    guards.append(obuf)
    torch.cuda.synchronize()
    for buf in guards:
        iv = buf.view(torch.int16 if buf.element_size() == 2 else torch.int32)
        assert torch.all(iv[:CANARY] == 0x5A5A) and torch.all(iv[-CANARY:] == 0x5A5A)


RESCUE_VARIANTS = {
    "bf16": ["vgpr<bf16,tpr=8,npt=1,wg=256,k=-1,nt>", "vgpr<bf16,tpr=64,npt=2,wg=256,k=-1,nt>",
             "vgpr<bf16,tpr=128,npt=2,wg=256,k=-1,nt>", "vgpr<bf16,tpr=512,npt=1,wg=512,k=1,nt>",
             "stream<bf16,v8,wg=512,lds,k=-1,unr=4,nt>", "stream<bf16,vec,wg=256,reread,k=-1,unr=2>",
             "stream<bf16,elem,wg=256,lds,k=-1,unr=4,nt>", None],
    "f32": ["vgpr<f32,tpr=16,npt=1,wg=256,k=0,nt>", "vgpr<f32,tpr=256,npt=2,wg=256,k=0,nt>",
            "stream<f32,v8,wg=256,lds,k=0,unr=4,nt>", "stream<f32,elem,wg=512,reread,k=0,unr=4>", None],
}


def _rescue_case(dtype, hidden, rows, k, eps, seed):
    """Rows of ordinary, huge (sum of squares past fp32's range) and tiny
    (squares below it) magnitudes, interleaved so that several rows of one
    workgroup or wave differ."""
    w = I.case(dtype, rows, hidden, k, seed=seed, std=0.5, eps=eps)
    d = I.make_inputs(w)
    scales = [1.0, 3e25, 1e-30, 1.0, 2e36, 5e-38, 1e-20]
    tensors = d["partials"] + [d["residual"]] if k else [d["x"]]
    for t in tensors:
        f = t.float()
        for i in range(rows):
            f[i] *= scales[i % len(scales)]
        t.copy_(f.to(t.dtype))
    return w, d


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rescaled_rows(dtype, monkeypatch):
    """Rows whose fp32 sum of squares overflows or underflows still match the
    double oracle, in every kernel family, with eps = 0 and eps > 0."""
    for i, variant in enumerate(RESCUE_VARIANTS[dtype]):
        kc = -1 if variant is None else int(variant.split("k=")[1].split(",")[0].rstrip(">"))
        k = {0: 0, 1: 1, -1: 2}[kc]
        if variant is None:
            B.tune(None)
            hidden = 4096
        else:
            B.tune(variant)
            hidden = None
            for h in (40, 512, 1000, 2048, 4096, 3000, 3001, 40000, 30000, 12000):
                try:
                    B.rmsnorm_plan(21, h, k, dtype)
                    hidden = h
                    break
                except B.RmsnormError:
                    continue
            assert hidden is not None, variant
        for eps in (0.0, 1e-6):
            w, d = _rescue_case(dtype, hidden, 21, k, eps, seed=100 + i)
            check(w, d, f"rescaled rows {variant} H={hidden} eps={eps}")
    B.tune(None)


def test_graph_capture_general_interface_and_block_sum():
    """The general interface (strided view, fp32 gamma, fp32 output) and the
    block sum (its completion counters reset by the kernel itself) captured
    in one graph; every replay, with eager work in between, equals the eager
    result bit for bit."""
    w = I.case("bf16", 96, 3072, 1, seed=61)
    d = I.make_inputs(w)
    big = torch.zeros(96, 3200, dtype=torch.bfloat16, device=DEV)
    p = big[:, 64:64 + 3072]
    p.copy_(d["partials"][0].to(DEV))
    r0 = d["residual"].to(DEV)
    g = I.gamma(w, DEV, dtype="f32")
    xs = I.make_inputs(I.case("bf16", 512, 1024, 0, seed=62))["x"].to(DEV).reshape(-1)
    ws = torch.zeros(B.BRS_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    r_e = r0.clone()
    out_e = torch.empty(96, 3072, dtype=torch.float32, device=DEV)
    B.add_rmsnorm_fwd_ex(out_e, r_e, [p], g, w.eps)
    s_e = torch.empty(1, dtype=torch.float32, device=DEV)
    B.block_all_reduce_sum_fwd(s_e, xs, ws)
    torch.cuda.synchronize()
    r = torch.empty_like(r0)
    out = torch.empty_like(out_e)
    s = torch.empty_like(s_e)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r.copy_(r0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            B.add_rmsnorm_fwd_ex(out, r, [p], g, w.eps)
            B.block_all_reduce_sum_fwd(s, xs, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        r.copy_(r0)
        out.fill_(float("nan"))
        s.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(r.view(torch.int16), r_e.view(torch.int16)), rep
        assert torch.equal(out.view(torch.int32), out_e.view(torch.int32)), rep
        assert torch.equal(s.view(torch.int32), s_e.view(torch.int32)), rep
        assert int(ws[:B.BRS_WORKSPACE_HEADER].count_nonzero()) == 0, rep
