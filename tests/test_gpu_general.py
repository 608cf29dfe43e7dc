"""GPU parity of the general interface (rmsnorm_fwd_ex / add_rmsnorm_fwd_ex,
include/rmsnorm.h) against the oracle's general form.

The general interface takes the input as [..., hidden] (page "RMSNorm
kernel", section 2): every tensor is a view with its own row stride, gamma may
be fp32 with 16-bit data, and the output may have a dtype of its own.  The bar
is the one in ``tests/parity.py``, applied in the output's dtype; the residual
(in the data dtype) is byte-exact.  Every view sits inside a larger buffer
whose other bytes hold a sentinel, so a write outside the rows fails the test.
"""
from __future__ import annotations

import sys

import pytest
import torch

from row_wise_normalization_rmsnorm_amd import binding as B
from row_wise_normalization_rmsnorm_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DTYPES = ["f32", "f16", "bf16"]
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# (data, gamma, output): gamma in the data dtype or fp32; every output dtype
COMBOS = [(d, g, o) for d in DTYPES for g in sorted({d, "f32"}) for o in DTYPES]
# (hidden, k, layout, rows): register path (16-byte chunks, several rows per
# wave, one row per workgroup), element and 8/4-byte chunks from odd pitches,
# and the streaming path (LDS-staged)
CASES = [(64, 2, "pad16", 200), (1592, 0, "contig", 37), (4096, 1, "pad16", 33),
         (7, 3, "odd", 41), (3000, 3, "odd", 19), (20000, 1, "pad16", 9)]
PADS = {"contig": (0, 0, 0), "pad16": (16, 32, 48), "odd": (3, 5, 2)}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Embedded:
    """A [rows, hidden] view at column `off` of a [rows, hidden + pad] buffer
    filled with a sentinel; `outside_intact()` checks the sentinel."""

    def __init__(self, src, dtype, pad, off=0, fill=None):
        rows, hidden = src.shape if src is not None else fill
        self.buf = torch.full((rows, hidden + pad), -7.0, dtype=TD[dtype], device=DEV)
        self.view = self.buf[:, off:off + hidden]
        self.off, self.hidden = off, hidden
        if src is not None:
            self.view.copy_(src.to(DEV))
        else:
            self.view.fill_(float("nan"))

    def outside_intact(self):
        b = self.buf.cpu().float()
        keep = torch.ones_like(b, dtype=torch.bool)
        keep[:, self.off:self.off + self.hidden] = False
        return bool((b[keep] == -7.0).all())


def _run(d, g, o, hidden, k, layout, rows, seed):
    w = I.case(d, rows, hidden, k, seed=seed, std=0.6)
    inp = I.make_inputs(w)
    gamma = I.gamma(w, DEV, dtype=g)
    pin, pout, pres = PADS[layout]
    off = 1 if layout == "odd" else 0
    out = Embedded(None, o, pout, off, fill=(rows, hidden))
    plan = B.rmsnorm_plan_ex(rows, hidden, k, d, g, o)
    say(f"[gpu] general {d},g={g},o={o} H={hidden} k={k} {layout}: contiguous plan {plan}")
    if k:
        parts = [Embedded(p, d, pin + 8 * j, off) for j, p in enumerate(inp["partials"])]
        res = Embedded(inp["residual"], d, pres, off)
        B.add_rmsnorm_fwd_ex(out.view, res.view, [p.view for p in parts], gamma, w.eps)
    else:
        parts = [Embedded(inp["x"], d, pin, off)]
        res = None
        B.rmsnorm_fwd_ex(out.view, parts[0].view, gamma, w.eps)
    torch.cuda.synchronize()
    ref = P.run_oracle(d, w.eps, x=inp.get("x"), partials=inp.get("partials"),
                       residual=inp.get("residual"), gamma=gamma.cpu(), out_dtype=o)
    stats = P.compare(o, out.view.cpu().contiguous(), ref,
                      res.view.cpu().contiguous() if res else None,
                      what=f"{d},g={g},o={o} H={hidden} k={k} {layout}", res_dtype=d)
    assert out.outside_intact(), "write outside the output rows"
    for t in parts + ([res] if res else []):
        assert t.outside_intact(), "write outside an input's rows"
    if not k:
        assert torch.equal(parts[0].view.cpu(), inp["x"]), "x modified"
    return stats


@pytest.mark.parametrize("d,g,o", COMBOS)
def test_general_combinations(d, g, o):
    for i, (hidden, k, layout, rows) in enumerate(CASES):
        _run(d, g, o, hidden, k, layout, rows, seed=100 + i)


def test_nd_views_collapse_to_one_row_stride():
    w = I.case("bf16", 12, 1000, 2, seed=7)
    inp = I.make_inputs(w)
    big = [torch.full((6, 4, 1016), -7.0, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    views = [b[1:4, :, 8:1008] for b in big]          # [3, 4, 1000], row stride 1016
    for v, t in zip(views, inp["partials"] + [inp["residual"]]):
        v.copy_(t.view(3, 4, 1000).to(DEV))
    out = torch.empty(3, 4, 1000, dtype=torch.float32, device=DEV)
    assert B.row_view(views[0], "x") == (12, 1000, 1016)
    B.add_rmsnorm_fwd_ex(out, views[2], views[:2], I.gamma(w, DEV), w.eps)
    torch.cuda.synchronize()
    ref = P.run_oracle("bf16", w.eps, partials=inp["partials"], residual=inp["residual"],
                       gamma=I.gamma(w), out_dtype="f32")
    P.compare("f32", out.view(12, 1000).cpu(), ref, views[2].reshape(12, 1000).cpu(),
              what="N-D views", res_dtype="bf16")
    with pytest.raises(B.RmsnormError):
        B.row_view(big[0].transpose(0, 1)[:, :, :1000], "x")   # leading dims do not collapse


def test_interleaved_rows_of_one_buffer():
    """x and out are alternate halves of each row of one buffer: equal
    pitches, no shared byte, so the call is legal."""
    w = I.case("f16", 50, 2048, 0, seed=9)
    x = I.make_inputs(w)["x"]
    buf = torch.empty(50, 4096, dtype=torch.float16, device=DEV)
    buf[:, :2048].copy_(x.to(DEV))
    buf[:, 2048:].fill_(float("nan"))
    B.rmsnorm_fwd_ex(buf[:, 2048:], buf[:, :2048], I.gamma(w, DEV), w.eps)
    torch.cuda.synchronize()
    ref = P.run_oracle("f16", w.eps, x=x, gamma=I.gamma(w))
    P.compare("f16", buf[:, 2048:].cpu().contiguous(), ref, what="interleaved")
    assert torch.equal(buf[:, :2048].cpu(), x)


def test_in_place_strided_and_alias_errors():
    w = I.case("bf16", 20, 512, 1, seed=11)
    inp = I.make_inputs(w)
    p = Embedded(inp["partials"][0], "bf16", 24)
    r = Embedded(inp["residual"], "bf16", 24)
    B.add_rmsnorm_fwd_ex(p.view, r.view, [p.view], I.gamma(w, DEV, dtype="f32"), w.eps)
    torch.cuda.synchronize()
    ref = P.run_oracle("bf16", w.eps, partials=inp["partials"], residual=inp["residual"],
                       gamma=I.gamma(w, dtype="f32"))
    P.compare("bf16", p.view.cpu().contiguous(), ref, r.view.cpu().contiguous(), what="in place")
    # out over its input with another dtype, or shifted by one element: refused
    buf = torch.zeros(20, 1024, dtype=torch.float32, device=DEV)
    x = buf[:, :512]
    g = torch.ones(512, dtype=torch.float32, device=DEV)
    with pytest.raises(B.RmsnormError) as e:
        B.rmsnorm_fwd_ex(buf.view(torch.bfloat16)[:, :512], x, g, 1e-6)
    assert e.value.code == -5
    with pytest.raises(B.RmsnormError) as e:
        B.rmsnorm_fwd_ex(buf[:, 1:513], x, g, 1e-6)
    assert e.value.code == -5
    with pytest.raises(B.RmsnormError) as e:       # gamma fp16 with bf16 data
        B.rmsnorm_fwd_ex(torch.empty(20, 512, dtype=torch.bfloat16, device=DEV),
                         torch.zeros(20, 512, dtype=torch.bfloat16, device=DEV),
                         torch.ones(512, dtype=torch.float16, device=DEV), 1e-6)
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert int(buf.count_nonzero()) == 0           # nothing was launched


def test_convenience_wrappers_pick_the_general_form():
    w = I.case("bf16", 16, 768, 0, seed=13)
    x = I.make_inputs(w)["x"].to(DEV)
    y = B.rmsnorm(x[:, :], I.gamma(w, DEV, dtype="f32"), w.eps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = P.run_oracle("bf16", w.eps, x=x.cpu(), gamma=I.gamma(w, dtype="f32"), out_dtype="f32")
    P.compare("f32", y.cpu(), ref, what="wrapper")


@pytest.mark.parametrize("d,g,o", [c for c in COMBOS if not (c[0] == c[1] == c[2])])
def test_every_mixed_variant(d, g, o, monkeypatch):
    """Every compiled variant of each general combination, forced through
    rmsnorm_tune on a case it can run (contiguous rows)."""
    names = B.rmsnorm_variants_ex(d, g, o)
    assert names
    say(f"[gpu] {len(names)} variants of {d},g={g},o={o}")
    for i, name in enumerate(names):
        hidden, rows, k = P.variant_case(d, name)
        w = I.case(d, rows, hidden, k, seed=i, std=0.5)
        B.tune(name)
        assert B.rmsnorm_plan_ex(rows, hidden, k, d, g, o) == name
        inp = I.make_inputs(w)
        gamma = I.gamma(w, DEV, dtype=g)
        out = torch.full((rows, hidden), float("nan"), dtype=TD[o], device=DEV)
        res = None
        if k:
            res = inp["residual"].to(DEV)
            B.add_rmsnorm_fwd_ex(out, res, [p.to(DEV) for p in inp["partials"]], gamma, w.eps)
        else:
            B.rmsnorm_fwd_ex(out, inp["x"].to(DEV), gamma, w.eps)
        torch.cuda.synchronize()
        ref = P.run_oracle(d, w.eps, x=inp.get("x"), partials=inp.get("partials"),
                           residual=inp.get("residual"), gamma=gamma.cpu(), out_dtype=o)
        P.compare(o, out.cpu(), ref, res.cpu() if k else None, what=f"variant {name}", res_dtype=d)
    B.tune(None)


def test_random_general_calls():
    """Seeded random calls of the general interface: dtype triple, shape, K,
    a pad (row pitch) and a base offset for every tensor independently."""
    import numpy as np
    rng = np.random.default_rng(77)
    for t in range(60):
        d, g, o = COMBOS[int(rng.integers(len(COMBOS)))]
        hidden = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 9000)),
                                 int(rng.integers(9000, 30000))], p=[0.35, 0.5, 0.15]))
        if rng.random() < 0.5:
            hidden = max(8, hidden // 8 * 8)
        k = int(rng.choice([0, 1, 2, 5]))
        rows = int(rng.integers(1, 60))
        rows = max(1, min(rows, (2 << 20) // (hidden * (k + 2))))
        w = I.case(d, rows, hidden, k, seed=1000 + t, std=float(rng.choice([0.3, 1.0, 20.0])),
                   eps=float(rng.choice([1e-6, 1e-5])))
        inp = I.make_inputs(w)
        gamma = I.gamma(w, DEV, dtype=g)

        def emb(src, dt, fill=None):
            pad = int(rng.choice([0, int(rng.integers(1, 40)), 8 * int(rng.integers(1, 6))]))
            off = int(rng.choice([0, 0, int(rng.integers(0, pad + 1))]))
            return Embedded(src, dt, pad, off, fill=fill)

        out = emb(None, o, fill=(rows, hidden))
        what = f"random general #{t}: {d},g={g},o={o} rows={rows} H={hidden} k={k}"
        say(f"[gpu] {what}")
        if k:
            parts = [emb(p, d) for p in inp["partials"]]
            res = emb(inp["residual"], d)
            B.add_rmsnorm_fwd_ex(out.view, res.view, [p.view for p in parts], gamma, w.eps)
        else:
            parts, res = [emb(inp["x"], d)], None
            B.rmsnorm_fwd_ex(out.view, parts[0].view, gamma, w.eps)
        torch.cuda.synchronize()
        ref = P.run_oracle(d, w.eps, x=inp.get("x"), partials=inp.get("partials"),
                           residual=inp.get("residual"), gamma=gamma.cpu(), out_dtype=o)
        P.compare(o, out.view.cpu().contiguous(), ref,
                  res.view.cpu().contiguous() if res else None, what=what, res_dtype=d)
        assert out.outside_intact() and all(p.outside_intact() for p in parts), what
        assert res is None or res.outside_intact(), what
