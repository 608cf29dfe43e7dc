"""Oracle pins at the workloads' own shapes and seeded inputs.

On every workload (all rows of the 512-row ones, a seeded row sample of the
larger ones):
  * the oracle's unrounded y equals torch's float64 RMSNorm (the definition
    page "RMSNorm kernel" links in section 1 Background) of the row it
    normalised, within 1e-12 relative;
  * its rounded y is that value rounded once (torch / numpy converters);
  * in the fused form, the residual equals numpy's binary32 sum
    p_0 + ... + p_{K-1} + r rounded by torch, byte for byte (page "Tokenweave
    fused-RMSNorm-AR kernel", "Code walkthrough").
It also fingerprints the input generator (SHA-256 of the seeded bytes).
"""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
from row_wise_normalization_rmsnorm_amd import inputs as I
from row_wise_normalization_rmsnorm_amd.workloads import RMSNORM_WORKLOADS, WORKLOADS
from tests import independent as ind

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _rows_for(w):
    """All rows of the small workloads; of the large ones, the first and last
    16 rows, a seeded random sample, and (where present) special rows."""
    if w.rows * w.hidden <= 4 * 1024 * 1024:
        return None
    rng = np.random.default_rng(w.rows)
    pick = set(range(16)) | set(range(w.rows - 16, w.rows))
    pick |= set(rng.choice(w.rows, size=96, replace=False).tolist())
    scaled, zeroed = I.special_rows(w)
    pick |= set(scaled[:4].tolist()) | set(zeroed[:4].tolist())
    return sorted(pick)


@pytest.mark.parametrize("name", RMSNORM_WORKLOADS)
def test_oracle_matches_definition_on_workload(name):
    w = WORKLOADS[name]
    rows = _rows_for(w)
    d = I.make_inputs(w, rows=rows)
    g = I.to_storage(d["gamma"])
    if w.fused:
        ps = I.storage_list(d["partials"])
        r = I.to_storage(d["residual"])
        out, rnew, rstd, y = oracle.add_rmsnorm(ps, r, g, w.eps, w.dtype, want_f64=True)
        # residual: binary32 sequential sum, rounded once by torch
        acc = d["partials"][0].float()
        for p in d["partials"][1:]:
            acc = acc + p.float()
        acc = acc + d["residual"].float()
        want_r = I.to_storage(acc.to(TORCH[w.dtype]))
        assert np.array_equal(rnew, want_r)
        v = ind.decode_np(rnew, w.dtype)
    else:
        x = I.to_storage(d["x"])
        out, rstd, y = oracle.rmsnorm(x, g, w.eps, w.dtype, want_f64=True)
        v = ind.decode_np(x, w.dtype)
    H = w.hidden
    ref = torch.nn.functional.rms_norm(torch.from_numpy(v), [H],
                                       torch.from_numpy(ind.decode_np(g, w.dtype)),
                                       float(np.float32(w.eps))).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)
    # the rounding step: single rounding from double
    if w.dtype == "f16":
        want_out = y.astype(np.float16).view(np.uint16)
    elif w.dtype == "f32":
        want_out = y.astype(np.float32)
    else:
        want_out = None  # bf16: checked through exact rounding on a sample below
    if want_out is not None:
        assert np.array_equal(out.view(np.uint16 if w.dtype == "f16" else np.uint32),
                              want_out.view(np.uint16 if w.dtype == "f16" else np.uint32))
    else:
        from fractions import Fraction
        flat_y, flat_o = y.ravel(), out.ravel()
        idx = np.random.default_rng(0).choice(flat_y.size, size=min(4000, flat_y.size), replace=False)
        for j in idx:
            want, _ = ind.round_signed(Fraction(float(flat_y[j])), float(flat_y[j]), "bf16")
            assert int(flat_o[j]) == ind.bits(want, "bf16")
    if w.special_frac:
        _, zeroed = I.special_rows(w)
        for i, row in enumerate(rows):
            if row in set(zeroed.tolist()):
                assert np.all(v[i] == 0) and np.all(y[i] == 0)


def _fingerprint(w):
    rows = list(range(min(w.rows, 48))) + [w.rows - 1]
    d = I.make_inputs(w, rows=rows)
    h = hashlib.sha256()
    for t in ([d["x"]] if not w.fused else d["partials"] + [d["residual"]]) + [d["gamma"]]:
        h.update(I.to_storage(t).tobytes())
    return h.hexdigest()


def _gemm_fingerprint(w):
    """rows 0..47 and the last row of a GEMM workload's A and B (and C)."""
    h = hashlib.sha256()
    for tid, rows, cols, std in ((I.GEMM_A_ID, w.m, w.k, w.a_std), (I.GEMM_B_ID, w.n, w.k, w.b_std)) + \
            (((I.GEMM_C_ID, w.m, w.n, 1.0),) if w.with_c else ()):
        idx = list(range(min(rows, 48))) + [rows - 1]
        h.update(I.to_storage(I.matrix(w.seed, tid, rows, cols, std, w.dtype, row_idx=idx)).tobytes())
    return h.hexdigest()


def test_input_generator_fingerprint():
    """The seeded inputs are the recorded ones (tests/golden/input_fingerprints.json,
    written by tests/golden/make_input_fingerprints.py)."""
    with open(os.path.join(GOLDEN, "input_fingerprints.json")) as f:
        want = json.load(f)["fingerprints"]
    for name, w in WORKLOADS.items():
        assert _fingerprint(w) == want[name], name


def test_gemm_input_generator_fingerprint():
    """The GEMM workloads' seeded operands are the recorded ones (same file)."""
    from row_wise_normalization_rmsnorm_amd.workloads import GEMM_WORKLOADS
    with open(os.path.join(GOLDEN, "input_fingerprints.json")) as f:
        want = json.load(f)["gemm_fingerprints"]
    assert set(want) == set(GEMM_WORKLOADS)
    for name, w in GEMM_WORKLOADS.items():
        assert _gemm_fingerprint(w) == want[name], name


def test_generator_rows_subset_equals_full():
    w = WORKLOADS["rmsnorm_bf16_512x1592"]
    full = I.make_inputs(w)["x"]
    rows = [0, 15, 16, 17, 300, 511]
    sub = I.make_inputs(w, rows=rows)["x"]
    assert torch.equal(full[rows], sub)


def test_special_rows_recipe():
    w = WORKLOADS["add_rmsnorm_bf16_65536x16384_k1"]
    scaled, zeroed = I.special_rows(w)
    assert len(scaled) == len(zeroed) == 655
    assert not set(scaled.tolist()) & set(zeroed.tolist())
    d = I.make_inputs(w, rows=[int(zeroed[0]), int(scaled[0])])
    for t in d["partials"] + [d["residual"]]:
        assert torch.all(t[0] == 0)
        assert t[1].float().abs().max() > 100
