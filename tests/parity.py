"""Comparison of the HIP path with the oracle (test helper).

The bar (written here once, used by every GPU parity test):
  * residual (fused form): byte-for-byte equal to the oracle's;
  * out, fp32: |gpu - o| <= 1e-5 * |o| elementwise, o the oracle's unrounded
    double value; o == 0 requires gpu == 0;
  * out, fp16 / bf16: at most 2 units in the last place from the oracle's
    once-rounded value;
  * NaN positions identical.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle
from row_wise_normalization_rmsnorm_amd import inputs as I
from tests import independent as ind

F32_REL_TOL = 1e-5
HALF_ULP_TOL = 2


def storage(t) -> np.ndarray:
    """dtype storage of a torch tensor (numpy arrays pass through)."""
    return t if isinstance(t, np.ndarray) else I.to_storage(t)


GAMMA_NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def run_oracle(dtype: str, eps: float, x=None, partials=None, residual=None, gamma=None,
               out_dtype: str = None):
    """Oracle on CPU copies of torch tensors (gamma in its own dtype; the
    output in out_dtype, default dtype).  Returns dict with out, y64,
    (residual)."""
    g = storage(gamma)
    kw = dict(gamma_dtype=GAMMA_NAME[gamma.dtype], out_dtype=out_dtype or dtype, want_f64=True)
    if partials is None:
        out, _, y64 = oracle.rmsnorm(storage(x), g, eps, dtype, **kw)
        return {"out": out, "y64": y64}
    out, rnew, _, y64 = oracle.add_rmsnorm([storage(p) for p in partials], storage(residual), g,
                                           eps, dtype, **kw)
    return {"out": out, "y64": y64, "residual": rnew}


def compare(dtype: str, gpu_out: torch.Tensor, ref: dict, gpu_residual: torch.Tensor = None,
            what: str = "", res_dtype: str = None) -> dict:
    """Assert the bar; return error statistics.  dtype is the output's dtype;
    res_dtype the residual's (default: the same)."""
    go = storage(gpu_out)
    stats = {}
    res_dtype = res_dtype or dtype
    if gpu_residual is not None:
        gr = storage(gpu_residual)
        same = np.array_equal(gr.view(np.uint8), ref["residual"].view(np.uint8))
        if not same:
            wide = np.uint32 if res_dtype == "f32" else np.uint16
            bad = np.argwhere(gr.view(wide) != ref["residual"].view(wide))
            raise AssertionError(f"{what}: residual differs at {len(bad)} elements, first {bad[:4].tolist()}")
        stats["residual_bit_exact"] = True
    y64 = ref["y64"]
    gv = ind.decode_np(go, dtype)
    nan_g, nan_o = np.isnan(gv), np.isnan(y64)
    assert np.array_equal(nan_g, nan_o), f"{what}: NaN positions differ ({nan_g.sum()} vs {nan_o.sum()})"
    ok = ~nan_o
    if dtype == "f32":
        o = y64[ok]
        g = gv[ok]
        zero = o == 0
        assert np.all(g[zero] == 0), f"{what}: nonzero output where the oracle is 0"
        rel = np.abs(g[~zero] - o[~zero]) / np.abs(o[~zero]) if (~zero).any() else np.zeros(1)
        mx = float(rel.max()) if rel.size else 0.0
        if mx > F32_REL_TOL:
            j = int(np.argmax(rel))
            raise AssertionError(f"{what}: fp32 rel err {mx:.3g} > {F32_REL_TOL} (gpu {g[~zero][j]!r} "
                                 f"oracle {o[~zero][j]!r})")
        stats["max_rel_err"] = mx
    else:
        ulps = ind.ulp_distance(go[ok], ref["out"][ok], dtype)
        mx = int(ulps.max()) if ulps.size else 0
        if mx > HALF_ULP_TOL:
            j = int(np.argmax(ulps))
            raise AssertionError(f"{what}: {mx} ulp > {HALF_ULP_TOL} at flat {j} (gpu bits "
                                 f"{int(go[ok][j]):#06x}, oracle {int(ref['out'][ok][j]):#06x})")
        stats["max_ulp"] = mx
        stats["frac_not_equal"] = float((ulps > 0).mean()) if ulps.size else 0.0
        nz = y64[ok] != 0
        if nz.any():
            stats["max_rel_err"] = float((np.abs(gv[ok][nz] - y64[ok][nz]) / np.abs(y64[ok][nz])).max())
    return stats


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compare_whole(dtype: str, eps: float, gpu_out: np.ndarray, gpu_res, gamma: np.ndarray,
                  *, x: np.ndarray = None, partials=None, residual: np.ndarray = None,
                  what: str = "", block_elems: int = 1 << 22, threads: int = 0) -> dict:
    """Every row of a full-size result against the oracle.  All arrays are
    host storage (numpy) of the same [rows, hidden] shape: the GPU's output
    and residual (gpu_res None for the plain form), and the inputs as they
    were before the launch.  The oracle runs over blocks of about
    ``block_elems`` elements, one block per task on the host's threads, and
    each block is compared with ``compare`` as soon as it is computed, so the
    oracle's double-precision output never exists for the whole tensor.
    Returns the statistics over all rows."""
    rows, hidden = gpu_out.shape
    br = max(1, block_elems // hidden)
    blocks = [(a, min(rows, a + br)) for a in range(0, rows, br)]

    def job(b):
        a, z = b
        if partials is None:
            o, _, y64 = oracle.rmsnorm(x[a:z], gamma, eps, dtype, want_f64=True)
            ref = {"out": o, "y64": y64}
            st = compare(dtype, gpu_out[a:z], ref, what=f"{what} rows [{a}, {z})")
        else:
            o, rn, _, y64 = oracle.add_rmsnorm([p[a:z] for p in partials], residual[a:z], gamma,
                                               eps, dtype, want_f64=True)
            ref = {"out": o, "y64": y64, "residual": rn}
            st = compare(dtype, gpu_out[a:z], ref, gpu_res[a:z], what=f"{what} rows [{a}, {z})")
        st["elements"] = (z - a) * hidden
        return st

    with cf.ThreadPoolExecutor(threads or host_threads()) as ex:
        stats = list(ex.map(job, blocks))
    n = sum(s["elements"] for s in stats)
    out = {"rows_checked": rows, "elements_checked": n}
    if gpu_res is not None:
        out["residual_bit_exact"] = all(s.get("residual_bit_exact") for s in stats)
    if dtype == "f32":
        out["max_rel_err"] = max(s["max_rel_err"] for s in stats)
    else:
        out["max_ulp"] = max(s["max_ulp"] for s in stats)
        out["frac_not_equal"] = sum(s["frac_not_equal"] * s["elements"] for s in stats) / n
        rel = [s["max_rel_err"] for s in stats if "max_rel_err" in s]
        if rel:
            out["max_rel_err"] = max(rel)
    return out


# ---- kernel variants ----------------------------------------------------------

def parse_variant(name):
    kind = name.split("<")[0]
    body = name[name.index("<") + 1:-1].split(",")
    kv = dict(p.split("=") for p in body if "=" in p)
    flags = [p for p in body if "=" not in p]
    return kind, flags, {k: (int(v) if v.lstrip("-").isdigit() else v) for k, v in kv.items()}


WIDTH_BYTES = {"vec": 16, "v8": 8, "v4": 4, "elem": 0}


def variant_case(dtype, name):
    """A (hidden, rows, k) that the named variant (over data dtype `dtype`)
    can run, chosen so that a narrower chunk width is also the widest its row
    length allows."""
    kind, flags, kv = parse_variant(name)
    s = 4 if dtype == "f32" else 2
    V = 16 // s
    kc = kv["k"]
    # runtime K: 3 partials; two per step: 4 (one pair, then one alone)
    k = {-1: 3, -2: 4}.get(kc, kc)
    if kind == "vgpr":
        tpr, npt, wg = kv["tpr"], kv["npt"], kv["wg"]
        chunks = max(1, tpr * npt - 3)
        hidden = chunks * V
        rows = 2 * (wg // tpr) + 1
    else:
        vb = WIDTH_BYTES[next(f for f in flags if f in WIDTH_BYTES)]
        base = 3000 if "lds" in flags else (40000 if s == 2 else 20000)
        hidden = base + {16: 0, 8: 8 // s, 4: 4 // s, 0: 1}[vb]
        rows = 5
    return hidden, rows, k
