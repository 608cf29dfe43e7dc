"""Seeded synthetic inputs shared by the GPU path's tests and the oracle.

This module holds none of the method's arithmetic: it only draws random
numbers and rounds them to the storage dtype.  Recipe:

* Every tensor is split into blocks of ``BLOCK_ROWS`` rows.  Block b of tensor
  t of a workload is drawn from its own generator,
  ``numpy.random.Generator(PCG64(SeedSequence([seed, t, b])))``, so any row can
  be regenerated alone, and the result does not depend on threading or on
  how many rows are drawn at once.
* Draws are float32: x and the partials are ``standard_normal * part_std``;
  the residual is ``standard_normal``; gamma is ``uniform(0.5, 1.5)``.
* For workloads with ``special_frac`` > 0, ``floor(special_frac * rows)`` rows
  are scaled by 1e3 and as many other rows are set to +0.0, the same rows in
  x and in the residual (row indices drawn without replacement from their own
  generator; the two sets are disjoint).  Scaling happens in float32.
* The float32 values are rounded to bf16 / fp16 by ``torch.Tensor.to``
  (round to nearest, ties to even).

Tensor ids: partial/x j -> j, residual -> 100, gamma -> 200, special rows -> 300.

GEMM workloads draw A [m, k] (std ``a_std``), B [n, k] (std ``b_std``) and C
[m, n] (std 1) by the same block recipe, with tensor ids 400, 401 and 402.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from .workloads import GemmWorkload, Workload

BLOCK_ROWS = 16
RESIDUAL_ID = 100
GAMMA_ID = 200
SPECIAL_ID = 300
GEMM_A_ID, GEMM_B_ID, GEMM_C_ID = 400, 401, 402

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8_e4m3": torch.float8_e4m3fn, "fp8_e5m2": torch.float8_e5m2, "i8": torch.int8}


def _rng(seed: int, tensor_id: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, block])))


def special_rows(w: Workload):
    """(scaled_rows, zero_rows) as sorted int64 arrays (empty if none)."""
    n = int(w.special_frac * w.rows)
    if n == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    pick = _rng(w.seed, SPECIAL_ID, 0).choice(w.rows, size=2 * n, replace=False)
    return np.sort(pick[:n]).astype(np.int64), np.sort(pick[n:]).astype(np.int64)


def _draw_block(w: Workload, tensor_id: int, block: int, std: float, scaled, zeroed) -> np.ndarray:
    r0 = block * BLOCK_ROWS
    nr = min(BLOCK_ROWS, w.rows - r0)
    if w.dtype == "i8":  # int8 inputs: uniform over the whole int8 range
        return _rng(w.seed, tensor_id, block).integers(-128, 128, (nr, w.hidden), dtype=np.int8)
    a = _rng(w.seed, tensor_id, block).standard_normal((nr, w.hidden), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if scaled is not None:
        for r in scaled[(scaled >= r0) & (scaled < r0 + nr)]:
            a[r - r0] *= np.float32(1e3)
        for r in zeroed[(zeroed >= r0) & (zeroed < r0 + nr)]:
            a[r - r0] = 0.0
    return a


def _to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "i8":
        return torch.from_numpy(a)
    return torch.from_numpy(a).to(TORCH_DTYPE[dtype])


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def tensor_rows(w: Workload, tensor_id: int, rows: Optional[Sequence[int]] = None,
                device: str = "cpu") -> torch.Tensor:
    """Rows of one [rows, hidden] tensor (all rows, or the given row indices,
    in the given order) as a torch tensor of the workload's dtype."""
    std = 1.0 if tensor_id == RESIDUAL_ID else w.part_std
    scaled, zeroed = special_rows(w) if w.special_frac > 0 else (None, None)
    if rows is not None:
        idx = np.asarray(rows, dtype=np.int64)
        out = torch.empty((len(idx), w.hidden), dtype=TORCH_DTYPE[w.dtype])
        cache: Dict[int, np.ndarray] = {}
        for i, r in enumerate(idx):
            b = int(r) // BLOCK_ROWS
            if b not in cache:
                cache[b] = _draw_block(w, tensor_id, b, std, scaled, zeroed)
            out[i] = _to_dtype(cache[b][int(r) - b * BLOCK_ROWS].copy(), w.dtype)
        return out.to(device)

    out = torch.empty((w.rows, w.hidden), dtype=TORCH_DTYPE[w.dtype], device=device)
    nblocks = (w.rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    # Blocks are drawn in parallel (numpy releases the GIL while filling) and
    # copied out in chunks, so the full-size tensors never exist in float32.
    chunk_blocks = max(1, (1 << 24) // (BLOCK_ROWS * w.hidden))
    with cf.ThreadPoolExecutor(_threads()) as ex:
        for c0 in range(0, nblocks, chunk_blocks):
            blocks = range(c0, min(nblocks, c0 + chunk_blocks))
            parts = list(ex.map(lambda b: _draw_block(w, tensor_id, b, std, scaled, zeroed), blocks))
            a = np.concatenate(parts, axis=0)
            r0 = c0 * BLOCK_ROWS
            out[r0:r0 + a.shape[0]].copy_(_to_dtype(a, w.dtype))
    return out


def gamma(w: Workload, device: str = "cpu", dtype: Optional[str] = None) -> torch.Tensor:
    """gamma[hidden] ~ U(0.5, 1.5), drawn in float32 and rounded to ``dtype``
    (default: the workload's dtype; "f32" keeps the full draw)."""
    a = _rng(w.seed, GAMMA_ID, 0).uniform(0.5, 1.5, w.hidden).astype(np.float32)
    return _to_dtype(a, dtype or w.dtype).to(device)


def make_inputs(w: Workload, rows: Optional[Sequence[int]] = None, device: str = "cpu") -> Dict:
    """All inputs of a workload: {"x": tensor} for plain RMSNorm, or
    {"partials": [tensors], "residual": tensor} for the fused form; plus
    {"gamma": tensor}.  ``rows`` restricts to those row indices."""
    d: Dict = {"gamma": gamma(w, device)}
    if w.fused:
        d["partials"] = [tensor_rows(w, j, rows, device) for j in range(w.k)]
        d["residual"] = tensor_rows(w, RESIDUAL_ID, rows, device)
    else:
        d["x"] = tensor_rows(w, 0, rows, device)
    return d


def to_storage(t: torch.Tensor) -> np.ndarray:
    """A CPU tensor's storage as numpy: float32 values, uint16 bit patterns
    for fp16 / bf16, uint8 codes for fp8, int8 for int8 (the oracle's array
    convention)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32 or t.dtype == torch.int8:
        return t.numpy()
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def from_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of ``to_storage``."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(TORCH_DTYPE[dtype])


def storage_list(ts: List[torch.Tensor]) -> List[np.ndarray]:
    return [to_storage(t) for t in ts]


def case(dtype: str, rows: int, hidden: int, k: int = 0, seed: int = 1, std: float = 1.0,
         eps: float = 1e-6) -> Workload:
    """An ad-hoc seeded test case with the workloads' value distributions
    (k = 0: plain RMSNorm, else k partials plus a residual)."""
    return Workload(f"case_{dtype}_{rows}x{hidden}_k{k}_s{seed}",
                    "add_rmsnorm" if k else "rmsnorm", dtype, rows, hidden, k, eps, std,
                    seed=seed)


def device_tensor(w: Workload, tensor_id: int, device: str) -> torch.Tensor:
    """A [rows, hidden] tensor drawn directly on the device by torch's own
    seeded generator (keyed by seed and tensor id): for sizes too large to
    draw on the host in reasonable time.  Same distributions as above, but
    not the same numbers as ``tensor_rows``."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1_000_003 + tensor_id)
    std = 1.0 if tensor_id == RESIDUAL_ID else w.part_std
    out = torch.empty((w.rows, w.hidden), dtype=TORCH_DTYPE[w.dtype], device=device)
    step = max(1, (1 << 26) // w.hidden)
    for r0 in range(0, w.rows, step):
        a = torch.randn((min(step, w.rows - r0), w.hidden), generator=g, device=device,
                        dtype=torch.float32)
        out[r0:r0 + a.shape[0]].copy_(a.mul_(std))
    return out


def matrix(seed: int, tensor_id: int, rows: int, cols: int, std: float, dtype: str,
           row_idx: Optional[Sequence[int]] = None, device: str = "cpu") -> torch.Tensor:
    """A seeded [rows, cols] matrix by the block recipe (N(0, std^2))."""
    w = Workload(f"matrix_{tensor_id}", "matrix", dtype, rows, cols, 0, 0.0, std, seed=seed)
    return tensor_rows(w, tensor_id, row_idx, device)


def gemm_inputs(w: GemmWorkload, device: str = "cpu") -> Dict:
    """{"a": [m, k], "b": [n, k], "c": [m, n] or None} of a GEMM workload."""
    return {"a": matrix(w.seed, GEMM_A_ID, w.m, w.k, w.a_std, w.dtype, device=device),
            "b": matrix(w.seed, GEMM_B_ID, w.n, w.k, w.b_std, w.dtype, device=device),
            "c": matrix(w.seed, GEMM_C_ID, w.m, w.n, 1.0, w.dtype, device=device)
            if w.with_c else None}
