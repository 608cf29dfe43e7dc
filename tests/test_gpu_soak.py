"""Seeded random soaks of the three GPU paths against their oracles, long
runs of the same checks the other GPU tests apply (marked slow: they run
only with RMSNORM_SLOW_TESTS=1).  Each stops at its first failure and names
the case; every case is reproducible from its seed and index.

Command:
    RMSNORM_SLOW_TESTS=1 python -u -m pytest tests/test_gpu_soak.py -m gpu -x -v -s
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from row_wise_normalization_rmsnorm_amd import binding as B
from row_wise_normalization_rmsnorm_amd import inputs as I
from tests import test_gpu_allgather as AG
from tests import test_gpu_gemm_scatter as G
from tests.test_gpu_parity import check, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

RMSNORM_CASES, RMSNORM_SEED = 1800, 9001
GEMM_CASES, GEMM_SEED = 620, 9002
AG_CASES, AG_SEED = 300, 9003


def test_soak_rmsnorm():
    """Plain and fused RMSNorm: dtype, hidden 1-70000 (half the time a
    multiple of 8), K 0-16, eps 0-1e-2, inputs scaled 0.01-30, up to 4 Mi
    input elements per case."""
    rng = np.random.default_rng(RMSNORM_SEED)
    for t in range(RMSNORM_CASES):
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        hidden = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 9000)),
                                 int(rng.integers(9000, 70001))], p=[0.35, 0.45, 0.2]))
        if rng.random() < 0.5:
            hidden = max(8, hidden // 8 * 8)
        k = int(rng.integers(0, 17))
        rows = int(rng.integers(1, 80))
        rows = max(1, min(rows, (4 << 20) // (hidden * (k + 1))))
        eps = float(rng.choice([0.0, 1e-6, 1e-5, 1e-2]))
        std = float(rng.choice([0.01, 0.3, 1.0, 30.0]))
        if dtype == "f16":
            std = min(std, 1.0)       # keep fp16 sums of squares of the rows finite
        w = I.case(dtype, rows, hidden, k, seed=RMSNORM_SEED * 10000 + t, std=std, eps=eps)
        check(w, I.make_inputs(w), f"rmsnorm soak #{t} ({dtype} rows={rows} hidden={hidden} "
                                   f"k={k} eps={eps} std={std})")


def test_soak_gemm_scatter():
    """GEMM with the scatter epilogue: dtype, ragged m, n and k (k from 0),
    world 1-16 and rank, alpha, beta, optional C, padded strides, both
    output alignments, every tile width and every tile height."""
    rng = np.random.default_rng(GEMM_SEED)
    for i in range(GEMM_CASES):
        dtype = str(rng.choice(["bf16", "f16"]))
        world = int(rng.choice([1, 2, 3, 4, 8, 16]))
        m = world * int(rng.integers(1, max(2, 1100 // world)))
        n = int(rng.integers(1, 1400))
        k = 8 * int(rng.integers(0, 80))
        with_c = bool(rng.random() < 0.5)
        alpha = float(np.float32(rng.choice([1.0, -0.5, 1.75])))
        beta = float(np.float32(rng.choice([0.0, 1.0, -2.0]))) if with_c else 0.0
        rank = int(rng.integers(world))
        pads = [int(8 * rng.integers(0, 3)) for _ in range(2)]
        a, b, c = G.make(dtype, m, n, k, with_c, seed=GEMM_SEED * 10000 + i, lda_pad=pads[0],
                         ldb_pad=pads[1], ldc_pad=int(rng.integers(0, 5)))
        if k == 0:
            a, b = a.contiguous(), b.contiguous()
        col = int(rng.choice([4, 8]))
        pad = (-(n + 8 + col)) % 8 if col == 8 else int(rng.integers(0, 4))
        tile_n = int(rng.choice((0,) + G.WIDTHS))
        tile_m = int(rng.choice((0, 256, 192, 160)))
        what = (f"gemm soak #{i} ({dtype} m={m} n={n} k={k} world={world} rank={rank} "
                f"c={with_c} col={col} tile_n={tile_n} tile_m={tile_m})")
        say(f"[gpu] {what}")
        got, _ = G.run(a, b, c, alpha, beta, world, rank=rank, ldd_pad=pad, col=col, tile_n=tile_n,
                       tile_m=tile_m)
        want, y, mag = G.oracle_rows(a, b, c, alpha, beta, world, dtype)
        G.compare(got, want, y, mag, k, dtype, what, min_exact=0.5)


def test_soak_allgather():
    """The all-gather epilogue: dtype, K 1-16, 1-16 outputs, hidden
    1-60000, bases shifted by 0-4 elements (narrower chunks)."""
    rng = np.random.default_rng(AG_SEED)
    for t in range(AG_CASES):
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        hidden = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 9000)),
                                 int(rng.integers(9000, 60001))], p=[0.35, 0.45, 0.2]))
        k = int(rng.integers(1, 17))
        nout = int(rng.integers(1, 17))
        rows = max(1, min(int(rng.integers(1, 40)), (2 << 20) // (hidden * (k + nout))))
        shift = int(rng.integers(0, 5))
        w = I.case(dtype, rows, hidden, k, seed=AG_SEED * 10000 + t, std=0.5)
        AG.check_ag(w, I.make_inputs(w), nout, f"all-gather soak #{t} ({dtype} rows={rows} "
                                               f"hidden={hidden} k={k} nout={nout} shift={shift})",
                    shift=shift)
