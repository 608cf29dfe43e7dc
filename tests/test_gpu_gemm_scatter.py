"""GPU parity of the GEMM with a reduce-scatter epilogue (include/gemm_scatter.h)
against the CPU oracle.

Bar (floating point, derived from the arithmetic): the GPU accumulates k
exact products in fp32 on the matrix cores, scales by alpha and adds beta * C
with one fused multiply-add, then rounds once to the 16-bit type.  Against
the oracle's exact value y (double) each element satisfies

    |gpu - y| <= (k + 2) * 2^-24 * mag + 2^-p * |y| + 2^-p * tiny

with mag = |alpha| * sum |a b| + |beta c| (from the oracle), p = 8 for bf16
and 11 for fp16 (half an ulp of the stored value) and tiny the smallest
normal of the type.  Beyond the bound, most elements must equal the oracle's
rounded value exactly (they differ only where the fp32 error straddles a
rounding boundary).  NaN positions and infinities match exactly.  Guard
bands around every output chunk must stay untouched.  Every tile shape (256
or 128 columns; 256, 192 or 160 rows) runs the same products in the same k
order, so their outputs must be bitwise equal.  The benchmark's workloads are
checked whole: every row of every chunk.
"""
from __future__ import annotations

import concurrent.futures as cf
import sys

import numpy as np
import pytest
import torch

import oracle
from row_wise_normalization_rmsnorm_amd import binding as B
from row_wise_normalization_rmsnorm_amd import inputs as I
from row_wise_normalization_rmsnorm_amd.workloads import GEMM_WORKLOADS, GemmWorkload
from tests import independent as ind
from tests.parity import host_threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}
P_BITS = {"bf16": 8, "f16": 11}
TINY = {"bf16": 2.0 ** -126, "f16": 2.0 ** -14}
GUARD = 0x7E5A  # a NaN pattern in both formats: never a computed value here
WIDTHS = (B.GEMM_SCATTER_TILE_N, B.GEMM_SCATTER_TILE_N_NARROW)
# every tile shape (rows, columns): the 256-wide tiles at each height, and
# the 128-wide ones
TILES = ((256, 256), (192, 256), (160, 256), (256, 128))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def st(t: torch.Tensor) -> np.ndarray:
    return I.to_storage(t)


def run(a, b, c, alpha, beta, world, rank=0, ldd_pad=0, flags=None, epoch=0, col=4, tile_n=0,
        tile_m=0):
    """Launch into guarded chunk buffers; returns (assembled [m, n] storage,
    the raw buffer).  Each chunk sits at column ``col`` of a [rows + 2,
    n + ldd_pad + 8 + col] block whose first and last rows and other columns
    are guards.  col = 8 with a row pitch that is a multiple of 8 elements
    gives 16-byte aligned rows (the staged tile stores); col = 4, 8-byte.
    tile_m forces the height of 256-wide tiles (0: automatic)."""
    m, n = a.shape[0], b.shape[0]
    rows = m // world
    width = n + ldd_pad + 8 + col
    buf = torch.full((world, rows + 2, width), GUARD, dtype=torch.int16, device=DEV)
    bufv = buf.view(a.dtype)
    dst = [bufv[q, 1:rows + 1, col:col + n] for q in range(world)]
    with B.gemm_tile_m(tile_m):
        B.gemm_scatter_fwd(dst, a, b, c, alpha, beta, rank, flags, epoch, tile_n=tile_n)
    torch.cuda.synchronize()
    host = buf.cpu()
    inner = host[:, 1:rows + 1, col:col + n]
    guard = host.clone()
    guard[:, 1:rows + 1, col:col + n] = GUARD
    assert bool((guard == GUARD).all()), "a write landed outside the output chunks"
    return inner.reshape(m, n).numpy().view(np.uint16), host


def oracle_rows(a, b, c, alpha, beta, world, dtype, rows=None):
    ac, bc = st(a.cpu()), st(b.cpu())
    cc = st(c.cpu()) if c is not None else None
    chunks, y, mag = oracle.gemm_scatter(ac, bc, cc, alpha, beta, world, dtype, rows=rows,
                                         want_f64=True)
    full = np.concatenate(chunks, axis=0)
    r0, r1 = rows if rows is not None else (0, full.shape[0])
    return full[r0:r1], y, mag


def compare(got: np.ndarray, want: np.ndarray, y: np.ndarray, mag: np.ndarray, k: int,
            dtype: str, what: str, min_exact: float = 0.8, quiet: bool = False):
    g = ind.decode_np(got, dtype)
    nan_y = np.isnan(y)
    assert np.array_equal(np.isnan(g), nan_y), f"{what}: NaN positions differ"
    inf_y = np.isinf(y)
    assert np.array_equal(g[inf_y], y[inf_y]), f"{what}: infinities differ"
    fin = ~nan_y & ~inf_y
    bound = (k + 2) * 2.0 ** -24 * mag + 2.0 ** -P_BITS[dtype] * (np.abs(y) + TINY[dtype])
    with np.errstate(invalid="ignore"):
        err = np.abs(g - y)
    bad = fin & ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the bound, first at "
                             f"{tuple(i)}: gpu {g[tuple(i)]!r} exact {y[tuple(i)]!r} "
                             f"bound {bound[tuple(i)]!r}")
    exact = float((got[fin] == want[fin]).mean()) if fin.any() else 1.0
    ratio = float((err[fin] / bound[fin]).max()) if fin.any() else 0.0
    if not quiet:
        say(f"[gpu] {what}: error / bound max {ratio:.3g}, equal to the oracle's rounding "
            f"{100 * exact:.2f}%")
    assert exact >= min_exact, f"{what}: only {exact:.3f} of elements equal the oracle's"
    return ratio, exact


def make(dtype, m, n, k, with_c, seed, lda_pad=0, ldb_pad=0, ldc_pad=0):
    """Seeded operands (A ~ N(0,1), B ~ N(0, 1/(8k)), C ~ N(0,1)), optionally
    as views into wider buffers (row strides k + pad)."""
    w = GemmWorkload("case", dtype, m, n, k, 1, seed=seed)

    def padded(t, pad):
        if not pad:
            return t.to(DEV)
        big = torch.zeros(t.shape[0], t.shape[1] + pad, dtype=t.dtype, device=DEV)
        big[:, :t.shape[1]] = t.to(DEV)
        return big[:, :t.shape[1]]

    a = I.matrix(seed, I.GEMM_A_ID, m, k, w.a_std, dtype) if k else torch.zeros(m, 0, dtype=TORCH[dtype])
    b = I.matrix(seed, I.GEMM_B_ID, n, k, w.b_std if k else 1.0, dtype) if k else torch.zeros(n, 0, dtype=TORCH[dtype])
    c = I.matrix(seed, I.GEMM_C_ID, m, n, 1.0, dtype) if with_c else None
    return padded(a, lda_pad), padded(b, ldb_pad), (padded(c, ldc_pad) if c is not None else None)


SHAPES = [  # m, n, k, world, with_c
    (512, 768, 256, 8, False),
    (776, 300, 136, 8, True),      # ragged m, n and k; chunks of 97 rows
    (256, 256, 64, 1, False),      # one tile
    (8, 40, 8, 2, True),           # far below one tile
    (64, 1000, 72, 2, False),
    (1024, 512, 1024, 4, True),
    (768, 520, 8, 16, True),       # the most chunks (16, of 48 rows), one 8-wide k chunk
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}w{s[3]}{'c' if s[4] else ''}"
                                               for s in SHAPES])
def test_parity(dtype, shape):
    """Each shape at every tile shape (both widths, the 256-wide tiles at
    each height), with 8-byte and with 16-byte aligned output rows (the
    interior tiles of the latter take the LDS-staged stores)."""
    m, n, k, world, with_c = shape
    a, b, c = make(dtype, m, n, k, with_c, seed=m + n + k)
    alpha, beta = (0.5, -1.25) if with_c else (1.0, 0.0)
    want, y, mag = oracle_rows(a, b, c, alpha, beta, world, dtype)
    first = None
    for tile_m, tile_n in TILES:
        for col, pad in ((4, 0), (8, (-(n + 16)) % 8)):
            say(f"[gpu] gemm_scatter {dtype} m={m} n={n} k={k} world={world} c={with_c} "
                f"col={col} tile {tile_m}x{tile_n}")
            got, _ = run(a, b, c, alpha, beta, world, rank=world - 1, ldd_pad=pad, col=col,
                         tile_n=tile_n, tile_m=tile_m)
            compare(got, want, y, mag, k, dtype, f"{dtype} {shape} col {col} tile {tile_m}x{tile_n}")
            if first is None:
                first = got
            assert np.array_equal(got, first), "tile shapes or store paths differ"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_k_around_whole_steps(dtype):
    """k around multiples of the 64-wide k step.  Both kernels load the k
    steps that lie wholly inside k with global loads and the last, partial
    step (and the steps past the end, which must read as zeros) with
    range-checked buffer loads, in two loops; the boundary moves with k.
    The wide kernel loads up to two steps ahead into a ring of five operand
    slots, so k from one step to seven whole steps (and one past) covers
    every way the ring's prologue and its two loops split.  Ragged and whole
    tiles, every tile shape against the oracle and bitwise equal to each
    other."""
    for m, n, world in ((264, 520, 2), (512, 512, 4)):
        for k in (8, 56, 64, 72, 120, 128, 136, 184, 192, 200, 256, 264, 320, 384, 448, 456):
            a, b, c = make(dtype, m, n, k, False, seed=k + m)
            want, y, mag = oracle_rows(a, b, c, 1.0, 0.0, world, dtype)
            first = None
            for tile_m, tile_n in TILES:
                say(f"[gpu] k steps {dtype} m={m} n={n} k={k} tile {tile_m}x{tile_n}")
                got, _ = run(a, b, c, 1.0, 0.0, world, ldd_pad=(-(n + 16)) % 8, col=8,
                             tile_n=tile_n, tile_m=tile_m)
                compare(got, want, y, mag, k, dtype, f"{dtype} {m}x{n}x{k} tile {tile_m}x{tile_n}")
                if first is None:
                    first = got
                assert np.array_equal(got, first), f"tile shapes differ at k = {k}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_strided_operands(dtype):
    """Row strides wider than the rows for A, B, C and the output (one odd,
    which takes the element-wise store path)."""
    m, n, k, world = 384, 264, 200, 4
    for (ldd_pad, ldc_pad), (tile_m, tile_n) in zip(((8, 3), (3, 8), (8, 8), (3, 3)), TILES):
        say(f"[gpu] strided {dtype} ldd_pad={ldd_pad} ldc_pad={ldc_pad} tile {tile_m}x{tile_n}")
        a, b, c = make(dtype, m, n, k, True, seed=7, lda_pad=8, ldb_pad=24, ldc_pad=ldc_pad)
        got, _ = run(a, b, c, 1.5, 0.75, world, rank=1, ldd_pad=ldd_pad, tile_n=tile_n,
                     tile_m=tile_m)
        want, y, mag = oracle_rows(a, b, c, 1.5, 0.75, world, "bf16" if dtype == "bf16" else "f16")
        compare(got, want, y, mag, k, dtype, f"strided {dtype} {ldd_pad}/{ldc_pad}")


def test_empty_products_launch_nothing():
    """m = 0 or n = 0: nothing to compute, nothing written, no error."""
    a = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(128, 64, dtype=torch.bfloat16, device=DEV)
    B.gemm_scatter_fwd([torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)] * 2, a, b)
    a = torch.ones(64, 64, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    sentinel = torch.full((64, 8), 7.0, dtype=torch.bfloat16, device=DEV)
    dst = [sentinel[:32, :0], sentinel[32:, :0]]
    B.gemm_scatter_fwd(dst, a, b)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_broadcast_operands_are_rejected():
    """A broadcast operand (row stride 0) or output rows that overlap are
    turned away before any launch; the output is untouched."""
    row = torch.ones(1, 64, dtype=torch.bfloat16, device=DEV)
    b = torch.ones(128, 64, dtype=torch.bfloat16, device=DEV)
    sentinel = torch.full((64, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    dst = [sentinel[:32], sentinel[32:]]
    for a_, b_ in ((row.expand(64, 64), b), (b[:64], row.expand(128, 64))):
        with pytest.raises(B.RmsnormError):
            B.gemm_scatter_fwd(dst, a_, b_)
    out_row = torch.empty(1, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.RmsnormError):
        B.gemm_scatter_fwd([out_row.expand(32, 128)] * 2, b[:64], b)
    # flags in host memory, or operands in host memory, are refused as well
    host_flags = torch.zeros(B.gemm_scatter_tiles(64, 128), dtype=torch.int32)
    with pytest.raises(B.RmsnormError, match="flags must be a device tensor"):
        B.gemm_scatter_fwd(dst, b[:64], b, flags=host_flags, epoch=1)
    with pytest.raises(B.RmsnormError, match="b must be a device tensor"):
        B.gemm_scatter_fwd(dst, b[:64], b.cpu())
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()) and bool((host_flags == 0).all())


def test_k_zero_gives_beta_c():
    a, b, c = make("bf16", 300, 200, 0, True, seed=3)
    say("[gpu] k = 0")
    got, _ = run(a.contiguous(), b.contiguous(), c, 1.0, -2.0, 4)
    want, y, mag = oracle_rows(a, b, c, 1.0, -2.0, 4, "bf16")
    compare(got, want, y, mag, 0, "bf16", "k = 0", min_exact=1.0)


@pytest.mark.parametrize("tile_m,tile_n", ((0, 0),) + TILES, ids=lambda v: str(v))
def test_flags_epoch_and_rank_independence(tile_m, tile_n):
    """Every tile's flag gets the epoch (slots past the tiles stay as they
    were), and the values do not depend on the rank (only the order of the
    tiles does)."""
    m, n, k, world = 1024, 768, 192, 8
    a, b, c = make("bf16", m, n, k, False, seed=11)
    with B.gemm_tile_m(tile_m):
        tiles = B.gemm_scatter_tiles(m, n, tile_n)
    flags = torch.full((tiles + 5,), 3, dtype=torch.int32, device=DEV)
    say(f"[gpu] flags tile {tile_m}x{tile_n} tiles={tiles}")
    ref, _ = run(a, b, None, 1.0, 0.0, world, rank=0, flags=flags, epoch=41, tile_n=tile_n,
                 tile_m=tile_m)
    f = flags.cpu()
    assert bool((f[:tiles] == 41).all()) and bool((f[tiles:] == 3).all())
    for rank in (3, 7):
        got, _ = run(a, b, None, 1.0, 0.0, world, rank=rank, flags=flags, epoch=42 + rank,
                     tile_n=tile_n, tile_m=tile_m)
        assert np.array_equal(got, ref), rank
        assert bool((flags.cpu()[:tiles] == 42 + rank).all())


@pytest.mark.parametrize("name", list(GEMM_WORKLOADS))
def test_full_size(name):
    """The benchmark's workload at full size, in the benchmark's launch: every
    row against the oracle (computed in row blocks on the host's threads), a
    second launch bitwise equal to the first, direct stores and every other
    tile shape bitwise equal too."""
    w = GEMM_WORKLOADS[name]
    say(f"[gpu] full size {w.describe()} (tile width {B.gemm_scatter_tile_n(w.m, w.n)})")
    d = I.gemm_inputs(w)
    a, b = d["a"].to(DEV), d["b"].to(DEV)
    c = d["c"].to(DEV) if d["c"] is not None else None
    got, _ = run(a, b, c, w.alpha, w.beta, w.world, rank=w.rank, col=8)
    again, _ = run(a, b, c, w.alpha, w.beta, w.world, rank=w.rank, col=8)
    assert np.array_equal(got, again), "two launches differ"
    other, _ = run(a, b, c, w.alpha, w.beta, w.world, rank=w.rank, col=4)
    assert np.array_equal(got, other), "staged and direct stores differ"
    for tile_m, tile_n in TILES:
        other, _ = run(a, b, c, w.alpha, w.beta, w.world, rank=w.rank, col=8, tile_n=tile_n,
                       tile_m=tile_m)
        assert np.array_equal(got, other), f"tile {tile_m}x{tile_n} differs"
    ac, bc = st(d["a"]), st(d["b"])
    cc = st(d["c"]) if d["c"] is not None else None
    say(f"[gpu] {name}: every row against the oracle on {host_threads()} host threads")

    def job(blk):
        r0, r1 = blk
        want, y, mag = oracle.gemm_scatter(ac, bc, cc, w.alpha, w.beta, w.world, w.dtype,
                                           rows=(r0, r1), want_f64=True, scatter=False)
        ratio, exact = compare(got[r0:r1], want, y, mag, w.k, w.dtype, f"{name} rows [{r0}, {r1})",
                               min_exact=0.7, quiet=True)
        return ratio, exact, (r1 - r0) * w.n

    blocks = [(r, min(w.m, r + 64)) for r in range(0, w.m, 64)]
    with cf.ThreadPoolExecutor(host_threads()) as ex:
        res = list(ex.map(job, blocks))
    n_el = sum(r[2] for r in res)
    assert n_el == w.m * w.n
    say(f"[gpu] {name}: " + repr({"max_error_over_bound": float(f"{max(r[0] for r in res):.3g}"),
                                  "min_equal_frac": float(f"{min(r[1] for r in res):.4f}"),
                                  "rows_checked": w.m, "elements_checked": n_el}))


def test_special_values():
    """inf in A, NaN in C, and a zero weight row: IEEE results as the oracle
    gives them."""
    m, n, k, world = 256, 64, 64, 2
    a, b, c = make("bf16", m, n, k, True, seed=5)
    a, b, c = a.clone(), b.clone(), c.clone()
    a[3, 10] = float("inf")
    a[7, :] = 0.0
    b[5, :] = 0.0                 # inf * 0 -> NaN in row 3, column 5
    c[9, 11] = float("nan")
    say("[gpu] special values")
    got, _ = run(a, b, c, 1.0, 1.0, world)
    want, y, mag = oracle_rows(a, b, c, 1.0, 1.0, world, "bf16")
    assert np.isnan(y[3, 5]) and np.isinf(y[3, 0]) and np.isnan(y[9, 11])
    compare(got, want, y, mag, k, "bf16", "special values")


def test_fp16_subnormal_operands():
    """fp16 operands in the subnormal range (and products far below the
    smallest normal): the result stays within the bound, whose absolute
    floor is half an ulp at the smallest normal."""
    m, n, k = 256, 64, 64
    rng = np.random.default_rng(8)
    a = torch.from_numpy(rng.integers(1, 1024, (m, k)).astype(np.float32) * 2.0 ** -24).to(torch.float16)
    b = torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).to(torch.float16)
    # rows 8.. mix normal and subnormal columns; rows 0..7 stay all subnormal,
    # so their results (about k * 2^-24) would show a flush to zero
    a[8:, ::2] = torch.from_numpy(rng.standard_normal((m - 8, k // 2)).astype(np.float32)).to(torch.float16)
    say("[gpu] fp16 subnormal operands")
    got, _ = run(a.to(DEV), b.to(DEV), None, 1.0, 0.0, 2)
    want, y, mag = oracle_rows(a, b, None, 1.0, 0.0, 2, "f16")
    compare(got, want, y, mag, k, "f16", "fp16 subnormal operands")


def test_reduce_scatter_then_add_rmsnorm():
    """Eight ranks emulated on one GPU: rank r multiplies its own A_r, B_r and
    scatters chunk q into rank q's receive buffer (slot r); rank q then sums
    its eight received chunks with its residual and normalises
    (add_rmsnorm_fwd, K = 8).  The received chunks match the oracle's GEMM,
    and rank q's new residual is bit-exact against the oracle's fused
    normalisation of the same received chunks."""
    world, m, n, k = 8, 512, 1024, 256
    chunk = m // world
    recv = torch.empty(world, world, chunk, n, dtype=torch.bfloat16, device=DEV)  # [q][r]
    ops = []
    for r in range(world):
        a, b, _ = make("bf16", m, n, k, False, seed=100 + r)
        ops.append((a, b))
        B.gemm_scatter_fwd([recv[q, r] for q in range(world)], a, b, None, 1.0, 0.0, rank=r)
    torch.cuda.synchronize()
    say("[gpu] reduce-scatter emulation: 8 GEMMs done")
    for r in (0, 5):
        a, b = ops[r]
        full = torch.cat([recv[q, r] for q in range(world)]).cpu()
        want, y, mag = oracle_rows(a, b, None, 1.0, 0.0, world, "bf16")
        compare(st(full), want, y, mag, k, "bf16", f"rank {r} partial")
    q = 6
    res = I.matrix(9, I.RESIDUAL_ID, chunk, n, 1.0, "bf16").to(DEV)
    gam = I.matrix(9, I.GAMMA_ID, 1, n, 0.25, "bf16").reshape(n).to(DEV) + 1.0
    parts = [recv[q, r].contiguous() for r in range(world)]
    res_in = res.clone()
    out = torch.empty(chunk, n, dtype=torch.bfloat16, device=DEV)
    B.add_rmsnorm_fwd(out, res, parts, gam, 1e-5)
    torch.cuda.synchronize()
    o_out, o_res, _ = oracle.add_rmsnorm([st(p.cpu()) for p in parts], st(res_in.cpu()),
                                         st(gam.cpu()), 1e-5, "bf16")
    assert np.array_equal(st(res.cpu()), o_res), "new residual differs from the oracle"
    d = ind.ulp_distance(st(out.cpu()), o_out, "bf16")
    assert int(d.max()) <= 2


def test_random_calls():
    """Seeded random calls: dtype, shape (ragged m, n, k), world and rank,
    alpha, beta, optional C, padded strides and both output alignments."""
    rng = np.random.default_rng(2024)
    for i in range(14):
        dtype = str(rng.choice(["bf16", "f16"]))
        world = int(rng.choice([1, 2, 3, 4, 8, 16]))
        m = world * int(rng.integers(1, 48))
        n = int(rng.integers(1, 700))
        k = 8 * int(rng.integers(0, 48))
        with_c = bool(rng.random() < 0.5)
        alpha = float(np.float32(rng.choice([1.0, -0.5, 1.75])))
        beta = float(np.float32(rng.choice([0.0, 1.0, -2.0]))) if with_c else 0.0
        rank = int(rng.integers(world))
        pads = [int(8 * rng.integers(0, 3)) for _ in range(2)]
        a, b, c = make(dtype, m, n, k, with_c, seed=1000 + i, lda_pad=pads[0],
                       ldb_pad=pads[1], ldc_pad=int(rng.integers(0, 5)))
        if k == 0:
            a, b = a.contiguous(), b.contiguous()
        col = int(rng.choice([4, 8]))
        pad = (-(n + 8 + col)) % 8 if col == 8 else int(rng.integers(0, 4))
        tile_n = int(rng.choice((0,) + WIDTHS))
        tile_m = int(rng.choice((0, 256, 192, 160)))
        say(f"[gpu] random #{i}: {dtype} m={m} n={n} k={k} world={world} rank={rank} "
            f"c={with_c} col={col} tile_n={tile_n} tile_m={tile_m}")
        got, _ = run(a, b, c, alpha, beta, world, rank=rank, ldd_pad=pad, col=col, tile_n=tile_n,
                     tile_m=tile_m)
        want, y, mag = oracle_rows(a, b, c, alpha, beta, world, dtype)
        compare(got, want, y, mag, k, dtype, f"random #{i}", min_exact=0.6)


def test_graph_capture_gemm_then_add_rmsnorm():
    """The reduce-scatter pipeline captured in one HIP graph: four emulated
    ranks' GEMMs (both tile widths and a forced height, one with tile flags)
    scatter into receive
    buffers, then every receiving rank sums its four chunks with its residual
    and normalises (add_rmsnorm_fwd, K = 4).  Each replay, with eager resets
    and poisoning in between, equals the eager run bit for bit, flags
    included."""
    world, m, n, k = 4, 512, 1024, 256
    chunk = m // world
    ops = [make("bf16", m, n, k, False, seed=300 + r)[:2] for r in range(world)]
    shapes = [(0, 0), (0, 256), (0, 128), (192, 256)]      # (tile height, tile width)
    res0 = I.matrix(31, I.RESIDUAL_ID, m, n, 1.0, "bf16").to(DEV)
    gam = I.matrix(31, I.GAMMA_ID, 1, n, 0.25, "bf16").reshape(n).to(DEV) + 1.0
    tiles = B.gemm_scatter_tiles(m, n, shapes[1][1])

    def step(recv, res, out, flags):
        for r, ((a, b), (tm, tn)) in enumerate(zip(ops, shapes)):
            with B.gemm_tile_m(tm):
                B.gemm_scatter_fwd([recv[q, r] for q in range(world)], a, b, rank=r, tile_n=tn,
                                   flags=flags if r == 1 else None, epoch=77)
        for q in range(world):
            B.add_rmsnorm_fwd(out[q], res[q], [recv[q, r] for r in range(world)], gam, 1e-5)

    def buffers():
        return (torch.empty(world, world, chunk, n, dtype=torch.bfloat16, device=DEV),
                torch.empty(world, chunk, n, dtype=torch.bfloat16, device=DEV),
                torch.empty(world, chunk, n, dtype=torch.bfloat16, device=DEV),
                torch.zeros(tiles, dtype=torch.int32, device=DEV))

    recv_e, res_e, out_e, flags_e = buffers()
    res_e.copy_(res0.view(world, chunk, n))
    step(recv_e, res_e, out_e, flags_e)
    torch.cuda.synchronize()
    assert bool((flags_e == 77).all())
    recv, res, out, flags = buffers()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        res.copy_(res0.view(world, chunk, n))
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step(recv, res, out, flags)
    torch.cuda.synchronize()
    say("[gpu] graph: 4 GEMMs + 4 add_rmsnorm captured")
    for rep in range(4):
        res.copy_(res0.view(world, chunk, n))     # eager work between replays
        recv.fill_(float("nan"))
        out.fill_(float("nan"))
        flags.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(recv.view(torch.int16), recv_e.view(torch.int16)), rep
        assert torch.equal(res.view(torch.int16), res_e.view(torch.int16)), rep
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), rep
        assert torch.equal(flags, flags_e), rep
    # the eager run itself against the oracle for one receiving rank
    q = 2
    parts = [st(recv_e[q, r].cpu()) for r in range(world)]
    o_out, o_res, _ = oracle.add_rmsnorm(parts, st(res0.view(world, chunk, n)[q].cpu()),
                                         st(gam.cpu()), 1e-5, "bf16")
    assert np.array_equal(st(res_e[q].cpu()), o_res)
    assert int(ind.ulp_distance(st(out_e[q].cpu()), o_out, "bf16").max()) <= 2


def test_operand_offsets_past_4gib():
    """A of 65536 x 33280 bf16 (4.36 GB, drawn on the device): rows whose
    byte offset passes 2^31 and 2^32, in every chunk, against the oracle row
    by row (each row's values do not depend on the chunk split), at every
    tile shape, which must agree bit for bit."""
    m, n, k, world = 65536, 264, 33280, 8
    chunk = m // world
    w = I.case("bf16", m, k, 1, seed=71, std=1.0)
    a = I.device_tensor(w, I.GEMM_A_ID, DEV)
    b = I.matrix(71, I.GEMM_B_ID, n, k, (8.0 * k) ** -0.5, "bf16").to(DEV)
    assert a.numel() * 2 > 1 << 32
    say(f"[gpu] offsets past 4 GiB: A {tuple(a.shape)}, {a.numel() * 2 / 2**30:.2f} GiB")
    got = None
    for tile_m, tile_n in TILES:
        g, _ = run(a, b, None, 1.0, 0.0, world, rank=3, col=8, tile_n=tile_n, tile_m=tile_m)
        if got is None:
            got = g
        assert np.array_equal(g, got), f"tile {tile_m}x{tile_n} differs"
    row_bytes = k * 2
    rows = sorted({0, chunk - 1, chunk, (1 << 31) // row_bytes, (1 << 31) // row_bytes + 1,
                   (1 << 32) // row_bytes + 1, m - 2, m - 1})
    bc = st(b.cpu())
    for r in rows:
        ar = st(a[r:r + 1].cpu())
        chunks, y, mag = oracle.gemm_scatter(ar, bc, None, 1.0, 0.0, 1, "bf16", want_f64=True)
        compare(got[r:r + 1], chunks[0], y, mag, k, "bf16", f"row {r} (byte offset {r * row_bytes:#x})",
                min_exact=0.7)
    del a
    torch.cuda.empty_cache()
