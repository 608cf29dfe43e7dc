"""The GEMM + reduce-scatter epilogue's C ABI without a GPU: the library
exports what include/gemm_scatter.h declares, invalid arguments are rejected
with the documented codes before any HIP call, and the tile schedule puts the
other ranks' chunks first and the local chunk last (the order the oracle
states), spreads each round of tiles over the eight XCDs in contiguous runs,
and covers every tile exactly once, at either tile width and every tile
height; the automatic width and height follow their documented rules."""
from __future__ import annotations

import ctypes

import pytest

import oracle
from row_wise_normalization_rmsnorm_amd import binding as B
from tests.test_capi_cpu import FAKE, declared

TM = B.GEMM_SCATTER_TILE_M
WIDTHS = (B.GEMM_SCATTER_TILE_N, B.GEMM_SCATTER_TILE_N_NARROW)
HEIGHTS = (256, 192, 160)   # of the 256-wide tiles


def test_exports_every_declared_function():
    names = declared("gemm_scatter.h")
    assert names == set(B.GEMM_SCATTER_EXPORTS)
    for n in names:
        assert hasattr(B.lib(), n), n


def test_tile_count():
    f = B.lib().gemm_scatter_tiles
    assert f(4096, 8192, 256) == 16 * 32 and f(4096, 8192, 128) == 16 * 64
    assert f(4096, 8192, 0) == 16 * 32                  # 512 wide tiles: stays wide
    assert f(256, 257, 128) == 3 and f(256, 129, 128) == 2
    with B.gemm_tile_m(256):
        assert f(1, 1, 256) == 1 and f(0, 5, 256) == 0 and f(257, 256, 256) == 2
        assert f(256, 257, 256) == 2
    with B.gemm_tile_m(160):
        assert f(256, 257, 256) == 4 and f(320, 256, 256) == 2 and f(321, 256, 256) == 3
        assert f(4096, 8192, 128) == 16 * 64            # the height applies to 256-wide tiles only
    with B.gemm_tile_m(192):
        assert f(1536, 8192, 256) == 8 * 32 and f(1537, 8192, 0) == 9 * 32
    assert f(-1, 4, 0) == -1 and f(4, 1 << 31, 0) == -1
    assert f(256, 256, 64) == -1 and f(256, 256, -1) == -1 and f(256, 256, 512) == -1


def wide_cost(m: int, n: int, h: int) -> int:
    """The header's estimate for 256-wide tiles h rows high, restated."""
    t = -(-m // h) * -(-n // 256)
    full, rem = divmod(t, 256)
    rounds = 1000 * full + (700 + 300 * rem // 256 if rem else 0)
    return rounds * (390 + 1000 * h // 256)


def test_automatic_tile_height():
    """256-wide tiles take the cheapest of 256, 192 and 160 rows by the
    rounds estimate (ties to the taller tile); 128-wide tiles stay 256 rows.
    The measured bf16 shapes (n = 8192, k = 3584) take the height that timed
    fastest: 192 rows at 1536 and 3072 tokens, 160 at 2560, 256 elsewhere."""
    h = B.gemm_scatter_tile_m
    measured = {1536: 192, 2048: 256, 2560: 160, 3072: 192, 4096: 256, 5120: 256, 8192: 256,
                16384: 256}
    for m, height in measured.items():
        assert B.gemm_scatter_tile_n(m, 8192) == 256 and h(m, 8192, 0) == height, m
    assert h(1024, 8192, 0) == 256 and B.gemm_scatter_tile_n(1024, 8192) == 128
    assert h(4096, 8192, 128) == 256 and h(4096, 4096, 0) == 256
    assert h(-1, 5, 0) == -1 and h(5, 1 << 31, 0) == -1 and h(5, 5, 64) == -1

    def rule(m, n):
        costs = [(wide_cost(m, n, x), -x) for x in HEIGHTS]
        return -min(costs)[1]

    import random
    rng = random.Random(6)
    for _ in range(300):
        m, n = rng.randint(1, 40000), rng.randint(1, 20000)
        assert h(m, n, 256) == rule(m, n), (m, n)
        t = h(m, n, 256)
        assert B.gemm_scatter_tiles(m, n, 256) == -(-m // t) * -(-n // 256)


def test_tune_forces_the_tile_height():
    """gemm_scatter_tune(h) makes every later call use h-row 256-wide tiles
    (queries, tile counts and schedules alike); 0 restores the automatic
    height; other values are rejected and change nothing."""
    try:
        for x in HEIGHTS:
            assert B.lib().gemm_scatter_tune(x) == 0
            assert B.gemm_scatter_tile_m(4096, 8192, 0) == x
            assert B.gemm_scatter_tile_m(1024, 8192, 0) == 256   # automatic width: 128-wide
            assert B.gemm_scatter_tiles(4096, 8192, 256) == -(-4096 // x) * 32
        assert B.lib().gemm_scatter_tune(128) == -2 and B.lib().gemm_scatter_tune(-1) == -2
        assert B.gemm_scatter_tile_m(4096, 8192, 0) == 160           # unchanged by the rejected calls
        assert B.lib().gemm_scatter_tune(0) == 0
        assert B.gemm_scatter_tile_m(2560, 8192, 0) == 160 and B.gemm_scatter_tile_m(4096, 8192, 0) == 256
    finally:
        B.gemm_scatter_tune(0)


def test_automatic_tile_width():
    """The automatic width counts rounds of workgroups over 256 CUs: narrow
    exactly when ceil(T128 / 256) <= ceil(T256 / 256) (and there are tiles).
    The cases are the measured bf16 shapes (n = 8192, k = 3584), where the
    faster width was taken at each, and edges of the rule."""
    w = B.gemm_scatter_tile_n
    assert B.GEMM_SCATTER_CUS == 256
    measured = {1024: 128, 1536: 256, 2048: 256, 2560: 256, 3072: 256, 4096: 256,
                5120: 256, 8192: 256, 16384: 256}
    for m, width in measured.items():
        assert w(m, 8192) == width, m
    assert w(1024, 8193) == 256          # 4 x 33 = 132 wide tiles, 4 x 65 = 260 narrow
    assert w(256 * 128, 256) == 128 and w(256 * 129, 256) == 256
    assert w(1, 1) == 128 and w(0, 0) == 256      # nothing to launch: no round either way
    assert w(-1, 5) == -1 and w(5, 1 << 31) == -1

    def rule(m, n):
        tm = -(-m // 256)
        wide, narrow = tm * -(-n // 256), tm * -(-n // 128)
        return 128 if wide > 0 and -(-narrow // 256) <= -(-wide // 256) else 256

    import random
    rng = random.Random(5)
    for _ in range(300):
        m, n = rng.randint(0, 40000), rng.randint(0, 20000)
        assert w(m, n) == rule(m, n), (m, n)
        assert B.gemm_scatter_tiles(m, n) == B.gemm_scatter_tiles(m, n, w(m, n))


def call(**kw):
    """gemm_scatter_fwd with valid defaults on fake, well-separated device
    addresses (every call here must fail validation before any launch)."""
    world = kw.pop("world", 2)
    d = kw.pop("dst", None)
    if d is None:
        d = [FAKE + (q + 1) * (1 << 28) for q in range(world)]
    args = dict(ldd=64, rank=0, a=FAKE + (1 << 32), lda=64, b=FAKE + (2 << 32), ldb=64, c=None,
                ldc=0, alpha=1.0, beta=0.0, m=128, n=64, k=64, dtype=2, flags=None, epoch=1,
                tile_n=0)
    args.update(kw)
    arr = (ctypes.c_void_p * max(len(d), 1))(*d)
    return B.lib().gemm_scatter_fwd(arr, args["ldd"], world, args["rank"], args["a"], args["lda"],
                                    args["b"], args["ldb"], args["c"], args["ldc"],
                                    ctypes.c_float(args["alpha"]), ctypes.c_float(args["beta"]),
                                    args["m"], args["n"], args["k"], args["dtype"], args["flags"],
                                    ctypes.c_uint32(args["epoch"]), args["tile_n"], None)


def test_error_codes():
    assert call(dtype=0) == -3 and call(dtype=5) == -3
    assert call(m=-1) == -2 and call(k=1 << 31) == -2
    assert call(world=0, dst=[FAKE]) == -2 and call(world=17) == -2
    assert call(rank=2) == -2 and call(rank=-1) == -2
    assert call(m=129) == -2                                   # m % world
    assert call(dst=[FAKE, None]) == -1
    assert call(a=None) == -1 and call(b=None) == -1
    assert call(ldd=32) == -2 and call(lda=32) == -2
    assert call(c=FAKE + (3 << 32), ldc=32) == -2
    assert call(k=60, lda=64, ldb=64) == -2                     # k % 8
    assert call(lda=68) == -2                                   # lda % 8
    assert call(a=FAKE + (1 << 32) + 8) == -2                   # a not 16-byte aligned
    assert call(dst=[FAKE + 1, FAKE + (1 << 28)]) == -2         # dst misaligned
    assert call(flags=FAKE + (5 << 32) + 2) == -2               # flags misaligned
    assert call(lda=1 << 22, k=64) == -2                        # 255 * lda + k too large
    assert call(tile_n=64) == -2 and call(tile_n=-1) == -2      # width not 0, 128 or 256
    # overlaps: a dst chunk over a, over another chunk, over flags
    assert call(dst=[FAKE + (1 << 32), FAKE + (1 << 28)]) == -5
    assert call(dst=[FAKE + (1 << 28), FAKE + (1 << 28) + 64]) == -5
    assert call(flags=FAKE + (1 << 28) + 16) == -5
    assert call(c=FAKE + (2 << 28), ldc=64) == -5
    # flags over an operand: a, b, c
    assert call(flags=FAKE + (1 << 32) + 64) == -5 and call(flags=FAKE + (2 << 32)) == -5
    assert call(c=FAKE + (3 << 32), ldc=64, flags=FAKE + (3 << 32) + 1024) == -5
    # nothing to do: valid, and nothing launched
    assert call(m=0) == 0 and call(n=0) == 0
    assert call(m=0, tile_n=128) == 0 and call(n=0, tile_n=256) == 0


def tile_chunk(tile: int, m: int, n: int, world: int, width: int) -> int:
    tn = -(-n // width)
    return ((tile // tn) * B.gemm_scatter_tile_m(m, n, width)) // (m // world)


GROUP_ROWS = 8  # tile-rows per schedule group


@pytest.mark.parametrize("shape", [(256, 256), (256, 128), (192, 256), (160, 256), (0, 256)],
                         ids=lambda s: f"{s[0] or 'auto'}x{s[1]}")
@pytest.mark.parametrize("m,n,world", [(4096, 8192, 8), (4096, 8192, 1), (8192, 4096, 8),
                                       (1024, 1024, 4), (777 * 8, 300, 8), (256, 256, 2),
                                       (2048, 2560, 16), (24576, 2048, 8), (4096, 8192, 2),
                                       (1024, 8192, 8), (1536, 8192, 8), (2560, 8192, 8)])
def test_schedule_is_remote_first_and_complete(m, n, world, shape):
    height, width = shape
    with B.gemm_tile_m(height):
        check_schedule(m, n, world, width)


def check_schedule(m, n, world, width):
    tiles = B.gemm_scatter_tiles(m, n, width)
    tn = -(-n // width)
    for rank in range(world):
        wg, pos = B.gemm_scatter_schedule(m, n, world, rank, width)
        assert sorted(wg) == list(range(tiles)) and sorted(pos) == list(range(tiles))
        order = oracle.gemm_scatter_chunk_order(world, rank)
        rank_of = {q: i for i, q in enumerate(order)}
        seq = [rank_of[tile_chunk(t, m, n, world, width)] for t in pos]
        # the local chunk's tiles come last
        local = [i for i, q in enumerate(seq) if q == world - 1]
        assert not local or local == list(range(tiles - len(local), tiles)), (m, n, world, rank)
        # the other chunks in ring order, group by group (a group of up to
        # eight tile-rows may hold several chunks, never out of order)
        remote = seq[:tiles - len(local)]
        step = GROUP_ROWS * tn
        blocks = [remote[i:i + step] for i in range(0, len(remote), step)]
        for x, y in zip(blocks, blocks[1:]):
            assert max(x) <= min(y), (m, n, world, rank)
        # inside a group, tiles go down the group's tile-rows first
        for i in range(0, len(remote), step):
            block = pos[i:min(i + step, len(remote))]
            cols = [t % tn for t in block]
            assert cols == sorted(cols)


@pytest.mark.parametrize("shape", [(256, 256), (256, 128), (192, 256), (160, 256)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_workgroups_are_dealt_to_xcds_in_contiguous_runs(shape):
    m, n, world = 4096, 8192, 8
    with B.gemm_tile_m(shape[0]):
        wg, pos = B.gemm_scatter_schedule(m, n, world, 3, shape[1])
    at = {t: s for s, t in enumerate(pos)}
    positions = [at[t] for t in wg]
    rnd = 8 * 32
    for base in range(0, len(wg) - len(wg) % rnd, rnd):
        for x in range(8):
            ps = [positions[w] for w in range(base + x, base + rnd, 8)]
            assert ps == list(range(base + 32 * x, base + 32 * x + 32))


def test_binding_checks_shapes_before_the_library():
    import torch
    a = torch.empty(8, 16, dtype=torch.bfloat16)
    with pytest.raises(B.RmsnormError):
        B.gemm_scatter_fwd([a[:4], a[4:]], a, a.to(torch.float16))


def test_binding_passes_the_real_row_stride():
    """A broadcast or overlapping operand keeps its short row stride, which
    the library rejects, instead of being described as distinct rows."""
    import torch
    base = torch.empty(1, 64, dtype=torch.bfloat16)
    assert B.matrix_ld(tuple(base.expand(128, 64).shape), base.expand(128, 64).stride()) == 0
    assert B.matrix_ld((128, 64), (64, 1)) == 64
    assert B.matrix_ld((128, 64), (72, 1)) == 72          # padded rows
    assert B.matrix_ld((128, 64), (32, 1)) == 32          # overlapping rows, rejected below
    assert B.matrix_ld((1, 64), (0, 1)) == 64             # one row: its own length
    assert B.matrix_ld((128, 0), (1, 1)) == 1
    for shape, strides in (((128, 64), (64, 2)), ((8, 8, 8), (64, 8, 1)), ((64,), (1,))):
        with pytest.raises(B.RmsnormError):
            B.matrix_ld(shape, strides)
    # the library turns such strides away before any launch
    assert call(lda=0) == -2 and call(ldb=0) == -2 and call(ldd=0) == -2
    assert call(lda=32) == -2


def test_schedule_random_shapes():
    """Seeded random shapes: every schedule is a permutation, the local chunk
    runs last, and the other chunks keep ring order group by group."""
    import random
    rng = random.Random(77)
    for _ in range(60):
        world = rng.choice([1, 2, 3, 4, 5, 7, 8, 16])
        m = world * rng.randint(1, 700)
        n = rng.randint(1, 3000)
        rank = rng.randrange(world)
        width = rng.choice((0,) + WIDTHS)
        B.gemm_scatter_tune(rng.choice((0,) + HEIGHTS))
        try:
            tiles = B.gemm_scatter_tiles(m, n, width)
            used = width or B.gemm_scatter_tile_n(m, n)
            tn = -(-n // used)
            wg, pos = B.gemm_scatter_schedule(m, n, world, rank, width)
            seq_chunks = [tile_chunk(t, m, n, world, used) for t in pos]
        finally:
            B.gemm_scatter_tune(0)
        assert sorted(wg) == list(range(tiles)) == sorted(pos)
        order = oracle.gemm_scatter_chunk_order(world, rank)
        rank_of = {q: i for i, q in enumerate(order)}
        seq = [rank_of[q] for q in seq_chunks]
        local = [i for i, q in enumerate(seq) if q == world - 1]
        assert not local or local == list(range(tiles - len(local), tiles)), (m, n, world, rank)
        remote = seq[:tiles - len(local)]
        step = GROUP_ROWS * tn
        blocks = [remote[i:i + step] for i in range(0, len(remote), step)]
        for x, y in zip(blocks, blocks[1:]):
            assert max(x) <= min(y), (m, n, world, rank)
