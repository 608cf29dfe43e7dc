"""The measurement aids bench.py loads (libstreamprobe.so, librowprobe.so,
libgemmprobe.so) load without a GPU and reject, before any HIP call, the
arguments they do not take."""
import ctypes
import os

import pytest

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "row_wise_normalization_rmsnorm_amd")


def _lib(name):
    path = os.path.join(PKG, name)
    if not os.path.exists(path):
        pytest.skip(f"{name} not built")
    return ctypes.CDLL(path)


# fake, 256-byte aligned device addresses: every call below fails validation
# before anything could touch them
A, B, D0, D1 = 0x10000, 0x20000000, 0x40000000, 0x50000000


def test_gemm_probe_rejects_before_launch():
    lib = _lib("libgemmprobe.so")
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.gemm_probe.argtypes = [ctypes.c_int] * 3 + [vp, i64, ctypes.c_int, vp, i64, vp, i64,
                                                    i64, i64, i64, ctypes.c_int, vp]
    dst = (ctypes.c_void_p * 2)(D0, D1)

    def call(design=0, mode=0, nbuf=4, dst=dst, ldd=512, world=2, a=A, lda=256, b=B, ldb=256,
             m=512, n=512, k=256, dtype=2):
        return lib.gemm_probe(design, mode, nbuf, dst, ldd, world, a, lda, b, ldb, m, n, k,
                              dtype, None)

    bad = [dict(design=4), dict(design=-1), dict(mode=5), dict(design=0, mode=1),
           dict(design=1, mode=2), dict(design=2, nbuf=3), dict(design=3, nbuf=6),
           dict(dtype=0), dict(dtype=3), dict(world=0), dict(world=17), dict(m=511),
           dict(m=0), dict(n=0), dict(k=-8), dict(k=12), dict(lda=260), dict(ldb=250),
           dict(lda=128), dict(ldd=500), dict(a=A + 8), dict(b=B + 2), dict(a=None),
           dict(dst=None), dict(dst=(ctypes.c_void_p * 2)(D0, None)),
           dict(design=2, mode=1, m=128), dict(design=3, k=64, nbuf=4),
           dict(lda=1 << 22, k=256)]
    for kw in bad:
        assert call(**kw) == -1, kw


def test_row_probe_rejects_before_launch():
    lib = _lib("librowprobe.so")
    vp = ctypes.c_void_p
    lib.row_probe.argtypes = [ctypes.c_int] * 4 + [vp] * 4 + [ctypes.c_int64, ctypes.c_float, vp]
    loads, stores = (ctypes.c_int * 16)(), (ctypes.c_int * 16)()
    n = lib.row_probe_policies(loads, stores, 16)
    assert n >= 1 and (loads[0], stores[0]) == (2, 2)

    def call(design=0, lp=2, sp=2, grid=64, rows=64, x=A, r=B, o=D0, g=D1):
        return lib.row_probe(design, lp, sp, grid, x, r, o, g, rows, 1e-6, None)

    for kw in (dict(design=8), dict(design=-1), dict(design=5, grid=64), dict(design=6, grid=5),
               dict(design=7, grid=15), dict(lp=7), dict(sp=5), dict(grid=0), dict(rows=0),
               dict(grid=32), dict(design=2, rows=60, grid=60), dict(design=4, grid=64),
               dict(design=4, rows=63, grid=31), dict(x=None), dict(g=None)):
        assert call(**kw) == -1, kw


def test_stream_probe_rejects_before_launch():
    lib = _lib("libstreamprobe.so")
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.stream_probe_pol.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, vp] + \
        [ctypes.c_int] * 5 + [vp]
    lc, sc = ctypes.c_int(), ctypes.c_int()
    assert lib.stream_probe_policy(0, ctypes.byref(lc), ctypes.byref(sc)) == 0
    assert (lc.value, sc.value) == (2, 2)
    assert lib.stream_probe_policy(9, ctypes.byref(lc), ctypes.byref(sc)) == -1
    reads = (ctypes.c_void_p * 2)(A, B)
    writes = (ctypes.c_void_p * 1)(D0,)

    def call(nr=2, nw=1, n16=1024, sink=D1, grid=64, block=256, unroll=4, contig=0, policy=0):
        return lib.stream_probe_pol(reads, nr, writes, nw, n16, sink, grid, block, unroll,
                                    contig, policy, None)

    for kw in (dict(nr=17), dict(nw=-1), dict(n16=-1), dict(sink=None), dict(grid=0),
               dict(policy=9), dict(policy=-1), dict(block=128), dict(unroll=3)):
        assert call(**kw) == -1, kw


def test_grid_cap_sweep_takes_only_fused_single_partial_workloads():
    """bench.py --grid-cap-sweep refuses, before touching a GPU, a workload
    it does not time (plain RMSNorm, K = 8)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for wl in ("add_rmsnorm_bf16_4096x8192_k8", "rmsnorm_f32_512x2048"):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--grid-cap-sweep",
                            "--workload", wl], capture_output=True, text=True, timeout=300)
        assert r.returncode != 0 and "one partial" in r.stderr, (wl, r.stderr[-300:])
