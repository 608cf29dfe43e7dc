"""Benchmark of the fused add + RMSNorm hot path on one MI355X.

One step = one ``add_rmsnorm_fwd`` launch over the whole workload (every step
of the path: load K partials and the residual, sum, write the residual, sum of
squares, reduce, scale, normalise, store); ``--workload`` selects another
workload (plain RMSNorm, the block all-reduce sum, or the GEMM with a
reduce-scatter epilogue, which reports TFLOP/s against the matrix-core
peak).  Inputs are seeded synthetic data
resident in HBM before timing starts.  Several copies of the buffers are
rotated so that consecutive steps never find their inputs in the 256 MB
Infinity Cache (by default at least 2 GiB of distinct buffers, 8x its
size: with fewer, stores that allocate in the caches have measured faster
only because a later step overwrote their lines before they were written
back).  Timing: W untimed warm-up steps, then exactly K steps
bracketed by ``torch.cuda.synchronize()`` and HIP events recorded on the
stream the kernels run on.  W defaults to 2000: after 20 the GPU's clocks
were still rising (the headline measured 45.1-45.3 us per step against
44.2-44.3 after 2000, the 1024-token GEMM 72.6 against 61.0).

Prints one JSON line.  ``roofline.achieved`` is the workload's algorithmic
bytes per launch divided by the average launch duration; ``cpu_baseline``
times the CPU oracle (row-parallel over the host cores) on the same workload.

``per_launch`` (context) adds single-launch timings, and for small
workloads a cache-flushed, a launch-and-synchronise and a graph-replay rate;
``stream_ceiling`` is a plain streaming kernel moving the same bytes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-cpu-baseline] [--no-ceiling] [--inplace] [--rotate-bytes GIB] [--rows N]
       [--resident-context]
       python bench.py --workload NAME --sweep [--repeat R] [--variant-filter S]
       python bench.py --ceiling-sweep | --copy-calibration | --gemm-shapes
       python bench.py --design-sweep | --gemm-design-sweep [--repeat R] [--steps K]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from row_wise_normalization_rmsnorm_amd.profiling import source_hash  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}  # MI355X dense matrix-core peaks


def traffic_for(kernel: str, workload: str, op: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != source_hash(op) or d.get("kernel") != kernel:
        return None
    return d.get("traffic_bytes_per_launch")


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, target_cpu_seconds: float = 12.0, max_passes: int = 40) -> dict:
    """The oracle, unchanged, over the workload's rows, split over the host's
    cores (each thread runs the oracle on its own row block); whole passes are
    repeated until about ``target_cpu_seconds`` of CPU work has been done."""
    import oracle
    from row_wise_normalization_rmsnorm_amd import inputs as I

    d = I.make_inputs(w)
    cores = host_cores()
    bounds = [(i * w.rows // cores, (i + 1) * w.rows // cores) for i in range(cores)]
    g = I.to_storage(d["gamma"]) if "gamma" in d else None
    if w.op == "block_sum":
        xs = I.to_storage(d["x"])

        def job(b):
            a, z = b
            return oracle.block_sum(xs[a:z].reshape(-1), w.dtype)
    elif w.fused:
        ps = I.storage_list(d["partials"])
        r = I.to_storage(d["residual"])

        def job(b):
            a, z = b
            return oracle.add_rmsnorm([p[a:z] for p in ps], r[a:z], g, w.eps, w.dtype)
    else:
        x = I.to_storage(d["x"])

        def job(b):
            a, z = b
            return oracle.rmsnorm(x[a:z], g, w.eps, w.dtype)
    oracle._load()
    passes = 0
    with cf.ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        c0 = time.process_time()
        while True:
            list(ex.map(job, bounds))
            passes += 1
            if time.process_time() - c0 >= target_cpu_seconds or passes >= max_passes:
                break
        dt = time.perf_counter() - t0
        cpu = time.process_time() - c0
    per_pass = dt / passes
    # the same oracle on one thread, over whole row blocks until about a
    # third of the multi-threaded budget is spent
    blocks, t1 = 0, time.perf_counter()
    while True:
        job(bounds[blocks % cores])
        blocks += 1
        if time.perf_counter() - t1 >= target_cpu_seconds / 3 or blocks >= max_passes * cores:
            break
    single = (time.perf_counter() - t1) / blocks * cores
    return {"value": round(w.algorithmic_bytes() / per_pass / 1e9, 3), "unit": "GB/s",
            "rows_per_s": round(w.rows / per_pass, 1), "seconds_per_pass": round(per_pass, 4),
            "cores": cores, "kind": "oracle",
            "sample": (f"{passes} full passes over all {w.rows} rows of {w.name} "
                       f"({cpu:.1f} CPU-seconds), rows split over {cores} threads"
                       + (f"; the oracle computes each output row once (the {w.gather} "
                          "gather copies are no arithmetic), the rate counts the workload's "
                          "algorithmic bytes" if w.gather else "")),
            "single_thread": {"value": round(w.algorithmic_bytes() / single / 1e9, 3),
                              "unit": "GB/s", "rows_per_s": round(w.rows / single, 1),
                              "cores": 1,
                              "sample": f"{blocks} row blocks of {w.rows // cores} rows, "
                                        "one thread"}}


def gemm_cpu_baseline(w, target_cpu_seconds: float = 12.0) -> dict:
    """The GEMM oracle, unchanged, on a sample of whole output rows spread
    over the m rows, one row per task over the host's cores, sized to about
    ``target_cpu_seconds`` of CPU work; then a few rows on one thread."""
    import oracle
    from row_wise_normalization_rmsnorm_amd import inputs as I

    d = I.gemm_inputs(w)
    ac, bc = I.to_storage(d["a"]), I.to_storage(d["b"])
    cc = I.to_storage(d["c"]) if d["c"] is not None else None

    def job(r):
        return oracle.gemm_scatter(ac, bc, cc, w.alpha, w.beta, w.world, w.dtype,
                                   rows=(r, r + 1), scatter=False)

    oracle._load()
    t0 = time.perf_counter()
    job(0)
    per_row = time.perf_counter() - t0
    cores = host_cores()
    nrows = max(cores, min(w.m, int(target_cpu_seconds / max(per_row, 1e-6)) // cores * cores))
    rows = [int(i * w.m // nrows) for i in range(nrows)]
    c0 = time.process_time()
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        list(ex.map(job, rows))
    dt = time.perf_counter() - t0
    cpu = time.process_time() - c0
    row_flops = 2 * w.n * w.k
    single_rows = max(1, min(8, int(4.0 / max(per_row, 1e-6))))
    t1 = time.perf_counter()
    for r in rows[:single_rows]:
        job(r)
    single = (time.perf_counter() - t1) / single_rows
    return {"value": round(nrows * row_flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "seconds_for_full_workload": round(dt * w.m / nrows, 1),
            "sample": (f"{nrows} of the {w.m} output rows of {w.name} (evenly spaced, every "
                       f"chunk), one row per task over {cores} threads ({cpu:.1f} CPU-seconds)"),
            "single_thread": {"value": round(row_flops / single / 1e12, 6), "unit": "TFLOP/s",
                              "cores": 1, "sample": f"{single_rows} rows, one thread"}}


def gemm_bench(a, name: str) -> int:
    """One step = one gemm_scatter_fwd launch over the whole workload."""
    import torch
    from row_wise_normalization_rmsnorm_amd import binding as B
    from row_wise_normalization_rmsnorm_amd import inputs as I
    from row_wise_normalization_rmsnorm_amd.workloads import GEMM_WORKLOADS

    w = GEMM_WORKLOADS[name]
    dev = "cuda:0"
    B.lib()
    print(f"[bench] {w.describe()}: generating inputs", file=sys.stderr, flush=True)
    d = I.gemm_inputs(w)
    nsets = max(1, int(-(-a.rotate_bytes * (1 << 30) // w.algorithmic_bytes())))
    sets = []
    for _ in range(nsets):
        s = {"a": d["a"].to(dev), "b": d["b"].to(dev),
             "c": d["c"].to(dev) if d["c"] is not None else None}
        s["dst"] = [torch.empty(w.m // w.world, w.n, dtype=s["a"].dtype, device=dev)
                    for _ in range(w.world)]
        sets.append(s)
    tile_n = B.gemm_scatter_tile_n(w.m, w.n)
    tile_m = B.gemm_scatter_tile_m(w.m, w.n, tile_n)
    kernel = f"gemm_scatter<{w.dtype},{tile_m}x{tile_n}x64,w4,mfma16x16x32>"

    def step(i):
        s = sets[i % nsets]
        B.gemm_scatter_fwd(s["dst"], s["a"], s["b"], s["c"], w.alpha, w.beta, w.rank)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / a.steps
    tflops = w.flops() / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    print(f"[bench] {kernel}: {ms * 1e3:.2f} us/launch, {tflops:.1f} TFLOP/s "
          f"({100 * tflops / peak:.1f}% of peak), {nsets} rotating sets, wall {wall:.2f}s",
          file=sys.stderr, flush=True)
    lat = {"batched": latency(step, min(a.steps, 200))}

    def timed(fn, n):
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # context: the vendor library's GEMM (torch.matmul -> hipBLASLt, plain
    # output) on the same rotated operands; with --resident-context also both
    # on one set of operands, which then stay in the 256 MB Infinity Cache
    # (kept out of the default run so that a kernel trace of it holds only
    # the rotated launches this line times)
    nctx = max(10, min(a.steps, 100))

    def tf(x):
        return round(w.flops() / (x * 1e-3) / 1e12, 1)

    # the library gets the warm-up the shape sweep gives it: a first batch
    # (its own set-up for the shape), then 100 ms of its launches
    lib = lambda i: torch.matmul(sets[i % nsets]["a"], sets[i % nsets]["b"].t())

    def lib_batch():
        for i in range(10):
            lib(i)
        torch.cuda.synchronize()

    lib_batch()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.1:
        lib_batch()
    lib_ms = timed(lib, nctx)
    print(f"[bench] torch.matmul (hipBLASLt) on the same rotated operands: {lib_ms * 1e3:.2f} us "
          f"({tf(lib_ms)} TFLOP/s)", file=sys.stderr, flush=True)
    resident = None
    if a.resident_context:
        hot_ms = timed(lambda i: B.gemm_scatter_fwd(sets[0]["dst"], sets[0]["a"], sets[0]["b"],
                                                    sets[0]["c"], w.alpha, w.beta, w.rank), nctx)
        lib_hot_ms = timed(lambda i: torch.matmul(sets[0]["a"], sets[0]["b"].t()), nctx)
        resident = {"what": "one set of operands, which stay in the Infinity Cache",
                    "kernel": {"us": round(hot_ms * 1e3, 2), "tflops": tf(hot_ms)},
                    "library": {"us": round(lib_hot_ms * 1e3, 2), "tflops": tf(lib_hot_ms)},
                    "kernel_over_library": round(lib_hot_ms / hot_ms, 4)}
        print(f"[bench] one operand set (cache-resident): kernel {hot_ms * 1e3:.2f} us "
              f"({tf(hot_ms)} TFLOP/s), torch.matmul {lib_hot_ms * 1e3:.2f} us "
              f"({tf(lib_hot_ms)} TFLOP/s)", file=sys.stderr, flush=True)

    result = {
        "metric": f"achieved TFLOP/s (% of dense {w.dtype} matrix-core peak), {w.describe()}",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accumulate_dtype": "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/(8k)) weights, resident in HBM)",
        "config": {"workload": w.name, "op": w.op, "m": w.m, "n": w.n, "k": w.k,
                   "world": w.world, "rank": w.rank, "kernel": kernel, "tile_n": tile_n,
                   "rotating_sets": nsets,
                   "flops_per_step": w.flops(),
                   "algorithmic_bytes_per_step": w.algorithmic_bytes()},
        "pct_of_peak": round(100 * tflops / peak, 2),
        "per_launch": lat,
        "library_context": {"what": "torch.matmul(a, b.t()) (hipBLASLt), same rotated "
                                    "operands, plain output",
                            "us": round(lib_ms * 1e3, 2), "tflops": tf(lib_ms),
                            "kernel_over_library": round(lib_ms / ms, 4)},
        "resident_context": resident,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": traffic_for(kernel, w.name, w.op)},
    }
    if not a.no_cpu_baseline:
        del sets
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = gemm_cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


GEMM_SHAPES = [  # (m tokens, n hidden, k intermediate slice, world)
    (1024, 8192, 3584, 8), (1536, 8192, 3584, 8), (2048, 8192, 3584, 8), (2560, 8192, 3584, 8),
    (3072, 8192, 3584, 8), (4096, 8192, 3584, 8), (5120, 8192, 3584, 8), (8192, 8192, 3584, 8),
    (4096, 4096, 1792, 8), (4096, 8192, 1024, 8), (4096, 8192, 7168, 8), (16384, 8192, 3584, 8),
]


def gemm_shapes(a) -> int:
    """One JSON line per shape of GEMM_SHAPES (bf16, operands rotated over
    about 1 GiB): the kernel at each tile width (and which one the automatic
    choice takes) against torch.matmul (hipBLASLt) on the same operands, all
    timed with HIP events over back-to-back launches, after 100 ms of
    warm-up, round-robin over three rounds (median)."""
    import statistics

    import torch
    from row_wise_normalization_rmsnorm_amd import binding as B
    from row_wise_normalization_rmsnorm_amd import inputs as I
    from row_wise_normalization_rmsnorm_amd.workloads import GemmWorkload

    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for (m, n, k, world) in GEMM_SHAPES:
        w = GemmWorkload(f"gemm_scatter_bf16_{m}x{n}x{k}_w{world}", "bf16", m, n, k, world)
        d = I.gemm_inputs(w)
        nsets = max(1, int(-(-(1 << 30) // w.algorithmic_bytes())))
        sets = []
        for _ in range(nsets):
            sa, sb = d["a"].to(dev), d["b"].to(dev)
            sets.append((sa, sb, [torch.empty(m // world, n, dtype=sa.dtype, device=dev)
                                  for _ in range(world)]))

        def timed(fn, reps):
            e0.record(stream)
            for i in range(reps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        reps = max(20, min(200, int(2e5 / max(w.flops() / 1.2e12, 1.0))))

        def shaped(tm, tn):
            def f(i):
                with B.gemm_tile_m(tm if tn == B.GEMM_SCATTER_TILE_N else 0):
                    B.gemm_scatter_fwd(sets[i % nsets][2], sets[i % nsets][0], sets[i % nsets][1], tile_n=tn)
            return f

        shapes = [(tm, B.GEMM_SCATTER_TILE_N) for tm in (256, 192, 160)] + \
            [(B.GEMM_SCATTER_TILE_M, B.GEMM_SCATTER_TILE_N_NARROW)]
        fns = {sh: shaped(*sh) for sh in shapes}
        fns["lib"] = lambda i: torch.matmul(sets[i % nsets][0], sets[i % nsets][1].t())
        # the GPU idles while the host builds a shape's inputs, and its clocks
        # take tens of milliseconds to rise again: warm up for 100 ms, then
        # time the three round-robin, three rounds, median
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < 0.1:
            for f in fns.values():
                for i in range(5):
                    f(i)
            torch.cuda.synchronize()
        runs = {key: [] for key in fns}
        for _ in range(3):
            for key, f in fns.items():
                runs[key].append(timed(f, reps))
        by_shape = {}
        for tm, tn in shapes:
            t_ms = statistics.median(runs[(tm, tn)])
            with B.gemm_tile_m(tm if tn == B.GEMM_SCATTER_TILE_N else 0):
                tiles = B.gemm_scatter_tiles(m, n, tn)
            by_shape[(tm, tn)] = {"tiles": tiles, "us": round(t_ms * 1e3, 2),
                                  "tflops": round(w.flops() / (t_ms * 1e-3) / 1e12, 1)}
        auto = B.gemm_scatter_tile_n(m, n)
        auto_m = B.gemm_scatter_tile_m(m, n, auto)
        a = by_shape[(auto_m, auto)]
        lib = statistics.median(runs["lib"])
        print(json.dumps({"workload": w.name, "m": m, "n": n, "k": k, "world": world,
                          "tile_n": auto, "tile_m": auto_m, "tiles": a["tiles"],
                          "us": a["us"], "tflops": a["tflops"],
                          "by_tile": {f"{tm}x{tn}": v for (tm, tn), v in by_shape.items()},
                          "library_us": round(lib * 1e3, 2),
                          "library_tflops": round(w.flops() / (lib * 1e-3) / 1e12, 1),
                          "rotating_sets": nsets, "launches": reps}), flush=True)
        del sets
        torch.cuda.empty_cache()
    return 0


def stream_ceiling(w, dev: str = "cuda:0", steps: int = 60, rotate_gib: float = 2.0,
                   inplace: bool = False) -> dict:
    """HBM bandwidth of a plain streaming kernel (libstreamprobe.so) moving the
    same bytes as one step of the workload, with the kernel's aliasing: the
    fused form reads K partials and the residual and writes the residual in
    place and the output (a separate buffer, or the first partial with
    ``inplace``); the plain form reads x and writes the output; the block sum
    only reads.  Each stream is one [rows, hidden] tensor; buffers rotate as
    in the benchmark."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "row_wise_normalization_rmsnorm_amd", "libstreamprobe.so")
    lib = ctypes.CDLL(path)
    lib.stream_probe.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    if w.op == "block_sum":
        nr, writes = 1, []
    elif w.gather:
        nr = w.k + 1                                          # p0..p(K-1), residual
        writes = [w.k] + [nr + j for j in range(w.gather)]    # residual in place, each output
    elif w.fused:
        nr = w.k + 1                                          # p0..p(K-1), residual
        writes = [w.k, 0 if inplace else nr]                  # residual in place, output
    else:
        nr = 1
        writes = [0 if inplace else 1]
    nw = len(writes)
    nbuf = max([nr] + [j + 1 for j in writes])
    tensor_bytes = w.rows * w.hidden * w.itemsize
    n16 = tensor_bytes // 16
    set_bytes = nbuf * tensor_bytes
    nsets = max(1, int(-(-rotate_gib * (1 << 30) // set_bytes)))
    bufs = [[torch.empty(n16 * 16, dtype=torch.uint8, device=dev).fill_(j + 1)
             for j in range(nbuf)] for _ in range(nsets)]
    sink = torch.zeros(64, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    best = None
    for grid in (2048, 4096, 8192):
        args = []
        for b in bufs:
            ra = (ctypes.c_void_p * nr)(*[t.data_ptr() for t in b[:nr]])
            wa = (ctypes.c_void_p * max(nw, 1))(*[b[j].data_ptr() for j in writes])
            args.append((ra, wa))

        def launch(i):
            ra, wa = args[i % nsets]
            rc = lib.stream_probe(ra, nr, wa, nw, n16, sink.data_ptr(), grid, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"stream_probe failed: {rc}")

        for i in range(5):
            launch(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            launch(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        gbs = (nr + nw) * tensor_bytes / us / 1e3
        if best is None or gbs > best["value"]:
            best = {"value": round(gbs, 1), "unit": "GB/s", "us": round(us, 2), "grid": grid}
    best.update({"reads": nr, "writes": nw, "writes_in_place": sum(j < nr for j in writes),
                 "kind": "plain nontemporal 16-byte streaming kernel",
                 "frac_of_peak": round(best["value"] / HBM_PEAK_GBS, 4)})
    del bufs
    return best


def latency(step, n: int, flush_bytes: int = 0) -> dict:
    """Per-launch durations from an event pair around each launch: median,
    p10 and p90 in microseconds.  ``flush_bytes`` > 0 clears a scratch
    buffer of that size before every launch, outside the event pair, so each
    launch starts with its inputs out of the caches."""
    import torch
    stream = torch.cuda.current_stream()
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0") if flush_bytes else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(ev):
        if scratch is not None:
            scratch.zero_()
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    q = lambda f: round(us[min(n - 1, int(f * n))], 3)  # noqa: E731
    return {"median_us": q(0.5), "p10_us": q(0.1), "p90_us": q(0.9), "launches": n,
            "flush_bytes": flush_bytes}


def sync_latency(step, n: int) -> dict:
    """"kernel-sync" mode: host wall time of one launch followed by a
    synchronisation, median over n (context: includes launch overhead)."""
    import statistics
    import torch
    ts = []
    torch.cuda.synchronize()
    for i in range(n):
        t0 = time.perf_counter()
        step(i)
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e6)
    return {"median_us": round(statistics.median(ts), 3), "launches": n}


def graph_replay(step, n: int, reps: int = 5) -> dict:
    """n launches captured once in a HIP graph and replayed: the device-side
    rate with no per-launch host work (context for launch-bound sizes)."""
    import statistics
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / n)
    del g
    return {"us_per_launch": round(statistics.median(per), 3), "launches": n, "replays": reps}


def sweep(w, step, a, B) -> int:
    """Time every compatible variant (the dispatcher's choice is marked).
    With --repeat R the variants are timed round-robin R times and the
    median is reported, so slow drifts of the clock do not favour one."""
    import statistics
    import torch
    plan = B.rmsnorm_plan_ag if w.gather else B.rmsnorm_plan
    default = plan(w.rows, w.hidden, w.k, w.dtype)
    names = []
    for v in (B.rmsnorm_variants_ag if w.gather else B.rmsnorm_variants)(w.dtype):
        if a.variant_filter and not any(f in v for f in a.variant_filter.split("|")):
            continue
        with B.forced(v):
            try:
                plan(w.rows, w.hidden, w.k, w.dtype)
                names.append(v)
            except B.RmsnormError:
                pass
    times = {v: [] for v in names}
    for rep in range(a.repeat):
        for v in names:
            with B.forced(v):
                for i in range(a.warmup):
                    step(i)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(a.steps):
                    step(i)
                e1.record()
                torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / a.steps * 1e3
            times[v].append(us)
            print(f"[sweep {rep}] {us:9.2f} us {w.algorithmic_bytes() / us / 1e3:7.0f} GB/s  {v}"
                  f"{'  <- dispatcher' if v == default else ''}", file=sys.stderr, flush=True)
    rows = sorted((statistics.median(t), v, t) for v, t in times.items())
    for us, v, t in rows:
        print(json.dumps({"workload": w.name, "variant": v, "us": round(us, 3),
                          "gbs": round(w.algorithmic_bytes() / us / 1e3, 1),
                          "runs_us": [round(x, 2) for x in t], "dispatcher": v == default}))
    return 0


# read/write mixes of the ceiling sweep: (name, read streams, write streams
# given as indices into the buffers -- an index below the read count writes
# that read stream in place)
CEILING_PATTERNS = [
    ("read 1", 1, []), ("read 2", 2, []), ("write 1", 0, [0]), ("write 2", 0, [0, 1]),
    ("copy 1R1W", 1, [1]), ("2R2W distinct", 2, [2, 3]),
    ("2R2W, one write in place (fused K=1)", 2, [1, 2]),
    ("2R2W, both writes in place", 2, [1, 0]),
    ("9R2W, one write in place (fused K=8)", 9, [8, 9]),
]


CEILING_GRIDS = (256, 384, 512, 768, 1024, 2048, 4096, 8192, 16384)
CEILING_POLICIES = 9  # libstreamprobe.so's cache policies (stream_probe_policy)


def ceiling_sweep(stream_mib: int = 64, steps: int = 40, patterns: str = "",
                  policies: str = "", rotate_gib: float = 1.0) -> int:
    """Time libstreamprobe.so over every read/write mix above (or those whose
    name contains one of the |-separated ``patterns``), every grid, workgroup
    size, unroll, layout and cache policy it offers; streams of stream_mib MiB
    rotated through >= 1 GiB.  One JSON line per configuration."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "row_wise_normalization_rmsnorm_amd", "libstreamprobe.so"))
    vp = ctypes.c_void_p
    lib.stream_probe_pol.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(vp),
                                     ctypes.c_int, ctypes.c_int64, vp, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    cpol = {}
    for pol in range(CEILING_POLICIES):
        lb, sb = ctypes.c_int(), ctypes.c_int()
        if lib.stream_probe_policy(pol, ctypes.byref(lb), ctypes.byref(sb)) != 0:
            raise RuntimeError(f"stream_probe_policy({pol}) failed")
        cpol[pol] = (("global " if pol == 0 else "buffer ") + cpol_name(lb.value),
                     ("global " if pol == 0 else "buffer ") + cpol_name(sb.value))
    pols = [int(x) for x in policies.split(",")] if policies else list(range(CEILING_POLICIES))
    nbytes = stream_mib << 20
    n16 = nbytes // 16
    sink = torch.zeros(64, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    for name, nr, writes in CEILING_PATTERNS:
        if patterns and not any(f in name for f in patterns.split("|")):
            continue
        nbuf = max([nr] + [j + 1 for j in writes])
        nsets = max(1, int(-(-rotate_gib * (1 << 30) // (nbuf * nbytes))))
        bufs = [[torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(j + 1)
                 for j in range(nbuf)] for _ in range(nsets)]
        args = [((vp * max(nr, 1))(*[t.data_ptr() for t in b[:nr]]),
                 (vp * max(len(writes), 1))(*[b[j].data_ptr() for j in writes])) for b in bufs]
        moved = (nr + len(writes)) * nbytes
        best = None
        shapes = [(g, b, u, c, p) for p in pols for c in (0, 1) for g in CEILING_GRIDS
                  for b in (256, 512, 1024) for u in (1, 2, 4, 8)]
        for grid, block, unroll, contig, pol in shapes:
            def launch(i):
                ra, wa = args[i % nsets]
                rc = lib.stream_probe_pol(ra, nr, wa, len(writes), n16, sink.data_ptr(),
                                          grid, block, unroll, contig, pol, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"stream_probe_pol failed: {rc}")
            for i in range(3):
                launch(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(steps):
                launch(i)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            row = {"pattern": name, "reads": nr, "writes": len(writes), "rotating_sets": nsets,
                   "in_place": sum(j < nr for j in writes), "grid": grid, "block": block,
                   "unroll": unroll, "layout": "contiguous" if contig else "grid-stride",
                   "policy": pol, "load_policy": cpol[pol][0], "store_policy": cpol[pol][1],
                   "us": round(us, 3), "gbs": round(moved / us / 1e3, 1)}
            print(json.dumps(row), flush=True)
            if best is None or row["gbs"] > best["gbs"]:
                best = row
        print(f"[ceiling] {name}: best {best['gbs']} GB/s (grid {best['grid']}, block "
              f"{best['block']}, unroll {best['unroll']}, {best['layout']}, loads "
              f"{best['load_policy']}, stores {best['store_policy']})", file=sys.stderr,
              flush=True)
        del bufs
        torch.cuda.empty_cache()
    return 0


def cpol_name(bits: int) -> str:
    """The cache-policy bits of a vector memory instruction, as the assembler
    spells them (bit 0 sc0, bit 1 nt, bit 4 sc1); "default" for none."""
    names = [n for b, n in ((1, "sc0"), (16, "sc1"), (2, "nt")) if bits & b]
    return " ".join(names) if names else "default"


DESIGN_NAMES = {0: "one row per workgroup, residual stored before the reduction",
                1: "one row per workgroup, residual stored after the reduction",
                2: "one row per workgroup, rows in contiguous eighths per XCD",
                3: "persistent, next row's loads issued before this row's work",
                4: "two rows per 1024-lane workgroup",
                5: "phased: two rows per wave, all loads before any store",
                6: "phased: four rows per wave, all loads before any store",
                7: "phased: one row per wave, all loads before any store"}


def design_sweep(a) -> int:
    """Time the row-kernel designs of librowprobe.so (4096-wide bf16 rows, one
    partial) beside the library's kernel on the same rotating buffers: every
    design and cache-policy pair it is built with, the persistent design at
    several grids.  Each is first checked against the library's kernel on one
    set (residual bit for bit, output within 2 ulp).  Designs are timed
    round-robin over ``--repeat`` rounds; the median is reported, one JSON
    line each."""
    import ctypes
    import statistics
    import torch
    from row_wise_normalization_rmsnorm_amd import binding as B
    from row_wise_normalization_rmsnorm_amd.workloads import WORKLOADS
    w = WORKLOADS["add_rmsnorm_bf16_8192x4096_k1"]
    rows = a.rows or w.rows
    lib = ctypes.CDLL(os.path.join(ROOT, "row_wise_normalization_rmsnorm_amd", "librowprobe.so"))
    vp = ctypes.c_void_p
    lib.row_probe.argtypes = [ctypes.c_int] * 4 + [vp] * 4 + [ctypes.c_int64, ctypes.c_float, vp]
    lp, sp = (ctypes.c_int * 16)(), (ctypes.c_int * 16)()
    npol = lib.row_probe_policies(lp, sp, 16)
    pols = [(lp[i], sp[i]) for i in range(npol)]
    dev = "cuda:0"
    H = w.hidden
    g = (torch.rand(H, device=dev) + 0.5).to(torch.bfloat16)
    tb = rows * H * 2
    nsets = max(1, int(-(-a.rotate_bytes * (1 << 30) // (3 * tb))))
    gen = torch.Generator(device=dev).manual_seed(0)
    sets = [(torch.randn(rows, H, device=dev, generator=gen).to(torch.bfloat16),
             torch.randn(rows, H, device=dev, generator=gen).to(torch.bfloat16),
             torch.empty(rows, H, device=dev, dtype=torch.bfloat16)) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream

    def probe(design, l, s_, grid):
        def step(i):
            x, r, o = sets[i % nsets]
            rc = lib.row_probe(design, l, s_, grid, x.data_ptr(), r.data_ptr(), o.data_ptr(),
                               g.data_ptr(), rows, w.eps, sid)
            if rc != 0:
                raise RuntimeError(f"row_probe({design}, {l}, {s_}, {grid}) failed: {rc}")
        return step

    def library(i):
        x, r, o = sets[i % nsets]
        B.add_rmsnorm_fwd(o, r, [x], g, w.eps)

    variants = {("library", B.rmsnorm_plan(rows, H, 1, "bf16"), "", 0): library}
    for d in (0, 1, 2, 4):
        for l, s_ in pols:
            grid = rows // 2 if d == 4 else rows
            variants[(d, DESIGN_NAMES[d], f"{l}/{s_}", grid)] = probe(d, l, s_, grid)
    for grid in (256, 512, 1024, 2048):
        for l, s_ in pols:
            if s_ in (2, 19):
                variants[(3, DESIGN_NAMES[3], f"{l}/{s_}", grid)] = probe(3, l, s_, grid)
    for d, per in ((5, 8), (6, 16), (7, 4)):
        for l, s_ in pols:
            grid = -(-rows // per)
            variants[(d, DESIGN_NAMES[d], f"{l}/{s_}", grid)] = probe(d, l, s_, grid)

    def ulps(t):
        i = t.view(torch.int16).int()
        return torch.where(i < 0, -(i & 0x7FFF), i)

    x0, r0, _ = sets[0]
    r_init = r0.clone()
    ref_r, ref_o = r0.clone(), torch.empty_like(r0)
    B.add_rmsnorm_fwd(ref_o, ref_r, [x0], g, w.eps)
    for key, f in variants.items():
        sets[0][1].copy_(r_init)
        f(0)
        torch.cuda.synchronize()
        same_r = torch.equal(sets[0][1].view(torch.int16), ref_r.view(torch.int16))
        d_ulp = int((ulps(sets[0][2]) - ulps(ref_o)).abs().max())
        if not same_r or d_ulp > 2:
            raise RuntimeError(f"design {key} differs from the library: residual exact "
                               f"{same_r}, output {d_ulp} ulp")
    print(f"[design] {len(variants)} variants agree with the library's kernel; timing "
          f"({nsets} rotating sets of {3 * tb / 2**20:.0f} MiB)", file=sys.stderr, flush=True)
    times = {k: [] for k in variants}
    for rep in range(a.repeat):
        for key, f in variants.items():
            for i in range(2 * nsets):
                f(i)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(a.steps):
                f(i)
            e1.record(stream)
            torch.cuda.synchronize()
            times[key].append(e0.elapsed_time(e1) / a.steps * 1e3)
        print(f"[design] round {rep} done", file=sys.stderr, flush=True)
    nbytes = rows * H * 2 * 4 + H * 2
    for key, t in times.items():
        us = statistics.median(t)
        print(json.dumps({"workload": f"{w.name}" if rows == w.rows else f"{w.name}_rows{rows}",
                          "rows": rows, "design": key[0], "what": key[1], "cpol": key[2],
                          "grid": key[3], "us": round(us, 3),
                          "gbs": round(nbytes / us / 1e3, 1), "rotating_sets": nsets,
                          "runs_us": [round(x, 2) for x in t]}), flush=True)
    return 0


def grid_cap_sweep(a) -> int:
    """Time the dispatcher's kernel for a fused K = 1 workload (default the
    8192 x 4096 one; --workload picks another) with its grid capped at
    several workgroup counts (rmsnorm_tune's grid cap: the workgroups then
    loop over the rows) beside the uncapped grid of one workgroup per row,
    on buffers rotated over --rotate-bytes GiB.  Caps are timed round-robin
    over --repeat rounds of --steps launches; the median is reported, one
    JSON line each."""
    import statistics
    import torch
    from row_wise_normalization_rmsnorm_amd import binding as B
    from row_wise_normalization_rmsnorm_amd.workloads import WORKLOADS
    w = WORKLOADS[a.workload or "add_rmsnorm_bf16_8192x4096_k1"]
    if w.op != "add_rmsnorm" or w.k != 1 or w.dtype != "bf16":
        raise SystemExit("--grid-cap-sweep takes a fused bf16 workload with one partial")
    rows, H = a.rows or w.rows, w.hidden
    dev = "cuda:0"
    tb = rows * H * 2
    nsets = max(1, int(-(-a.rotate_bytes * (1 << 30) // (3 * tb))))
    gen = torch.Generator(device=dev).manual_seed(0)
    g = (torch.rand(H, device=dev, generator=gen) + 0.5).to(torch.bfloat16)
    sets = [(torch.randn(rows, H, device=dev, generator=gen).to(torch.bfloat16),
             torch.randn(rows, H, device=dev, generator=gen).to(torch.bfloat16),
             torch.empty(rows, H, device=dev, dtype=torch.bfloat16)) for _ in range(nsets)]
    plan = B.rmsnorm_plan(rows, H, 1, "bf16")
    caps = [0] + [c for c in (256, 512, 1024, 2048, 4096, 8192, 16384) if c < rows]
    stream = torch.cuda.current_stream()

    def step(i):
        x, r, o = sets[i % nsets]
        B.add_rmsnorm_fwd(o, r, [x], g, w.eps)

    times = {c: [] for c in caps}
    for rep in range(a.repeat):
        for c in caps:
            with B.forced(None, c):
                for i in range(2 * nsets):
                    step(i)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(a.steps):
                    step(i)
                e1.record(stream)
                torch.cuda.synchronize()
                times[c].append(e0.elapsed_time(e1) / a.steps * 1e3)
        print(f"[grid-cap] round {rep} done", file=sys.stderr, flush=True)
    nbytes = rows * H * 2 * 4 + H * 2
    for c, t in times.items():
        us = statistics.median(t)
        print(json.dumps({"workload": w.name if rows == w.rows else f"{w.name}_rows{rows}",
                          "kernel": plan, "grid_cap": c or None, "us": round(us, 3),
                          "gbs": round(nbytes / us / 1e3, 1), "rotating_sets": nsets,
                          "runs_us": [round(x, 2) for x in t]}), flush=True)
    return 0


GEMM_DESIGNS = {0: "4 waves, 64-wide k stages in 2 LDS buffers, LDS reads and loads spread "
                    "between the products",
                 1: "4 waves, 64-wide k stages in 2 LDS buffers, LDS reads and loads in one "
                    "block before the products",
                 2: "4 waves, 32-wide k stages in {nbuf} LDS buffers (loads {nbuf} stages ahead), "
                    "spread",
                 3: "design 2 persistent: one workgroup per CU, pipeline across tiles, "
                    "results stored from registers"}
GEMM_MODES = {0: "the product", 1: "operands always in L2 (every workgroup computes tile 0)",
              2: "no loads in the loop", 3: "products only (no loads, no LDS reads in the loop)",
              4: "loads, no LDS reads in the loop"}


def gemm_design_sweep(a) -> int:
    """Time the 4-wave GEMM designs of libgemmprobe.so beside the library's
    kernel and torch.matmul (hipBLASLt) on the same rotating operands of a
    GEMM workload (default the 4096 x 8192 x 3584 bf16 one).  Every design is
    first checked bit for bit against the library's 256 x 256 kernel on the
    workload and on a ragged shape.  Design 2's timing modes (which skip
    work, so their results are not checked) and the library and hipBLASLt are
    also timed with k doubled, which takes each time apart into a part that
    grows with k and a fixed part.  Timed round-robin over --repeat rounds;
    one JSON line per variant with the median."""
    import ctypes
    import statistics
    import torch
    from row_wise_normalization_rmsnorm_amd import binding as B
    from row_wise_normalization_rmsnorm_amd import inputs as I
    from row_wise_normalization_rmsnorm_amd.workloads import GEMM_WORKLOADS, GEMM_HEADLINE, GemmWorkload

    w0 = GEMM_WORKLOADS[a.workload or GEMM_HEADLINE]
    dev = "cuda:0"
    dt = {"bf16": 2, "f16": 1}[w0.dtype]
    lib = ctypes.CDLL(os.path.join(ROOT, "row_wise_normalization_rmsnorm_amd", "libgemmprobe.so"))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.gemm_probe.argtypes = [ctypes.c_int] * 3 + [vp, i64, ctypes.c_int, vp, i64, vp, i64,
                                                    i64, i64, i64, ctypes.c_int, vp]
    sid = torch.cuda.current_stream().cuda_stream

    def probe(design, mode, nbuf, dst, x, y):
        ptrs = (ctypes.c_void_p * len(dst))(*[t.data_ptr() for t in dst])
        rc = lib.gemm_probe(design, mode, nbuf, ptrs, dst[0].stride(0), len(dst), x.data_ptr(),
                            x.stride(0), y.data_ptr(), y.stride(0), x.shape[0], y.shape[0],
                            x.shape[1], dt, sid)
        if rc != 0:
            raise RuntimeError(f"gemm_probe({design}, {mode}, {nbuf}) failed: {rc}")

    designs = [(0, 0, 0), (1, 0, 0), (2, 0, 4), (2, 0, 5), (3, 0, 4), (3, 0, 5)]
    # correctness: the workload's operands, and a ragged shape (partial tiles,
    # k not a multiple of 64, chunks not a multiple of the tile)
    d = I.gemm_inputs(w0)
    gen = torch.Generator().manual_seed(5)
    tdt = d["a"].dtype
    checks = [(w0.world, d["a"].to(dev), d["b"].to(dev)),
              (8, torch.randn(520, 3576, generator=gen).to(tdt).to(dev),
               torch.randn(768, 3576, generator=gen).to(tdt).to(dev))]
    for world, x, y in checks:
        m, n = x.shape[0], y.shape[0]
        ref = [torch.empty(m // world, n, dtype=tdt, device=dev) for _ in range(world)]
        B.gemm_scatter_fwd(ref, x, y, tile_n=B.GEMM_SCATTER_TILE_N)
        for design, mode, nbuf in designs:
            out = [torch.full((m // world, n), float("nan"), dtype=tdt, device=dev)
                   for _ in range(world)]
            probe(design, mode, nbuf, out, x, y)
            torch.cuda.synchronize()
            if not torch.equal(torch.cat(out).view(torch.int16), torch.cat(ref).view(torch.int16)):
                raise RuntimeError(f"design {design} (nbuf {nbuf}) differs from the library on "
                                   f"{m}x{n}x{x.shape[1]}")
    del checks
    print(f"[gemm-design] {len(designs)} designs agree with the library bit for bit",
          file=sys.stderr, flush=True)

    variants = {}
    groups = []
    for kmul in (1, 2):
        w = GemmWorkload(w0.name if kmul == 1 else f"{w0.name}_k{w0.k * kmul}", w0.dtype, w0.m,
                         w0.n, w0.k * kmul, w0.world)
        dk = d if kmul == 1 else I.gemm_inputs(w)
        nsets = max(1, int(-(-a.rotate_bytes * (1 << 30) // w.algorithmic_bytes())))
        sets = [(dk["a"].to(dev), dk["b"].to(dev),
                 [torch.empty(w.m // w.world, w.n, dtype=tdt, device=dev) for _ in range(w.world)])
                for _ in range(nsets)]
        groups.append((w, sets))

        def lib_step(i, sets=sets, nsets=nsets):
            x, y, o = sets[i % nsets]
            B.gemm_scatter_fwd(o, x, y)

        def blas_step(i, sets=sets, nsets=nsets):
            x, y, _ = sets[i % nsets]
            torch.matmul(x, y.t())

        def pstep(design, mode, nbuf, sets=sets, nsets=nsets):
            def f(i):
                x, y, o = sets[i % nsets]
                probe(design, mode, nbuf, o, x, y)
            return f

        tn = B.gemm_scatter_tile_n(w.m, w.n)
        tm = B.gemm_scatter_tile_m(w.m, w.n, tn)
        variants[(w.k, "library", f"gemm_scatter, {tm}x{tn} tiles, 4 waves", -1, 0)] = (w, lib_step)
        variants[(w.k, "hipBLASLt", "torch.matmul(a, b.t())", -1, 0)] = (w, blas_step)
        for mode in range(5):
            variants[(w.k, 2, GEMM_DESIGNS[2].format(nbuf=4), mode, 4)] = (w, pstep(2, mode, 4))
        if kmul == 1:
            for design, mode, nbuf in designs:
                if design != 2 or nbuf != 4:
                    variants[(w.k, design, GEMM_DESIGNS[design].format(nbuf=nbuf), mode, nbuf)] = \
                        (w, pstep(design, mode, nbuf))
    stream = torch.cuda.current_stream()
    times = {key: [] for key in variants}
    for rep in range(a.repeat):
        for key, (w, f) in variants.items():
            for i in range(10):
                f(i)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(a.steps):
                f(i)
            e1.record(stream)
            torch.cuda.synchronize()
            times[key].append(e0.elapsed_time(e1) / a.steps * 1e3)
        print(f"[gemm-design] round {rep} done", file=sys.stderr, flush=True)
    for key, t in times.items():
        w = variants[key][0]
        us = statistics.median(t)
        print(json.dumps({"workload": w0.name, "k": key[0], "design": key[1], "what": key[2],
                          "mode": key[3], "mode_what": GEMM_MODES.get(key[3], ""),
                          "nbuf": key[4], "us": round(us, 2),
                          "tflops": round(w.flops() / (us * 1e-6) / 1e12, 1),
                          "runs_us": [round(x, 2) for x in t]}), flush=True)
    return 0


def copy_calibration() -> None:
    """A plain device copy of known size (1 GiB), for scaling the HBM byte
    counters read by rocprofv3 --pmc."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="time the plain streaming probe over read/write mixes and launch "
                         "shapes (one JSON line each) and exit")
    ap.add_argument("--ceiling-patterns", default="",
                    help="ceiling sweep: only the mixes whose name contains one of these "
                         "|-separated substrings")
    ap.add_argument("--ceiling-policies", default="",
                    help="ceiling sweep: comma-separated cache policies (default: all)")
    ap.add_argument("--grid-cap-sweep", action="store_true",
                    help="time the fused K = 1 workload's kernel with its grid capped at "
                         "256-16384 workgroups beside one workgroup per row")
    ap.add_argument("--design-sweep", action="store_true",
                    help="time the alternative row-kernel designs of librowprobe.so beside the "
                         "library's kernel (4096-wide bf16 rows, one partial) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="time every compiled kernel variant that can run the workload "
                         "(forced through rmsnorm_tune) and print one line per variant")
    ap.add_argument("--repeat", type=int, default=1, help="sweep rounds (median reported)")
    ap.add_argument("--variant-filter", default="",
                    help="sweep only variants containing one of these |-separated substrings")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-ceiling probe")
    ap.add_argument("--rows", type=int, default=0,
                    help="run the workload with this many rows instead (not a headline figure)")
    ap.add_argument("--inplace", action="store_true",
                    help="write the output over the first input instead of a separate buffer")
    ap.add_argument("--rotate-bytes", type=float, default=2.0,
                    help="GiB of distinct buffers rotated through (cold cache)")
    ap.add_argument("--gemm-design-sweep", action="store_true",
                    help="time the 4-wave GEMM designs of libgemmprobe.so beside the library's "
                         "kernel and hipBLASLt (one JSON line each)")
    ap.add_argument("--gemm-shapes", action="store_true",
                    help="time the GEMM with the scatter epilogue over a list of shapes against "
                         "torch.matmul (one JSON line each) and exit")
    ap.add_argument("--resident-context", action="store_true",
                    help="GEMM workloads: also time the kernel and the library on one set of "
                         "operands (cache-resident)")
    a = ap.parse_args()

    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              "(rows are independent: each further GPU would run the same kernel on its own "
              "share of the rows, with no communication)",
              file=sys.stderr)
        return 2

    import torch
    from row_wise_normalization_rmsnorm_amd import binding as B
    from row_wise_normalization_rmsnorm_amd import inputs as I
    from row_wise_normalization_rmsnorm_amd.workloads import HEADLINE, WORKLOADS

    if a.copy_calibration:
        copy_calibration()
        return 0
    if a.ceiling_sweep:
        return ceiling_sweep(patterns=a.ceiling_patterns, policies=a.ceiling_policies,
                             rotate_gib=a.rotate_bytes)
    if a.design_sweep:
        return design_sweep(a)
    if a.grid_cap_sweep:
        return grid_cap_sweep(a)

    from row_wise_normalization_rmsnorm_amd.workloads import GEMM_WORKLOADS
    if a.gemm_design_sweep:
        return gemm_design_sweep(a)
    if a.gemm_shapes:
        return gemm_shapes(a)
    if a.workload in GEMM_WORKLOADS:
        return gemm_bench(a, a.workload)
    w = WORKLOADS[a.workload or HEADLINE]
    if a.inplace and w.gather:
        print("bench.py: --inplace does not apply to the all-gather form (its outputs are "
              "separate buffers by definition)", file=sys.stderr)
        return 2
    if a.rows:  # the same workload with another row count (footprint studies)
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}_rows{a.rows}", rows=a.rows)
    dev = "cuda:0"
    B.lib()
    print(f"[bench] {w.describe()}: generating inputs", file=sys.stderr, flush=True)
    base = I.make_inputs(w, device=dev)
    # distinct device bytes of one set of buffers: every input tensor, the
    # residual (read and written in place, counted once) and each output
    # (the output shares the first input's memory with --inplace)
    tensor = w.rows * w.hidden * w.itemsize
    if w.op == "block_sum":
        set_bytes = tensor
    elif w.fused:
        set_bytes = (w.k + 1 + (w.gather or (0 if a.inplace else 1))) * tensor
    else:
        set_bytes = (1 if a.inplace else 2) * tensor
    nsets = max(1, int(-(-a.rotate_bytes * (1 << 30) // set_bytes)))
    sets = []
    for i in range(nsets):
        s = {k: ([t.clone() for t in v] if isinstance(v, list) else v.clone())
             for k, v in base.items()}
        if w.op == "block_sum":
            s["x"] = s["x"].reshape(-1)
            s["out"] = torch.empty(1, device=dev,
                                   dtype=torch.int32 if w.dtype == "i8" else torch.float32)
        elif w.gather:
            s["outs"] = [torch.empty_like(s["residual"]) for _ in range(w.gather)]
        else:
            if a.inplace:  # the output written over the (first) input, as the fused
                s["out"] = s["partials"][0] if w.fused else s["x"]  # kernel of the pages does
            else:
                s["out"] = torch.empty_like(s["residual"] if w.fused else s["x"])
        sets.append(s)
    del base
    if w.op == "block_sum":
        if a.sweep:
            print("bench.py: --sweep applies to the RMSNorm kernels only", file=sys.stderr)
            return 2
        kernel = f"block_sum<{w.dtype}>"
        ws = B.block_sum_workspace(dev)
    elif w.gather:
        kernel = B.rmsnorm_plan_ag(w.rows, w.hidden, w.k, w.dtype)
    else:
        kernel = B.rmsnorm_plan(w.rows, w.hidden, w.k, w.dtype)

    def step(i):
        s = sets[i % nsets]
        if w.op == "block_sum":
            B.block_all_reduce_sum_fwd(s["out"], s["x"], ws)
        elif w.gather:
            B.add_rmsnorm_ag_fwd(s["outs"], s["residual"], s["partials"], s["gamma"], w.eps)
        elif w.fused:
            B.add_rmsnorm_fwd(s["out"], s["residual"], s["partials"], s["gamma"], w.eps)
        else:
            B.rmsnorm_fwd(s["out"], s["x"], s["gamma"], w.eps)

    if a.sweep:
        return sweep(w, step, a, B)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / a.steps
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    rows_per_s = w.rows / (ms * 1e-3)
    print(f"[bench] {kernel}: {ms * 1e3:.2f} us/launch, {gbs:.0f} GB/s "
          f"({100 * gbs / HBM_PEAK_GBS:.1f}% of peak), {rows_per_s:.3g} rows/s, "
          f"{nsets} rotating sets, wall {wall:.2f}s", file=sys.stderr, flush=True)

    # Context beside the graded number: the spread of single launches, and
    # for inputs far smaller than the 256 MB Infinity Cache the same with a
    # 1 GiB cache flush before each launch.
    lat = {"batched": latency(step, min(a.steps, 200))}
    if nbytes < (64 << 20):
        lat["flushed"] = latency(step, min(a.steps, 100), flush_bytes=1 << 30)
        lat["sync"] = sync_latency(step, min(a.steps, 100))
        lat["graph"] = graph_replay(step, min(a.steps, 200))
    for kind, l in lat.items():
        print(f"[bench] per-launch ({kind}): {json.dumps(l)}", file=sys.stderr, flush=True)

    # the all-gather form against the same work unfused: add_rmsnorm_fwd into
    # the first output, then device copies of it into the others
    unfused = None
    if w.gather:
        def unfused_step(i):
            s = sets[i % nsets]
            B.add_rmsnorm_fwd(s["outs"][0], s["residual"], s["partials"], s["gamma"], w.eps)
            for o in s["outs"][1:]:
                o.copy_(s["outs"][0])

        for i in range(5):
            unfused_step(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(a.steps):
            unfused_step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ums = e0.elapsed_time(e1) / a.steps
        unfused = {"what": f"add_rmsnorm_fwd, then {w.gather - 1} device copies of its output",
                   "us": round(ums * 1e3, 2), "fused_speedup": round(ums / ms, 3)}
        print(f"[bench] unfused (add_rmsnorm_fwd + {w.gather - 1} copies): {ums * 1e3:.2f} us, "
              f"fused {ms * 1e3:.2f} us", file=sys.stderr, flush=True)

    traffic = traffic_for(kernel, w.name, w.op)
    metric = ("achieved HBM GB/s (% of peak) + rows/s, add_rmsnorm bf16 8192x4096"
              if w.name == HEADLINE else f"achieved HBM GB/s (% of peak) + rows/s, {w.describe()}")
    result = {
        "metric": metric,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic the path computes in (fp32 adds, FMAs and scale on
        # 16-bit storage; int32 for the int8 sum); the tensors' dtype beside it
        "dtype": "i32" if w.dtype == "i8" else "f32",
        "storage_dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) / U(0.5,1.5) inputs, resident in HBM)",
        "config": {"workload": w.name, "op": w.op, "rows": w.rows, "hidden": w.hidden,
                   "k": w.k, "eps": w.eps, "kernel": kernel, "rotating_sets": nsets,
                   "out_over_input": bool(a.inplace),
                   "algorithmic_bytes_per_step": nbytes},
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "rows_per_s": round(rows_per_s, 1),
        "elements_per_s": round(w.rows * w.hidden / (ms * 1e-3), 1),
        "per_launch": lat,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if unfused:
        result["unfused_context"] = unfused
    if not a.no_ceiling:
        del sets
        torch.cuda.empty_cache()
        ceil = stream_ceiling(w, inplace=a.inplace, rotate_gib=a.rotate_bytes)
        ceil["kernel_frac_of_ceiling"] = round(gbs / ceil["value"], 4)
        result["stream_ceiling"] = ceil
        print(f"[bench] streaming ceiling for this mix: {ceil['value']:.0f} GB/s; kernel at "
              f"{100 * ceil['kernel_frac_of_ceiling']:.1f}% of it", file=sys.stderr, flush=True)
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
