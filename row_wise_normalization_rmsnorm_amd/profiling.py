"""Turn rocprofv3 output into the short summaries kept under profiles/.

Inputs (CSV, from ``rocprofv3 --output-format csv``):
  * a kernel trace with ``--stats``: ``<dir>/<name>_kernel_stats.csv``;
  * two counter runs of the same workload, ``--pmc FETCH_SIZE`` and
    ``--pmc WRITE_SIZE``: ``<dir>/<name>_counter_collection.csv``;
  * the same two counters over ``bench.py --copy-calibration`` (a plain 1 GiB
    device copy), which fixes the scale of each counter on this GPU.

Writes ``profiles/<kernel>__<workload>.md`` (average duration, achieved
bandwidth, HBM bytes per launch, with the commands) and
``profiles/traffic_<workload>.json`` (read by bench.py, tied to a hash of the
kernel sources so that a stale figure is never reported).

Usage: python -m row_wise_normalization_rmsnorm_amd.profiling --workload W
         --plan NAME --symbol SUBSTR --trace DIR --fetch DIR --write DIR
         --copy-fetch DIR --copy-write DIR [--bench-json FILE]
       python -m row_wise_normalization_rmsnorm_amd.profiling sweep --workload W FILE.jsonl
       python -m row_wise_normalization_rmsnorm_amd.profiling counters --workload W
         --plan NAME --symbol SUBSTR DIR
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")   # where the summaries are written
COPY_BYTES = 1 << 30


def kernel_sources(op: str) -> list:
    """The sources that fix a workload's kernel code: the block sum's file,
    the GEMM's file and its shared header, or the RMSNorm kernels' template
    header.  Which variant runs is
    checked by its name instead, which spells out every template parameter,
    so adding other variants or changing the host dispatcher leaves a
    measured figure valid."""
    pkg = os.path.join(ROOT, "row_wise_normalization_rmsnorm_amd")
    src = {"block_sum": ["block_sum.hip"],
           "gemm_scatter": ["gemm_scatter.hip", "gemm_scatter_kernels.hpp"]}.get(
        op, ["rmsnorm_kernels.hpp"])
    return [os.path.join(pkg, "csrc", f) for f in src]


def source_hash(op: str) -> str:
    """sha256 over the kernel source of ``op`` (its code, not its comments)
    and the compiler flags it is built with: a traffic figure taken on other
    code is stale."""
    import sys
    sys.path.insert(0, ROOT)
    from row_wise_normalization_rmsnorm_amd.build import FLAGS
    h = hashlib.sha256()
    for p in kernel_sources(op):
        h.update(code_only(open(p).read()).encode())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def code_only(src: str) -> str:
    """C++ source without comments and with whitespace collapsed, so that
    editing a comment does not change the hash."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def _one(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(d: str):
    rows = list(csv.DictReader(open(_one(d, "kernel_stats.csv"))))
    out = []
    for r in rows:
        out.append({"name": r["Name"], "calls": int(r["Calls"]),
                    "avg_ns": float(r["AverageNs"]), "min_ns": float(r["MinNs"]),
                    "max_ns": float(r["MaxNs"]), "pct": float(r["Percentage"])})
    return out


def launch_gaps(d: str, kernel_substr: str):
    """From the kernel trace: (median duration, median idle gap between one
    dispatch of the kernel and the next when nothing else ran between them,
    number of such pairs), in ns."""
    rows = list(csv.DictReader(open(_one(d, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs, gaps = [], []
    for a, b in zip(rows, rows[1:]):
        if kernel_substr in a["Kernel_Name"]:
            durs.append(int(a["End_Timestamp"]) - int(a["Start_Timestamp"]))
            if kernel_substr in b["Kernel_Name"]:
                gaps.append(int(b["Start_Timestamp"]) - int(a["End_Timestamp"]))
    if not durs:
        return None
    return statistics.median(durs), (statistics.median(gaps) if gaps else float("nan")), len(gaps)


def counter(d: str, name: str, kernel_substr: str):
    rows = list(csv.DictReader(open(_one(d, "counter_collection.csv"))))
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == name and kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise ValueError(f"{name}: no dispatch of a kernel matching {kernel_substr!r} in {d}")
    return statistics.median(vals), len(vals)


def short_name(plan: str) -> str:
    return re.sub(r"[^A-Za-z0-9]+", "_", plan).strip("_")


def sweep_summary(argv) -> int:
    """profiles/sweep__<workload>.md from the JSON lines of
    ``bench.py --workload W --sweep --repeat R``."""
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", default=None)
    ap.add_argument("jsonl")
    a = ap.parse_args(argv)
    rows = [json.loads(l) for l in open(a.jsonl) if l.startswith("{")]
    rows.sort(key=lambda r: r["us"])
    md = os.path.join(PROFILES, f"sweep__{a.workload}.md")
    with open(md, "w") as f:
        f.write(f"# Every compiled variant on {a.workload}\n\n")
        cmd = a.command or (f"python bench.py --workload {a.workload} --sweep --repeat 3")
        f.write(f"Command: `{cmd}` (HIP events over the timed launches of each variant, forced "
                "through rmsnorm_tune; variants timed round-robin, median of the rounds; "
                "buffers rotated as in the benchmark).\n\n")
        f.write("| rank | variant | median us | GB/s | rounds (us) | dispatcher |\n|---|---|---|---|---|---|\n")
        for i, r in enumerate(rows):
            if i < 15 or r["dispatcher"]:
                f.write(f"| {i + 1} | `{r['variant']}` | {r['us']:.2f} | {r['gbs']:.0f} | "
                        f"{', '.join(f'{x:.2f}' for x in r['runs_us'])} | "
                        f"{'yes' if r['dispatcher'] else ''} |\n")
        f.write(f"\n{len(rows)} variants can run this workload; the 15 fastest and the "
                "dispatcher's choice are listed.\n")
    print(md)
    return 0


def ceiling_summary(argv) -> int:
    """profiles/hbm_ceiling_sweep.md from the JSON lines of
    ``bench.py --ceiling-sweep``: the best launch shape of the plain
    streaming probe for every read/write mix, the best per grid size and per
    cache policy, and the spread over shapes."""
    ap = argparse.ArgumentParser()
    ap.add_argument("jsonl")
    ap.add_argument("--command", default="python bench.py --ceiling-sweep")
    ap.add_argument("--name", default="hbm_ceiling_sweep")
    a = ap.parse_args(argv)
    rows = [json.loads(l) for l in open(a.jsonl) if l.startswith("{")]
    order = []
    for r in rows:
        if r["pattern"] not in order:
            order.append(r["pattern"])
    grids = sorted({r["grid"] for r in rows})
    pols = sorted({(r.get("policy", 0), r.get("load_policy", "global nt"),
                    r.get("store_policy", "global nt")) for r in rows})
    md = os.path.join(PROFILES, a.name + ".md")
    nsets = sorted({r.get("rotating_sets", 0) for r in rows})
    with open(md, "w") as f:
        f.write("# HBM ceiling of a plain streaming kernel, by read/write mix\n\n")
        f.write(f"Command: `{a.command}` (libstreamprobe.so: 16-byte loads and stores, every lane "
                "`unroll` chunks in flight per stream; 64 MiB per stream, buffers rotated through "
                f"{'/'.join(map(str, nsets))} sets; HIP events over 40 launches per shape).  Swept: grid "
                f"{grids[0]}-{grids[-1]} workgroups ({', '.join(map(str, grids))}), workgroup "
                "256/512/1024 lanes, unroll 1/2/4/8, two layouts -- a grid-stride loop, or each "
                "workgroup streaming one contiguous range -- and the cache policies below "
                f"({len(rows) // max(1, len(order))} shapes per mix).  Policy 0 is the "
                "global_load/store_dwordx4 pair with the nontemporal bit, as the RMSNorm kernels "
                "issue them; the others are buffer_load/store_dwordx4 with the named "
                "cache-policy bits.\n\n")
        f.write("| mix | reads | writes (in place) | best GB/s | % of 8 TB/s | best shape "
                "(grid, block, unroll, layout) | best policy (loads / stores) | best with policy 0 "
                "GB/s | median over shapes GB/s |\n|---|---|---|---|---|---|---|---|---|\n")
        for name in order:
            rs = [r for r in rows if r["pattern"] == name]
            b = max(rs, key=lambda r: r["gbs"])
            p0 = [r["gbs"] for r in rs if r.get("policy", 0) == 0]
            med = statistics.median(r["gbs"] for r in rs)
            f.write(f"| {name} | {b['reads']} | {b['writes']} ({b['in_place']}) | {b['gbs']:.0f} | "
                    f"{b['gbs'] / 80:.1f} | {b['grid']}, {b['block']}, {b['unroll']}, "
                    f"{b.get('layout', 'grid-stride')} | {b.get('load_policy', 'global nt')} / "
                    f"{b.get('store_policy', 'global nt')} | {max(p0) if p0 else float('nan'):.0f} | "
                    f"{med:.0f} |\n")
        f.write("\n## Best GB/s per grid size (over workgroup size, unroll, layout and policy)\n\n")
        f.write("| mix | " + " | ".join(str(g) for g in grids) + " |\n|---|"
                + "---|" * len(grids) + "\n")
        for name in order:
            cells = []
            for g in grids:
                v = [r["gbs"] for r in rows if r["pattern"] == name and r["grid"] == g]
                cells.append(f"{max(v):.0f}" if v else "")
            f.write(f"| {name} | " + " | ".join(cells) + " |\n")
        f.write("\n## Best GB/s per cache policy (over every launch shape)\n\n")
        f.write("| mix | " + " | ".join(f"{p}: {l} / {s_}" for p, l, s_ in pols) + " |\n|---|"
                + "---|" * len(pols) + "\n")
        for name in order:
            cells = []
            for p, _, _ in pols:
                v = [r["gbs"] for r in rows if r["pattern"] == name and r.get("policy", 0) == p]
                cells.append(f"{max(v):.0f}" if v else "")
            f.write(f"| {name} | " + " | ".join(cells) + " |\n")
        f.write(f"\n{len(rows)} configurations timed.\n")
    print(md)
    return 0


def design_summary(argv) -> int:
    """profiles/design_sweep__<workload>.md from the JSON lines of
    ``bench.py --design-sweep``: every row-kernel design and cache policy
    beside the library's kernel, fastest first."""
    ap = argparse.ArgumentParser()
    ap.add_argument("jsonl")
    ap.add_argument("--command", default="python bench.py --design-sweep --repeat 3 --steps 100")
    a = ap.parse_args(argv)
    rows = [json.loads(l) for l in open(a.jsonl) if l.startswith("{")]
    lib = next(r for r in rows if r["design"] == "library")
    wl = lib["workload"]
    md = os.path.join(PROFILES, f"design_sweep__{wl}.md")
    with open(md, "w") as f:
        f.write(f"# Row-kernel designs on {wl}\n\n")
        f.write(f"Command: `{a.command}` (librowprobe.so's designs for 4096-wide bf16 rows with "
                "one partial, each checked against the library's kernel first -- residual bit "
                "for bit, output within 2 ulp -- then timed round-robin with HIP events over "
                f"the launches, median of the rounds; {lib['rotating_sets']} rotating buffer "
                "sets).  cpol = cache-policy bits of the loads / stores (1 sc0, 2 nt, 16 sc1).  "
                "% of peak counts the algorithmic bytes against 8 TB/s.\n\n")
        f.write("| rank | design | cpol (loads / stores) | grid | median us | GB/s | % of 8 TB/s "
                "| vs the library's kernel |\n|---|---|---|---|---|---|---|---|\n")
        for i, r in enumerate(sorted(rows, key=lambda r: r["us"])):
            what = (f"**library: `{r['what']}`**" if r["design"] == "library"
                    else f"{r['design']}: {r['what']}")
            f.write(f"| {i + 1} | {what} | {r['cpol']} | {r['grid']} | {r['us']:.2f} | "
                    f"{r['gbs']:.0f} | {r['gbs'] / 80:.1f} | {lib['us'] / r['us']:.3f}x |\n")
        f.write(f"\n{len(rows)} kernels timed.\n")
    print(md)
    return 0


COUNTERS = ["SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES",
            "TCC_HIT_sum", "TCC_MISS_sum"]


def gemm_design_summary(argv) -> int:
    """profiles/gemm_design_sweep__<workload>.md from the JSON lines of
    ``bench.py --gemm-design-sweep``: the 4-wave designs beside the library's
    kernel and hipBLASLt, and the time taken apart by design 2's modes at k
    and 2k (the part that grows with k, and the fixed rest)."""
    ap = argparse.ArgumentParser()
    ap.add_argument("jsonl")
    ap.add_argument("--command", default="python bench.py --gemm-design-sweep --repeat 3 --steps 50")
    a = ap.parse_args(argv)
    rows = [json.loads(l) for l in open(a.jsonl) if l.startswith("{")]
    wl = rows[0]["workload"]
    k1 = min(r["k"] for r in rows)
    k2 = max(r["k"] for r in rows)
    md = os.path.join(PROFILES, f"gemm_design_sweep__{wl}.md")
    lib = next(r for r in rows if r["design"] == "library" and r["k"] == k1)
    with open(md, "w") as f:
        f.write(f"# GEMM designs on {wl}\n\n")
        f.write(f"Command: `{a.command}` (libgemmprobe.so's designs; each checked bit for bit "
                "against the library's 256 x 256 kernel on the workload and on a ragged "
                "520 x 768 x 3576 product before timing; timed round-robin with HIP events over "
                "back-to-back launches on rotating operand sets, median of the rounds).  "
                "TFLOP/s counts 2 m n k; the dense bf16 matrix-core peak is 2500.\n\n")
        f.write(f"## Designs at k = {k1}\n\n| rank | kernel | median us | TFLOP/s | vs the library |\n"
                "|---|---|---|---|---|\n")
        first = [r for r in rows if r["k"] == k1 and r["mode"] in (0, -1)]
        for i, r in enumerate(sorted(first, key=lambda r: r["us"])):
            if r["design"] == "library":
                name = f"**library: {r['what']}**"
            elif r["design"] == "hipBLASLt":
                name = f"hipBLASLt: {r['what']}"
            else:
                bufs = f" ({r['nbuf']} LDS buffers)" if r["design"] == 3 else ""
                name = f"design {r['design']}{bufs}: {r['what']}"
            f.write(f"| {i + 1} | {name} | {r['us']:.1f} | {r['tflops']:.0f} | "
                    f"{lib['us'] / r['us']:.3f}x |\n")
        f.write(f"\n## Where the time goes: design 2 (4 buffers) by mode, at k = {k1} and {k2}\n\n"
                f"The part that grows with k is t({k2}) - t({k1}), for {k2 - k1} more k; the "
                f"fixed part is the rest of t({k1}).  Modes 1-4 skip work and give wrong "
                "results; they only take the time apart.\n\n"
                f"| kernel | mode | us at k = {k1} | us at k = {k2} | growing part, us per "
                f"{k2 - k1} k | fixed part, us |\n|---|---|---|---|---|---|\n")
        keyed = {}
        for r in rows:
            keyed.setdefault((r["design"], r["mode"], r["nbuf"]), {})[r["k"]] = r
        order = [("library", -1, 0), ("hipBLASLt", -1, 0)] + [(2, m, 4) for m in range(5)]
        for key in order:
            if key not in keyed or k1 not in keyed[key] or k2 not in keyed[key]:
                continue
            r1, r2 = keyed[key][k1], keyed[key][k2]
            slope = r2["us"] - r1["us"]
            name = key[0] if isinstance(key[0], str) else f"design {key[0]}"
            f.write(f"| {name} | {r1['mode_what'] or '-'} | {r1['us']:.1f} | {r2['us']:.1f} | "
                    f"{slope:.1f} | {r1['us'] - slope * k1 / (k2 - k1):.1f} |\n")
        f.write(f"\n{len(rows)} kernels timed.\n")
    print(md)
    return 0


def report_summary(argv) -> int:
    """profiles/per_config_report.md: for every workload, the GPU figures and
    the oracle's CPU rate (many cores and one) from ``bench.py --workload W``
    JSON lines, beside the parity statistics the GPU tests print ("[gpu]
    NAME: {stats}" lines of a ``pytest -s`` log)."""
    import ast
    ap = argparse.ArgumentParser()
    ap.add_argument("--tests-log", required=True)
    ap.add_argument("bench_json", nargs="+")
    a = ap.parse_args(argv)
    stats = {}
    for line in open(a.tests_log, errors="replace"):
        m = re.search(r"\[gpu\] (\w+): (?:whole tensor )?(\{.*\})\s*$", line)
        if m:
            try:
                stats[m.group(1)] = ast.literal_eval(m.group(2))
            except (ValueError, SyntaxError):
                pass
        m = re.search(r"\[gpu\] (\w+): error / bound = ([0-9.e+-]+)", line)
        if m:
            stats[m.group(1)] = {"error_over_bound": float(m.group(2))}
    rows, gemm_rows = [], []
    for path in a.bench_json:
        for line in open(path):
            if line.startswith("{"):
                d = json.loads(line)
                (gemm_rows if d["config"].get("op") == "gemm_scatter" else rows).append(d)
    md = os.path.join(PROFILES, "per_config_report.md")
    with open(md, "w") as f:
        f.write("# Per-workload report: GPU kernel, CPU oracle, parity\n\n")
        f.write("Commands: `python bench.py --workload W --no-ceiling` for every workload (the GPU "
                "step timed with HIP events; the oracle timed on the host's cores, and on one), and "
                "`python -m pytest tests/test_gpu_parity.py tests/test_gpu_allgather.py tests/test_gpu_block_sum.py "
                "tests/test_gpu_gemm_scatter.py -m gpu -s -k \"workloads or full_size\"` for the "
                "parity statistics (every row of every RMSNorm workload against the oracle, the "
                "full-size ones in row blocks; the elements checked are counted in the column).\n\n")
        f.write("| workload | GPU µs/step | GPU GB/s | % of 8 TB/s | GPU rows/s | oracle GB/s "
                "(cores) | oracle rows/s | oracle GB/s, 1 core | GPU ÷ oracle | parity |\n"
                "|---|---|---|---|---|---|---|---|---|---|\n")
        for r in rows:
            w = r["config"]["workload"]
            cb = r.get("cpu_baseline", {})
            st = stats.get(w, {})
            if "max_ulp" in st:
                par = (f"max {st['max_ulp']} ulp, rel {st.get('max_rel_err', 0):.2g}"
                       + (", residual bit-exact" if st.get("residual_bit_exact") else "")
                       + (f" ({st['elements_checked']:,} elements)" if "elements_checked" in st else ""))
            elif "max_rel_err" in st:
                par = (f"max rel {st['max_rel_err']:.2g}"
                       + (", residual bit-exact" if st.get("residual_bit_exact") else ""))
            elif "error_over_bound" in st:
                par = f"error / bound {st['error_over_bound']:.2g}"
            else:
                par = "see tests"
            one = cb.get("single_thread", {})
            f.write(f"| {w} | {r['ms_per_step'] * 1e3:.2f} | {r['value']:.0f} | "
                    f"{r['pct_of_peak']:.1f} | {r['rows_per_s']:.3g} | {cb.get('value', float('nan')):.3g} "
                    f"({cb.get('cores', '-')}) | {cb.get('rows_per_s', float('nan')):.3g} | "
                    f"{one.get('value', float('nan')):.3g} | "
                    f"{r['value'] / cb['value'] if cb.get('value') else float('nan'):.0f} | {par} |\n")
        if gemm_rows:
            f.write("\nGEMM with the reduce-scatter epilogue (bound by the matrix cores; the "
                    "library column is hipBLASLt's plain GEMM on the same rotated operands; parity "
                    "from `tests/test_gpu_gemm_scatter.py -k full_size`, every row of every "
                    "chunk):\n\n| workload | GPU µs/step | TFLOP/s | % of 2.5 PFLOP/s | hipBLASLt "
                    "µs | oracle TFLOP/s (cores) | oracle TFLOP/s, 1 core | GPU ÷ oracle | parity "
                    "|\n|---|---|---|---|---|---|---|---|---|\n")
            for r in gemm_rows:
                w = r["config"]["workload"]
                cb = r.get("cpu_baseline", {})
                one = cb.get("single_thread", {})
                st = stats.get(w, {})
                par = (f"error / bound max {st['max_error_over_bound']:.2g}, "
                       f"{100 * st['min_equal_frac']:.2f}%+ equal to the oracle's rounding "
                       f"({st['rows_checked']} rows"
                       + (f", {st['elements_checked']:,} elements)" if "elements_checked" in st else ")")
                       if "max_error_over_bound" in st
                       else "see tests")
                lib = r.get("library_context", {})
                f.write(f"| {w} | {r['ms_per_step'] * 1e3:.2f} | {r['value']:.1f} | "
                        f"{r['pct_of_peak']:.1f} | {lib.get('us', float('nan')):.1f} | "
                        f"{cb.get('value', float('nan')):.3g} ({cb.get('cores', '-')}) | "
                        f"{one.get('value', float('nan')):.3g} | "
                        f"{r['value'] / cb['value'] if cb.get('value') else float('nan'):.0f} | "
                        f"{par} |\n")
        f.write("\nThe oracle is the plain double-precision reference (test infrastructure), timed "
                "as it stands: a baseline, not a target.\n")
    print(md)
    return 0


def counters_summary(argv) -> int:
    """profiles/counters_<kernel>__<workload>.md from one rocprofv3 --pmc run
    of COUNTERS (LDS use and bank conflicts, waves, L2 hits and misses)."""
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--plan", required=True)
    ap.add_argument("--symbol", required=True)
    ap.add_argument("dir")
    a = ap.parse_args(argv)
    vals = {}
    for n in COUNTERS:
        try:
            vals[n] = counter(a.dir, n, a.symbol)
        except ValueError:
            pass
    md = os.path.join(PROFILES, f"counters_{short_name(a.plan)}__{a.workload}.md")
    with open(md, "w") as f:
        f.write(f"# LDS, wave and L2 counters: {a.plan} on {a.workload}\n\n")
        f.write("Command: `rocprofv3 --pmc " + " ".join(COUNTERS) + " --output-format csv -d <dir> "
                f"-o run -- python bench.py --workload {a.workload} --steps 5 --warmup 1 "
                "--no-cpu-baseline --no-ceiling`\n\n| counter | per dispatch (median) | dispatches |\n"
                "|---|---|---|\n")
        for n, (v, c) in vals.items():
            f.write(f"| {n} | {v:,.0f} | {c} |\n")
        if {"SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES"} <= set(vals):
            lds, conf, waves = (vals[n][0] for n in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
                                                     "SQ_WAVES"))
            f.write(f"\nLDS instructions per wave: {lds / waves:.1f}; bank-conflict cycles per "
                    f"wave: {conf / waves:.1f} ({conf / max(lds, 1):.2f} per LDS instruction).\n")
        if {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(vals):
            hit, miss = vals["TCC_HIT_sum"][0], vals["TCC_MISS_sum"][0]
            f.write(f"L2 (TCC) requests per dispatch: {hit + miss:,.0f}, hit rate "
                    f"{hit / max(hit + miss, 1):.3f}.  Hits include gamma, which every "
                    f"workgroup reads from L2; whether data comes from HBM more than once is "
                    f"settled by FETCH_SIZE / WRITE_SIZE in the traffic summary.\n")
        op = ("block_sum" if "block_sum" in a.symbol else
              "gemm_scatter" if "gemm_scatter" in a.symbol else "rmsnorm")
        f.write(f"\nKernel sources sha256: `{source_hash(op)}`\n")
    print(md)
    return 0


def gemm_counters_summary(argv) -> int:
    """profiles/counters_<kernel>__<workload>.md for a GEMM workload: the
    counters of one or more rocprofv3 --pmc runs (each ``counters=dir``) for
    the kernel and, side by side, for the vendor library's GEMM that bench.py
    runs on the same operands as context."""
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--plan", required=True)
    ap.add_argument("--symbol", required=True)
    ap.add_argument("--library-symbol", default="Cijk")
    ap.add_argument("runs", nargs="+", help="COUNTER,COUNTER,...=dir")
    a = ap.parse_args(argv)
    rows = []
    cmds = []
    for run in a.runs:
        names, d = run.split("=", 1)
        names = names.split(",")
        cmds.append("rocprofv3 --pmc " + " ".join(names) + " --output-format csv -d <dir> -o run "
                    f"-- python bench.py --workload {a.workload} --steps 10 --warmup 2 "
                    "--no-cpu-baseline")
        for n in names:
            mine = counter(d, n, a.symbol)
            try:
                lib = counter(d, n, a.library_symbol)[0]
            except ValueError:
                lib = None
            rows.append((n, mine[0], mine[1], lib))
    md = os.path.join(PROFILES, f"counters_{short_name(a.plan)}__{a.workload}.md")
    with open(md, "w") as f:
        f.write(f"# Matrix-core, LDS and wait counters: {a.plan} on {a.workload}\n\n")
        f.write("Commands:\n\n" + "".join(f"* `{c}`\n" for c in cmds) + "\n")
        f.write("The library column is hipBLASLt's GEMM (`Cijk_...`), which bench.py runs on the "
                "same operands as context.\n\n| counter | kernel, per dispatch (median) | "
                "dispatches | hipBLASLt, per dispatch (median) |\n|---|---|---|---|\n")
        for n, v, c, lib in rows:
            f.write(f"| {n} | {v:,.0f} | {c} | {'' if lib is None else f'{lib:,.0f}'} |\n")
        f.write(f"\nKernel sources sha256: `{source_hash('gemm_scatter')}`\n")
    print(md)
    return 0


def gemm_shapes_summary(argv) -> int:
    """profiles/gemm_scatter_bf16_shapes.md from ``bench.py --gemm-shapes``."""
    ap = argparse.ArgumentParser()
    ap.add_argument("jsonl")
    a = ap.parse_args(argv)
    rows = [json.loads(l) for l in open(a.jsonl) if l.startswith("{")]
    md = os.path.join(PROFILES, "gemm_scatter_bf16_shapes.md")
    with open(md, "w") as f:
        f.write("# GEMM with the scatter epilogue across shapes (bf16)\n\n")
        f.write("Command: `python bench.py --gemm-shapes` (HIP events over back-to-back launches, "
                "operands rotated over about 1 GiB, 100 ms of warm-up, every tile shape and the "
                "library timed round-robin over three rounds, median; the library column is "
                "torch.matmul, i.e. hipBLASLt's plain GEMM, on the same operands).  One workgroup "
                "per output tile on 256 CUs.  The automatic width takes 128-wide tiles only where "
                "they need no more rounds of 256 workgroups than 256-wide ones; the 256-wide tiles "
                "are 256, 192 or 160 rows high by an estimate of their rounds' cost "
                "(include/gemm_scatter.h).  Every tile shape gives bitwise the same results.\n\n")
        f.write("| m | n | k | chunks | automatic tile | tiles | kernel µs | TFLOP/s | "
                "% of 2.5 PFLOP/s | 256x256 µs | 192x256 µs | 160x256 µs | 256x128 µs | "
                "hipBLASLt µs | hipBLASLt TFLOP/s | kernel ÷ hipBLASLt |\n"
                "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        for r in rows:
            bt = r.get("by_tile", {})
            if not bt and "by_tile_n" in r:   # lines of the earlier format (heights of 256 only)
                bt = {f"256x{k}": v for k, v in r["by_tile_n"].items()}
            cell = lambda key: f"{bt[key]['us']:.1f}" if key in bt else "–"
            f.write(f"| {r['m']} | {r['n']} | {r['k']} | {r['world']} | "
                    f"{r.get('tile_m', 256)}x{r.get('tile_n', 256)} | "
                    f"{r['tiles']} | {r['us']:.1f} | {r['tflops']:.0f} | "
                    f"{100 * r['tflops'] / 2500:.1f} | {cell('256x256')} | {cell('192x256')} | "
                    f"{cell('160x256')} | {cell('256x128')} | "
                    f"{r['library_us']:.1f} | {r['library_tflops']:.0f} | "
                    f"{r['library_us'] / r['us']:.2f} |\n")
        f.write(f"\nKernel sources sha256: `{source_hash('gemm_scatter')}`\n")
    print(md)
    return 0


def main() -> int:
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "gemm-shapes":
        return gemm_shapes_summary(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "gemm-counters":
        return gemm_counters_summary(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "sweep":
        return sweep_summary(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        return counters_summary(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "ceiling":
        return ceiling_summary(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "design":
        return design_summary(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "gemm-design":
        return gemm_design_summary(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "report":
        return report_summary(sys.argv[2:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--plan", required=True, help="kernel variant name (bench.py prints it)")
    ap.add_argument("--symbol", required=True, help="substring of the kernel's mangled name")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--bench-json", default=None, help="bench.py output line (for the event timing)")
    a = ap.parse_args()

    import sys
    sys.path.insert(0, ROOT)
    from row_wise_normalization_rmsnorm_amd.workloads import GEMM_WORKLOADS, WORKLOADS
    w = WORKLOADS[a.workload] if a.workload in WORKLOADS else GEMM_WORKLOADS[a.workload]
    gemm = w.op == "gemm_scatter"
    nbytes = w.algorithmic_bytes()

    stats = kernel_stats(a.trace)
    mine = [s for s in stats if a.symbol in s["name"]]
    if not mine:
        raise SystemExit(f"kernel {a.symbol} not in trace")
    k = mine[0]
    fetch_kib, nf = counter(a.fetch, "FETCH_SIZE", a.symbol)
    write_kib, nw = counter(a.write, "WRITE_SIZE", a.symbol)
    cf_kib, _ = counter(a.copy_fetch, "FETCH_SIZE", "copyBuffer")
    cw_kib, _ = counter(a.copy_write, "WRITE_SIZE", "copyBuffer")
    fscale = COPY_BYTES / 1024 / cf_kib
    wscale = COPY_BYTES / 1024 / cw_kib
    read_b = fetch_kib * fscale * 1024
    write_b = write_kib * wscale * 1024
    traffic = read_b + write_b
    achieved = nbytes / (k["avg_ns"] * 1e-9) / 1e9
    event = None
    if a.bench_json and os.path.exists(a.bench_json):
        for line in open(a.bench_json):
            if line.startswith("{"):
                event = json.loads(line)

    name = short_name(a.plan)
    os.makedirs(PROFILES, exist_ok=True)
    md = os.path.join(PROFILES, f"{name}__{w.name}.md")
    with open(md, "w") as f:
        f.write(f"# {a.plan} on {w.name}\n\n")
        what = ("each element read once, the 4-byte sum written once" if w.op == "block_sum"
                else "A, B read once, the output written once" if gemm
                else "each tensor element read or written once, gamma once")
        f.write(f"Workload: {w.describe()}; algorithmic bytes per launch {nbytes:,} "
                f"({what}).\n\n")
        f.write("## Kernel trace (rocprofv3 --kernel-trace --stats)\n\n")
        f.write("Command: `rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                f"python bench.py --workload {w.name} --no-cpu-baseline`\n\n")
        f.write("| kernel | calls | avg us | min us | max us | % time |\n|---|---|---|---|---|---|\n")
        for s in stats[:4]:
            f.write(f"| {s['name'][:90]} | {s['calls']} | {s['avg_ns'] / 1e3:.2f} | "
                    f"{s['min_ns'] / 1e3:.2f} | {s['max_ns'] / 1e3:.2f} | {s['pct']:.1f} |\n")
        if gemm:
            f.write("\nThe `Cijk_...` kernel is hipBLASLt's GEMM, which bench.py runs on the same "
                    "rotated operands as context; it is not part of the path.\n")
        if gemm:
            tflops = w.flops() / (k["avg_ns"] * 1e-9) / 1e12
            f.write(f"\nAchieved ({w.flops():,} flop / average duration): **{tflops:.1f} "
                    f"TFLOP/s**, {100 * tflops / 2500:.1f}% of the 2.5 PFLOP/s dense "
                    f"{w.dtype} matrix-core peak; {achieved:.0f} GB/s of algorithmic bytes.\n")
        else:
            f.write(f"\nAchieved (algorithmic bytes / average duration): **{achieved:.0f} GB/s**, "
                    f"{100 * achieved / 8000:.1f}% of the 8 TB/s HBM peak.\n")
        gaps = launch_gaps(a.trace, a.symbol)
        if gaps:
            f.write(f"Back-to-back launches in the trace: median duration {gaps[0] / 1e3:.2f} us, "
                    f"median idle gap to the next launch {gaps[1] / 1e3:.2f} us ({gaps[2]} pairs; "
                    f"a gap means the host, slowed further by the profiler, issued launches "
                    f"more slowly than the kernel ran).\n")
        if event:
            f.write(f"bench.py (HIP events over the timed region, same command without the "
                    f"profiler): {event['ms_per_step'] * 1e3:.2f} us per launch, "
                    f"{event['value']:.{1 if gemm else 0}f} {event['unit']}.\n")
        f.write("\n## HBM bytes (rocprofv3 --pmc, one counter per run)\n\n")
        f.write("Commands: `rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python "
                f"bench.py --workload {w.name} --steps 10 --warmup 2 --no-cpu-baseline --no-ceiling`, "
                "the same "
                "with `--pmc WRITE_SIZE`, and both counters over `python bench.py "
                "--copy-calibration` (1 GiB device copy).\n\n")
        f.write("| counter | KiB per dispatch (median) | dispatches | copy-calibration KiB for "
                "1 GiB | scale | bytes per launch |\n|---|---|---|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {fetch_kib:,.1f} | {nf} | {cf_kib:,.1f} | {fscale:.4f} | "
                f"{read_b:,.0f} |\n")
        f.write(f"| WRITE_SIZE | {write_kib:,.1f} | {nw} | {cw_kib:,.1f} | {wscale:.4f} | "
                f"{write_b:,.0f} |\n")
        f.write(f"\nHBM traffic per launch {traffic:,.0f} B = {traffic / nbytes:.4f} x the "
                "algorithmic bytes" + (" (operand tiles fetched again by other workgroups "
                                       "once evicted from the L2 / Infinity Cache)" if gemm
                                       else "") + ".\n")
        f.write(f"\nKernel sources sha256: `{source_hash(w.op)}`\n")
    tj = os.path.join(PROFILES, f"traffic_{w.name}.json")
    json.dump({"workload": w.name, "kernel": a.plan, "traffic_bytes_per_launch": round(traffic),
               "read_bytes": round(read_b), "write_bytes": round(write_b),
               "algorithmic_bytes": nbytes, "fetch_kib": fetch_kib, "write_kib": write_kib,
               "copy_fetch_kib_per_gib": cf_kib, "copy_write_kib_per_gib": cw_kib,
               "avg_kernel_ns": k["avg_ns"], "source_sha256": source_hash(w.op)},
              open(tj, "w"), indent=1)
    print(md)
    print(tj)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
