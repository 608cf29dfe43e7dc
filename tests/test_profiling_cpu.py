"""Host logic of the measurement tools, on the CPU: the rocprofv3 CSV
parsing and summaries in profiling.py, and bench.py's refusal of more than
one GPU.  Synthetic CSV files stand in for rocprofv3 output."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

from row_wise_normalization_rmsnorm_amd import profiling as prof

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_launch_gaps_and_kernel_stats(tmp_path):
    d = tmp_path / "trace"
    hdr = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [["KERNEL_DISPATCH", "copyBuffer", 0, 50],
            ["KERNEL_DISPATCH", "row_vgpr_kernel<...>", 100, 1100],
            ["KERNEL_DISPATCH", "row_vgpr_kernel<...>", 1150, 2150],
            ["KERNEL_DISPATCH", "row_vgpr_kernel<...>", 2150, 3170],
            ["KERNEL_DISPATCH", "other", 3200, 3300],
            ["KERNEL_DISPATCH", "row_vgpr_kernel<...>", 3400, 4400]]
    _write_csv(str(d / "run_kernel_trace.csv"), hdr, rows[::-1])   # any order
    med_dur, med_gap, pairs = prof.launch_gaps(str(d), "row_vgpr_kernel")
    assert pairs == 2 and med_gap == 25.0     # gaps 50 and 0; the pair across "other" is skipped
    assert med_dur == 1000.0                  # durations 1000, 1000, 1020 (the last has no successor)
    _write_csv(str(d / "run_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [["row_vgpr_kernel<...>", 4, 1005.0, 1000, 1020, 99.0]])
    st = prof.kernel_stats(str(d))
    assert st[0]["avg_ns"] == 1005.0 and st[0]["calls"] == 4


def test_counter_median_and_missing_kernel(tmp_path):
    d = tmp_path / "pmc"
    _write_csv(str(d / "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["k_a", "FETCH_SIZE", 10.0], ["k_a", "FETCH_SIZE", 30.0], ["k_a", "FETCH_SIZE", 20.0],
                ["k_b", "FETCH_SIZE", 99.0], ["k_a", "WRITE_SIZE", 5.0]])
    assert prof.counter(str(d), "FETCH_SIZE", "k_a") == (20.0, 3)
    with pytest.raises(ValueError):
        prof.counter(str(d), "FETCH_SIZE", "k_c")


def test_traffic_summary_scales_counters_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE reading half of a copy's bytes gets scale 2; the summary
    and the JSON report bytes per launch in the algorithmic units."""
    monkeypatch.setattr(prof, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    w = "rmsnorm_f32_512x2048"
    t, fe, wr, cf, cw = (tmp_path / n for n in ("t", "f", "w", "cf", "cw"))
    _write_csv(str(t / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs",
                                                "Percentage"], [["row_vgpr_kernel<x>", 3, 4000, 3900, 4100, 90]])
    _write_csv(str(t / "run_kernel_trace.csv"), ["Kind", "Kernel_Name", "Start_Timestamp",
                                                "End_Timestamp"], [["K", "row_vgpr_kernel<x>", 0, 4000]])
    algo = 512 * 2048 * 4 * 2 + 2048 * 4
    _write_csv(str(fe / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["row_vgpr_kernel<x>", "FETCH_SIZE", 512 * 2048 * 4 / 1024 / 2]])
    _write_csv(str(wr / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["row_vgpr_kernel<x>", "WRITE_SIZE", 512 * 2048 * 4 / 1024]])
    _write_csv(str(cf / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["__amd_rocclr_copyBuffer", "FETCH_SIZE", (1 << 30) / 1024 / 2]])
    _write_csv(str(cw / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["__amd_rocclr_copyBuffer", "WRITE_SIZE", (1 << 30) / 1024]])
    argv = ["profiling", "--workload", w, "--plan", "vgpr<f32,x>", "--symbol", "row_vgpr_kernel",
            "--trace", str(t), "--fetch", str(fe), "--write", str(wr), "--copy-fetch", str(cf),
            "--copy-write", str(cw)]
    monkeypatch.setattr(sys, "argv", argv)
    assert prof.main() == 0
    d = json.load(open(tmp_path / "profiles" / f"traffic_{w}.json"))
    assert d["read_bytes"] == 512 * 2048 * 4 and d["write_bytes"] == 512 * 2048 * 4
    assert d["algorithmic_bytes"] == algo
    md = open(tmp_path / "profiles" / f"vgpr_f32_x__{w}.md").read()
    assert "4.00" in md and "scale" in md


def test_ceiling_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(prof, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    lines = [{"pattern": "read 1", "reads": 1, "writes": 0, "in_place": 0, "grid": g, "block": 256,
              "unroll": 4, "layout": lay, "us": 1.0, "gbs": v, "policy": pol,
              "load_policy": lp, "store_policy": sp}
             for g, lay, v, pol, lp, sp in (
                 (1024, "grid-stride", 5000.0, 0, "global nt", "global nt"),
                 (2048, "contiguous", 5100.0, 0, "global nt", "global nt"),
                 (4096, "grid-stride", 6000.0, 0, "global nt", "global nt"),
                 (512, "grid-stride", 6100.0, 5, "buffer sc0 sc1 nt", "buffer sc0 sc1 nt"))]
    src = tmp_path / "c.jsonl"
    src.write_text("\n".join(json.dumps(x) for x in lines) + "\n")
    assert prof.ceiling_summary([str(src)]) == 0
    md = open(tmp_path / "profiles" / "hbm_ceiling_sweep.md").read()
    # best overall (policy 5 at grid 512), best with policy 0, median of the four
    assert ("| read 1 | 1 | 0 (0) | 6100 | 76.2 | 512, 256, 4, grid-stride | buffer sc0 sc1 nt / "
            "buffer sc0 sc1 nt | 6000 | 5550 |") in md
    # per grid, in grid order
    assert "| read 1 | 6100 | 5000 | 5100 | 6000 |" in md
    # per policy
    assert "| read 1 | 6000 | 6100 |" in md


def test_gemm_design_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(prof, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    wl = "gemm_scatter_bf16_4096x8192x3584_w8"

    def row(k, design, mode, nbuf, us):
        return {"workload": wl, "k": k, "design": design, "what": f"w{design}", "mode": mode,
                "mode_what": "m" if mode > 0 else "", "nbuf": nbuf, "us": us,
                "tflops": 1.0, "runs_us": [us]}
    lines = [row(3584, "library", -1, 0, 200.0), row(7168, "library", -1, 0, 380.0),
             row(3584, "hipBLASLt", -1, 0, 160.0), row(7168, "hipBLASLt", -1, 0, 305.0),
             row(3584, 2, 0, 4, 190.0), row(7168, 2, 0, 4, 360.0),
             row(3584, 2, 3, 4, 130.0), row(7168, 2, 3, 4, 235.0),
             row(3584, 3, 0, 5, 250.0)]
    src = tmp_path / "g.jsonl"
    src.write_text("\n".join(json.dumps(x) for x in lines) + "\n")
    assert prof.gemm_design_summary([str(src)]) == 0
    md = open(tmp_path / "profiles" / f"gemm_design_sweep__{wl}.md").read()
    # ranking at the smaller k: timing modes left out, library marked
    assert "| 1 | hipBLASLt: w" in md and "| 2 | design 2: w2 | 190.0" in md
    assert "| 3 | **library: wlibrary** | 200.0 | 1 | 1.000x |" in md
    assert "| 4 | design 3 (5 LDS buffers): w3 | 250.0 | 1 | 0.800x |" in md
    # growing part t(2k) - t(k) and fixed part t(k) - growing part
    assert "| library | - | 200.0 | 380.0 | 180.0 | 20.0 |" in md
    assert "| design 2 | m | 130.0 | 235.0 | 105.0 | 25.0 |" in md


def test_report_reads_whole_tensor_statistics(tmp_path, monkeypatch):
    """The per-workload report takes each workload's parity statistics from
    the GPU tests' log, including the whole-tensor lines of the full-size
    workloads, and leaves "see tests" where the log has none."""
    monkeypatch.setattr(prof, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(tmp_path / "profiles")
    log = tmp_path / "tests.log"
    log.write_text(
        "[gpu] add_rmsnorm_bf16_8192x4096_k1: every row against the oracle\n"
        "[gpu] add_rmsnorm_bf16_8192x4096_k1: whole tensor {'rows_checked': 8192, "
        "'elements_checked': 33554432, 'residual_bit_exact': True, 'max_ulp': 1, "
        "'max_rel_err': 0.0039}\n"
        "[gpu] rmsnorm_f32_512x2048: {'max_rel_err': 2.2e-07}\n"
        "[gpu] block_sum_f32_1024x1024: error / bound = 1.5e-05\n")

    def line(name, op="add_rmsnorm"):
        return json.dumps({"config": {"workload": name, "op": op}, "ms_per_step": 0.05,
                           "value": 6000.0, "pct_of_peak": 75.0, "rows_per_s": 1.8e8,
                           "cpu_baseline": {"value": 2.0, "cores": 16, "rows_per_s": 6e4,
                                            "single_thread": {"value": 0.15}}})
    paths = []
    for i, (name, op) in enumerate((("add_rmsnorm_bf16_8192x4096_k1", "add_rmsnorm"),
                                    ("rmsnorm_f32_512x2048", "rmsnorm"),
                                    ("block_sum_f32_1024x1024", "block_sum"),
                                    ("add_rmsnorm_bf16_4096x8192_k8", "add_rmsnorm"))):
        f = tmp_path / f"b{i}.json"
        f.write_text(line(name, op) + "\n")
        paths.append(str(f))
    assert prof.report_summary(["--tests-log", str(log)] + paths) == 0
    md = open(tmp_path / "profiles" / "per_config_report.md").read()
    assert ("| add_rmsnorm_bf16_8192x4096_k1 |" in md and
            "max 1 ulp, rel 0.0039, residual bit-exact (33,554,432 elements) |" in md)
    assert "| max rel 2.2e-07 |" in md
    assert "| error / bound 1.5e-05 |" in md
    assert md.count("| see tests |") == 1


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments_not_code():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* fast */ }\n"
    b = "/* header */\nint f(int x) {\n  return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }"
    assert prof.code_only(a) == prof.code_only(b)
    assert prof.code_only(a) != prof.code_only(c)
    assert len(prof.source_hash("rmsnorm")) == 64
    assert prof.source_hash("rmsnorm") != prof.source_hash("block_sum")
