"""Build librmsnorm.so in-tree with hipcc for gfx950.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), the objects are linked into ``librmsnorm.so`` next to this file,
and the device assembly of every kernel is checked: no packed-fp32 VALU
instructions (they are disabled by a target-feature flag) and no kernel that
spills registers to scratch memory (either fails the build).

Usage: ``python -m row_wise_normalization_rmsnorm_amd.build [-j N] [-v]``.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librmsnorm.so")
PROBE_SRC = os.path.join(HERE, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(HERE, "libstreamprobe.so")
ROW_PROBE_SRC = os.path.join(HERE, "probe", "row_probe.hip")
ROW_PROBE_LIB = os.path.join(HERE, "librowprobe.so")
GEMM_PROBE_SRC = os.path.join(HERE, "probe", "gemm_probe.hip")
GEMM_PROBE_LIB = os.path.join(HERE, "libgemmprobe.so")
FASTCALL_SRC = os.path.join(HERE, "pyext", "fastcall.c")
FASTCALL_LIB = os.path.join(HERE, "_fastcall.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # packed fp32 VALU forms are disabled; the compiler emits scalar fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-save-temps",
]
FORBIDDEN = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def _compile(src: str, verbose: bool) -> str:
    name = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(os.path.dirname(HERE), "include"),
           "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def check_assembly() -> dict:
    """Scan the saved device assembly: forbid packed-fp32 VALU forms and
    report per-kernel VGPR / spill counts."""
    usage = {}
    for s in glob.glob(os.path.join(BUILD, f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s")):
        text = open(s).read()
        m = FORBIDDEN.search(text)
        if m:
            raise RuntimeError(f"{os.path.basename(s)} contains {m.group(0)}")
        for km in re.finditer(r"^\s+\.name:\s+(\S+)\s*$", text, re.M):
            pass
        for blk in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
            name, body = blk.group(1), blk.group(2)
            vg = re.search(r"\.amdhsa_next_free_vgpr (\d+)", body)
            sc = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body)
            usage[name] = (int(vg.group(1)) if vg else -1, int(sc.group(1)) if sc else -1)
    return usage


def build(jobs: int = 0, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    # the measurement aids used by bench.py (separate libraries): the
    # bandwidth-ceiling probe and the row-kernel and GEMM design probes
    for src, lib in ((PROBE_SRC, PROBE_LIB), (ROW_PROBE_SRC, ROW_PROBE_LIB),
                     (GEMM_PROBE_SRC, GEMM_PROBE_LIB)):
        ptmp = lib + ".tmp%d" % os.getpid()
        pcmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-fPIC", "-shared", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", ptmp, src]
        r = subprocess.run(pcmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"probe build failed for {src}:\n" + r.stdout + r.stderr)
        os.replace(ptmp, lib)
    # the binding's argument marshalling for the per-step calls (host C)
    import sysconfig
    ftmp = FASTCALL_LIB + ".tmp%d" % os.getpid()
    fcmd = ["gcc", "-O2", "-shared", "-fPIC", "-Wall", "-Wextra", "-Wno-cast-function-type",
            "-I", sysconfig.get_paths()["include"], "-o", ftmp, FASTCALL_SRC, "-ldl"]
    r = subprocess.run(fcmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("fastcall build failed:\n" + r.stdout + r.stderr)
    os.replace(ftmp, FASTCALL_LIB)
    usage = check_assembly()
    spills = {k: v for k, v in usage.items() if v[1] > 0}
    if verbose:
        for k, (vg, sc) in sorted(usage.items()):
            print(f"{vg:4d} vgpr {sc:5d} scratch  {k}")
    if spills:
        raise RuntimeError("kernel variants spill registers to scratch memory: "
                           + ", ".join(sorted(spills)))
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=0)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.v))
