"""Builds libsckv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Objects go to <repo>/_build/, the library next to this file.  Every call
recompiles (a build is the check that the sources compile).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsckv.so")
BENCH_LIB = os.path.join(PKG, "libsckv_bench.so")
BENCH_SOURCE = "bench_read.hip"

ARCH = os.environ.get("SCKV_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # keep hipcc from emitting packed fp32 arithmetic
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]
SOURCES = ["sckv_api.cpp", "compress.hip", "index.hip", "topk.hip", "attend.hip", "project.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # the benchmark's streaming-read reference, a library of its own
    bobj = _compile(BENCH_SOURCE)
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", bobj, "-o", BENCH_LIB + ".tmp"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(BENCH_LIB + ".tmp", BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
