"""Build the package's two shared libraries in-tree.

    python -m paged_kv_cache_245_amd.build [-v]

libpa.so: every csrc/*.hip (the gfx950 HIP kernels and their C ABI, include/pa.h)
compiled with hipcc to objects under _build/ (in parallel) and linked.
libpa_host.so: the host-side block pool and scheduler (include/pa_pool.h,
include/pa_sched.h), plain C++ built with g++; it needs no GPU and no ROCm.
Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")

SOURCES = ["pa_api.hip", "write_kv.hip", "decode.hip", "prefill.hip", "copy_blocks.hip",
           "gather_kv.hip", "bench_kernels.hip", "noalloc.hip"]
HOST_SOURCES = ["block_pool.cpp", "sched.cpp"]
HOST_LIB = os.path.join(PKG, "libpa_host.so")
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the device code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build_host(verbose: bool = False) -> str:
    """libpa_host.so with the host C++ compiler."""
    cxx = os.environ.get("CXX") or shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        raise RuntimeError("no host C++ compiler found for libpa_host.so")
    tmp = HOST_LIB + ".tmp"
    _run([cxx, "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", "-I", INCLUDE,
          *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", tmp], verbose)
    os.replace(tmp, HOST_LIB)
    return HOST_LIB


def build(verbose: bool = False, jobs: int | None = None) -> str:
    build_host(verbose)
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
