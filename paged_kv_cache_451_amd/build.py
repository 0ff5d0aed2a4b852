"""Build ``libpa.so`` (the gfx950 HIP library) in-tree.

    python -m paged_kv_cache_451_amd.build

Compiles every ``csrc/*.hip`` with hipcc for gfx950 into ``_build/`` and
links ``paged_kv_cache_451_amd/libpa.so``; the benchmark's measurement probe
(``csrc/probe/*.hip``, declared in ``include/pa_probe.h``) goes into
``paged_kv_cache_451_amd/libpa_probe.so``; the native host block manager
(``csrc/host/*.cpp``, declared in ``include/pa_host.h``) is built with the
host C++ compiler into ``paged_kv_cache_451_amd/libpa_host.so``.  Runs on a
machine without a GPU (hipcc cross-compiles).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
HOST_LIB = os.path.join(PKG, "libpa_host.so")
CXX = os.environ.get("CXX") or shutil.which("g++") or "g++"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or \
    "/opt/rocm/bin/hipcc"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}"
                           f"\n{r.stdout}\n{r.stderr}")
    return r


def _link(srcs, lib, verbose):
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, lib)


def _host_lib(verbose):
    """The native host block manager (host code only, include/pa_host.h)."""
    tmp = HOST_LIB + ".tmp"
    cmd = [CXX, "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall",
           f"-I{INCLUDE}", *sorted(glob.glob(os.path.join(CSRC, "host",
                                                          "*.cpp"))),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, HOST_LIB)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _link(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), LIB, verbose)
    _link(sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), PROBE_LIB,
          verbose)
    _host_lib(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
