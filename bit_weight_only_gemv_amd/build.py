"""Builds ``libwq.so`` (host encoder + gfx950 kernels) in-tree.

Host C++ is compiled by g++ with ``-ffp-contract=off`` (the encoder must round
exactly as written); HIP sources by hipcc for gfx950 only, with packed FP32
instructions disabled; hipcc links the shared library.

Usage: ``python -m bit_weight_only_gemv_amd.build`` (or ``build()``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwq.so")

ARCH = "gfx950"
HOST_SOURCES = ["wq_host.cpp"]
HIP_SOURCES = ["wq_gemv.hip", "wq_mma.hip", "wq_gemm.hip", "wq_misc.hip", "wq_refine.hip"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libwq.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compiles every source and links ``libwq.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    common = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall"]
    cmds = []
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *common, "-O2", "-ffp-contract=off", "-fno-fast-math",
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([hipcc, *common, f"--offload-arch={ARCH}",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-Wno-unused-command-line-argument",
                     "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
