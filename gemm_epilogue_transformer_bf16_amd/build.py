"""Build the HIP C-ABI library libcoda.so for gfx950, in-tree.

Every call recompiles all sources (in parallel) into ``_build/obj`` under the
repository root and links ``libcoda.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO, "include")
OBJ_DIR = os.path.join(REPO, "_build", "obj")
LIB_PATH = os.path.join(PKG_DIR, "libcoda.so")

# the fused kernel's compilation units first (the longest compiles), so they
# start together
HIP_SOURCES = [
    "coda_fused_t3n.hip", "coda_fused_t3.hip", "coda_fused_t1n.hip", "coda_fused_t1.hip",
    "coda_fused_t2n.hip", "coda_fused_t2.hip", "coda_fused_tf32.hip", "coda_fused.hip", "coda_unfused.hip",
    "coda_fold.hip", "coda_api.hip", "coda_noalloc.hip",
]
CPP_SOURCES = ["coda_plan.cpp"]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libcoda.so")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ_DIR, src + ".o")
        cmds.append([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    cxx = shutil.which("g++") or shutil.which("c++")
    for src in CPP_SOURCES:
        obj = os.path.join(OBJ_DIR, src + ".o")
        cmds.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # longest compiles first
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
