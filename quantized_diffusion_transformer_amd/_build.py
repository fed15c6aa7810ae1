"""Builds libqdt.so (the HIP path, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqdt.so")
SOURCES = ["qdt_abi.hip", "qdt_quant.hip", "qdt_gemm.hip", "qdt_wo.hip", "qdt_attn.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # fp32 arithmetic exactly as written: no contraction into FMA, no fast-math
    "-ffp-contract=off",
    # no packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), then links libqdt.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cflags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s.replace(".hip", ".o"))
        jobs.append((obj, [hipcc(), *cflags, "-c", "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, s),
                           "-o", obj]))

    def run(job):
        if verbose:
            print(" ".join(job[1]), flush=True)
        subprocess.run(job[1], check=True)
        return job[0]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(run, jobs))
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
