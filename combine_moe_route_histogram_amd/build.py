"""Builds libmoe.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m combine_moe_route_histogram_amd.build [-v]

Each .hip source under csrc/ is compiled to an object with hipcc in
parallel, then linked into combine_moe_route_histogram_amd/libmoe.so.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["route.hip", "rows.hip", "gemm.hip", "fused.hip", "bwd.hip", "tuning.hip", "moe_api.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"),
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # hipcc's host pass does not know the packed-fp32 feature flag; that note is harmless
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libmoe.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))

    def compile_one(i):
        _run([hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, srcs[i]), "-o", objs[i]], verbose)

    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, range(len(srcs))))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
