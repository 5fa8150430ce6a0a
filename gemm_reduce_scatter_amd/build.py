"""Compile libpk_gemm_rs.so for gfx950 with hipcc, in-tree.

``python -m gemm_reduce_scatter_amd.build`` or ``build_library()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n) for n in ("pk_gemm_rs.hip", "pk_consume.hip")]
OUT = os.path.join(HERE, "libpk_gemm_rs.so")
# The same sources with the phase recorder compiled in (PK_TIMELINE): a
# library of its own for timing studies; the product library never has it.
OUT_TIMELINE = os.path.join(HERE, "libpk_gemm_rs_timeline.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # packed fp32 instructions stay off (compiler must not form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_library(verbose: bool = False, timeline: bool = False) -> str:
    out = OUT_TIMELINE if timeline else OUT
    tmp = out + ".tmp"
    extra = ["-DPK_TIMELINE"] if timeline else []
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False):
    """Both libraries, compiled side by side."""
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(2) as ex:
        futs = [ex.submit(build_library, verbose, t) for t in (False, True)]
        return [f.result() for f in futs]


if __name__ == "__main__":
    import sys as _sys
    if "--timeline" in _sys.argv:
        print(build_library(verbose=True, timeline=True))
    elif "--all" in _sys.argv:
        print(build_all(verbose=True))
    else:
        print(build_library(verbose=True))
