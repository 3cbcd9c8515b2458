"""Build libdiffqkv.so (the C-ABI library with its gfx950 kernels) in-tree.

Usage: ``python -m asymmetric_head_kv_amd.build`` (or ``__graft_entry__.build()``).
Every call recompiles.  Objects go to ``_build/`` at the repository root; the
shared library lands next to this file, where the binding loads it.
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
LIB = os.path.join(PKG, "libdiffqkv.so")

SOURCES = ["api.hip", "kv_append.hip", "decode.hip", "prefill.hip", "selective.hip", "augq.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core results in ordinary VGPRs: the softmax reads them directly
    # instead of copying them out of accumulation registers every tile.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions.  The prefill kernel's softmax takes row maxima of
# matrix-core results that are never NaN: with relaxed NaN handling (and the
# IEEE mode bit off, which that permits) fmaxf needs no operand quieting.
EXTRA = {"prefill.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n"
                           f"{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source for gfx950 and link libdiffqkv.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for r in ex.map(_run, cmds):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
