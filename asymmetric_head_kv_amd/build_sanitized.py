"""Host-sanitizer build of the C ABI, for the CPU test-suite only.

Compiles api.hip (the ABI's argument checks, planning and workspace layout:
all host code) with AddressSanitizer and UndefinedBehaviorSanitizer on its
host side, links it with the ordinary objects of the kernel sources (built
first by build.py) into _build/sanitize/libdiffqkv_host_asan.so, and returns
that path.  GPU code is never built with a sanitizer.  Load the library into
a process that preloads the ASan runtime (asan_runtime()).
"""

from __future__ import annotations

import glob
import os
import subprocess

from .build import BUILD, CSRC, EXTRA, FLAGS, HIPCC, ROOT, SOURCES, build

OUT = os.path.join(BUILD, "sanitize")
LIB = os.path.join(OUT, "libdiffqkv_host_asan.so")
CLANGXX = os.path.join("/opt/rocm/llvm/bin", "clang++")

# Each sanitizer flag applies to the host compilation only.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime (it carries the UBSan handlers)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _objects_fresh() -> bool:
    """Whether every ordinary object is newer than every source and header."""
    deps = glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    newest = max(os.path.getmtime(d) for d in deps)
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < newest:
            return False
    return True


def build_sanitized() -> str:
    os.makedirs(OUT, exist_ok=True)
    if not _objects_fresh():
        build()  # the kernel objects (and the ordinary library)
    api_obj = os.path.join(OUT, "api.o")
    _run([HIPCC, *FLAGS, *EXTRA.get("api.hip", []), *HOST_SAN, "-c",
          os.path.join(CSRC, "api.hip"), "-o", api_obj])
    objs = [api_obj] + [os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
                        for s in SOURCES if s != "api.hip"]
    link_san = ["-fsanitize=address", "-fsanitize=undefined", "-shared-libasan"]
    _run([CLANGXX, "-shared", "-fPIC", *objs, *link_san, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", LIB])
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
