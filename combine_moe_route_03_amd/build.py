"""Build the gfx950 HIP library libmoe_route.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "moe_route.hip")
LIB = os.path.join(PKG, "libmoe_route.so")
BENCH_SRC = os.path.join(PKG, "csrc", "bench_copy.hip")
BENCH_LIB = os.path.join(PKG, "libmoe_bench_copy.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 add/mul/fma instructions.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE]


def _compile(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the routing library and the benchmark's copy kernel; returns the library path."""
    _compile(BENCH_SRC, BENCH_LIB, verbose)
    return _compile(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
