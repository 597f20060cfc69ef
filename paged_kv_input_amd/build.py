"""Build libpagedkv.so in-tree with hipcc for gfx950 (no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["api.cpp", "prepare.hip", "slots.hip", "scatter.hip", "step.hip", "state.hip",
           "rowpool.cpp", "gather.hip", "prefix.hip", "alloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions are kept out of every kernel (-packed-fp32-ops).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra", "-Werror",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(out: str = LIB, extra=()) -> str:
    """Compile every HIP source into one shared library (always rebuilds)."""
    cmd = [HIPCC, *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


C_CALLER = os.path.join(ROOT, "tests", "c_caller", "pages_example")


def build_c_caller(out: str = C_CALLER) -> str:
    """Compile the test suite's C-ABI caller (host code only, no kernels): it
    links libpagedkv.so and the HIP runtime, nothing from Python or torch."""
    lib_dir = os.path.dirname(LIB)
    rpath = os.path.relpath(lib_dir, os.path.dirname(out))
    cmd = [HIPCC, "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror", f"-I{INCLUDE}",
           out + ".cpp", f"-L{lib_dir}", "-lpagedkv", f"-Wl,-rpath,$ORIGIN/{rpath}",
           "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sources_newer_than(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    paths = [os.path.join(CSRC, s) for s in os.listdir(CSRC)] + [os.path.join(INCLUDE, "pagedkv.h")]
    return any(os.path.getmtime(p) > t for p in paths)


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
