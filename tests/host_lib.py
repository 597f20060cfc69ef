"""Host-only builds of libpagedkv for CPU tests: the C entry points (argument
checks and launch plans, csrc/api.cpp) and the row pool (csrc/rowpool.cpp),
compiled by g++ with the launchers replaced by logging stubs
(tests/host_build/launch_stubs.cpp), optionally under the address and
undefined-behaviour sanitizers.  No HIP compiler or GPU is involved; the
HIP runtime header only supplies hipError_t and hipStream_t."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_input_amd", "csrc")
SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "rowpool.cpp"),
           os.path.join(HERE, "host_build", "launch_stubs.cpp")]
SANITIZE = ("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all")


def build(out: str, sanitize: bool = False) -> str:
    cmd = ["g++", "-std=c++17", "-O1", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}", "-x", "c++", *SOURCES, "-o", out]
    # every symbol resolved at link time; a sanitized build leaves the sanitizer
    # runtimes to the process that loads it (preloaded)
    cmd[-2:-2] = list(SANITIZE) if sanitize else ["-Wl,--no-undefined"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str) -> ctypes.CDLL:
    from paged_kv_input_amd import _abi

    lib = _abi.load_library(path)
    lib.pkv_stub_log.restype = ctypes.c_char_p
    lib.pkv_stub_log.argtypes = []
    lib.pkv_stub_log_clear.restype = None
    lib.pkv_stub_log_clear.argtypes = []
    return lib


def launches(lib: ctypes.CDLL, fn, *args) -> tuple[int, list[str]]:
    """Return code of fn(*args) and the launches it enqueued, in order."""
    lib.pkv_stub_log_clear()
    rc = fn(*args)
    log = lib.pkv_stub_log().decode()
    return rc, [x for x in log.split(";") if x]
