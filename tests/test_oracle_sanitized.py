"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only): gcc builds a sanitized copy, and the pins run against it in a child
process with the ASan runtime preloaded, so any out-of-bounds access, overflow
or undefined shift in the oracle fails the test."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
lib = oracle.load({so!r})
pins.pin_pages_example(lib)
pins.pin_prefix_example(lib)
pins.pin_budget_tie_example(lib)
pins.pin_bruteforce(lib, seeds=range(60))
pins.pin_closed_forms(lib)
pins.pin_error_semantics(lib)
pins.pin_strided_kv(lib)
print("sanitized pins ok")
"""


def test_oracle_under_asan_ubsan(tmp_path):
    try:
        libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                                 capture_output=True, text=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("gcc not available")
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("libasan not installed")
    so = oracle.build(out=str(tmp_path / "liboracle_asan.so"),
                      extra_flags=("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                   "-fno-sanitize-recover=all"))
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(root=os.path.dirname(HERE), tests=HERE, so=so)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "sanitized pins ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
