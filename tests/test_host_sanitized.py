"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
g++ builds the C entry points (argument checks, launch plans; csrc/api.cpp)
and the row pool (csrc/rowpool.cpp) with the launchers stubbed out
(host_lib.py), and the host-side tests run against that build in a child
process with the ASan runtime preloaded -- every rejection case of
test_abi.py, pkv_step's plans and routing, and the row pool against the
oracle's model.  Any out-of-bounds access, overflow or undefined shift in that
code fails the test.  No GPU and no HIP compiler are involved."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import host_lib, test_abi, test_row_pool, test_step_plan
lib = host_lib.load({so!r})
for fn in (test_abi.test_host_argument_errors, test_abi.test_step_host_argument_errors,
           test_abi.test_gather_host_argument_errors, test_abi.test_prefix_host_argument_errors,
           test_abi.test_alloc_host_argument_errors, test_abi.test_state_host_argument_errors,
           test_abi.test_step_path_argument_errors, test_row_pool.test_pool_host_argument_errors,
           test_row_pool.test_pool_epoch_reuse, test_step_plan.check_plans,
           test_step_plan.check_routing):
    fn(lib)
for seed in range(30):
    test_row_pool.test_pool_matches_oracle(lib, seed)
print("sanitized host code ok")
"""


def test_host_code_under_asan_ubsan(tmp_path):
    import host_lib

    try:
        libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                                 capture_output=True, text=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("gcc not available")
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("libasan not installed")
    so = host_lib.build(str(tmp_path / "libpkv_host_asan.so"), sanitize=True)
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(root=os.path.dirname(HERE), tests=HERE, so=so)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "sanitized host code ok" in r.stdout, \
        r.stdout[-2000:] + r.stderr[-4000:]
