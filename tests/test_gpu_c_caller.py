"""The C ABI called from C: tests/c_caller/pages_example (built by build(),
host code linking libpagedkv.so and the HIP runtime only) runs the pages'
worked example through pkv_step and checks every output bit for bit."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BINARY = os.path.join(HERE, "c_caller", "pages_example")


def test_pages_example_from_c():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BINARY):
        pytest.fail(f"{BINARY} is not built: run `python __graft_entry__.py`")
    print("[case] C caller: pages example through pkv_step", flush=True)
    r = subprocess.run([BINARY], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "bit-exact" in r.stdout
