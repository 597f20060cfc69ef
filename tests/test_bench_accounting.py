"""CPU checks of the benchmark's own accounting: the algorithmic byte model the
roofline divides by, the guard that drops counter traffic taken on other
kernel sources, and the one-GPU limit of the command line."""
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_bytes_closed_form():
    """16 requests x 2048 new tokens from an empty history, block size 32,
    8 x 128 bf16 rows: every term of the byte model written out."""
    b = workloads.make("prefill_16x2048")
    ab = bench.algorithmic_bytes(b)
    T, n, row = 16 * 2048, 16, 8 * 128 * 2
    blocks = 16 * 2048 // 32                     # each touched once, all visible
    assert ab["kv"] == 4 * T * row                # read K, V; write both cache rows
    assert ab["tokens"] == T * (4 + 4 + 4) + 4 * T
    assert ab["requests"] == 24 * n + 4
    assert ab["block_table"] == 4 * blocks
    assert ab["pages"] == 8 * blocks
    assert ab["total"] == 268_972_420
    # the separate calls: the scatter moves the payload plus one slot per token
    assert bench.call_bytes(b)["scatter_kv"] == T * (4 * row + 4)


def test_head_shard_is_an_eighth_of_the_payload():
    full = bench.algorithmic_bytes(workloads.make("prefill_16x2048"))
    shard = bench.algorithmic_bytes(workloads.make("prefill_16x2048_tp8"))
    assert shard["kv"] * 8 == full["kv"]
    for key in ("tokens", "requests", "block_table", "pages"):
        assert shard[key] == full[key]               # same schedule and tables


def test_decode_bytes_closed_form():
    """256 decodes: one token each, so one touched block per request; the
    visible pages are ceil(seq_len / 16) per request."""
    import numpy as np

    b = workloads.make("decode_256x1")
    ab = bench.algorithmic_bytes(b)
    seq = b.completed[b.sched_rows].astype(np.int64) + 1
    assert ab["block_table"] == 4 * 256
    assert ab["pages"] == 8 * int(((seq + 15) // 16).sum())
    assert ab["kv"] == 4 * 256 * 2048


def test_traffic_guard(tmp_path, monkeypatch):
    """Counter traffic is reported only while the kernel's sources are the
    ones the counters were taken on."""
    csrc = tmp_path / "paged_kv_input_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "step.hip").write_text("kernel A\n")
    (csrc / "internal.h").write_text("helpers\n")
    (csrc / "geometry.h").write_text("launch geometry\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.source_digest(bench.kernel_sources("step"))
    (tmp_path / "profiles" / "step_toy_hbm_counters.md").write_text(
        f"source_sha256_16: {digest}\n\nhbm_bytes_per_launch: 12345\n")
    assert bench.traffic_from_profile("step", "toy") == 12345.0
    assert bench.traffic_from_profile("step", "other") is None     # no profile
    (csrc / "step.hip").write_text("kernel B\n")
    assert bench.traffic_from_profile("step", "toy") is None       # sources changed


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_wide_decode_bytes_closed_form():
    """4096 decodes among 8192 rows, contexts U{128..2048}, block size 16:
    one touched block per request, ceil(seq_len / 16) visible pages each."""
    import numpy as np

    b = workloads.make("decode_4096x1")
    assert (b.n, b.T, b.completed.shape[0]) == (4096, 4096, 8192)
    ab = bench.algorithmic_bytes(b)
    seq = b.completed[b.sched_rows].astype(np.int64) + 1
    assert seq.min() >= 129 and seq.max() <= 2049
    assert ab["block_table"] == 4 * 4096
    assert ab["pages"] == 8 * int(((seq + 15) // 16).sum())
    assert ab["kv"] == 4 * 4096 * 2048
    assert ab["requests"] == 24 * 4096 + 4
