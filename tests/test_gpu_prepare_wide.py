"""pkv_prepare_batch on wide batches (more than 1024 requests, up to
PKV_MAX_BATCH: sixteen requests ranked per workgroup) against the CPU oracle,
element by element, including the data errors; a prefill whose few requests
each get a workgroup of their own; and wide batches through the whole step."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_equal, say
from test_gpu_parity import run_and_compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_input_amd  # noqa: F401  (raises if the library is missing)
    yield
    torch.cuda.synchronize()


def prepare_on_gpu(rows, counts, completed, tok, T, with_ids=True):
    import torch
    from paged_kv_input_amd import api

    dev = torch.device("cuda")
    n = rows.shape[0]
    out = {
        "index_mapping": torch.full((n,), -7, dtype=torch.int32, device=dev),
        "query_start_loc": torch.full((n + 1,), -7, dtype=torch.int32, device=dev),
        "seq_lens": torch.full((n,), -7, dtype=torch.int32, device=dev),
        "positions": torch.full((T,), -7, dtype=torch.int32, device=dev),
        "input_ids": torch.full((T,), -7, dtype=torch.int32, device=dev) if with_ids else None,
    }
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    api.prepare_batch(t(rows), t(counts), t(completed), t(tok), T, status=status, **out)
    torch.cuda.synchronize()
    host = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    host["status"] = int(status.item()) & 0xFFFFFFFF
    return host


def compare_with_oracle(rows, counts, completed, tok, T=None, with_ids=True):
    if T is None:
        T = int(np.maximum(counts.astype(np.int64), 0).sum())
    say(f"[case] wide prepare n={rows.shape[0]} T={T} R={completed.shape[0]} ids={with_ids}")
    got = prepare_on_gpu(rows, counts, completed, tok, T, with_ids)
    want = oracle.prepare_batch(rows, counts, completed, tok, T=T, with_input_ids=with_ids)
    assert want["rc"] == 0
    keys = ["index_mapping", "query_start_loc", "seq_lens", "positions"]
    if with_ids:
        keys.append("input_ids")
    for key in keys:
        assert_equal(key, got[key], want[key])
    assert got["status"] == want["status"], (got["status"], want["status"])
    return got, want


def _wide(seed, n, decode_share, max_count, R_extra=None, L=512):
    rng = np.random.default_rng(seed)
    R = n + (R_extra if R_extra is not None else int(rng.integers(0, 2 * n + 1)))
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = rng.integers(0, max_count + 1, n).astype(np.int32)
    counts[rng.random(n) < decode_share] = 1
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, L - max_count, n)
    tok = rng.integers(0, 1 << 20, (R, L), dtype=np.int32)
    return rows, counts, completed, tok


@pytest.mark.parametrize("n", [1025, 1100, 2047, 2048, 2049, 3001, 4095, 4096])
def test_wide_random(n):
    """Mixed batches: many decodes (ties on the count), chunks, some empty runs."""
    rows, counts, completed, tok = _wide(7000 + n, n, 0.6, 200)
    compare_with_oracle(rows, counts, completed, tok)


@pytest.mark.parametrize("n", [1025, 4096])
def test_wide_all_decodes(n):
    """Every count 1: the order is the rows' order; rows spread over 8n state rows."""
    rows, counts, completed, tok = _wide(7100 + n, n, 1.0, 1, R_extra=7 * n, L=64)
    compare_with_oracle(rows, counts, completed, tok)


def test_wide_all_equal_rows_order():
    """Rows given in descending order with equal counts: the result is the rows ascending."""
    n = 3000
    rows = np.arange(n, dtype=np.int32)[::-1].copy()
    counts = np.full(n, 2, np.int32)
    completed = np.arange(n, dtype=np.int32) % 50
    tok = (np.arange(n)[:, None] * 64 + np.arange(64)[None, :]).astype(np.int32)
    got, _ = compare_with_oracle(rows, counts, completed, tok)
    assert got["index_mapping"].tolist() == list(range(n))
    assert got["query_start_loc"].tolist() == list(range(0, 2 * n + 1, 2))


def test_wide_without_input_ids():
    rows, counts, completed, tok = _wide(7200, 1500, 0.5, 40)
    compare_with_oracle(rows, counts, completed, tok, with_ids=False)


@pytest.mark.parametrize("delta", [-37, 0, 55])
def test_wide_data_errors(delta):
    """Rows outside [0, R), negative counts, duplicate rows, completed counts
    that put positions past the token table or below zero, and a host token
    count above, equal to or below the counts' sum: same outputs and flags."""
    rng = np.random.default_rng(7300 + delta)
    n, L = 2500, 128
    rows, counts, completed, tok = _wide(7300 + delta, n, 0.5, 30, L=L)
    R = completed.shape[0]
    bad = rng.choice(n, 40, replace=False)
    rows[bad[:10]] = -1 - rng.integers(0, 5, 10)            # negative rows
    rows[bad[10:20]] = R + rng.integers(0, 5, 10)           # rows past R
    counts[bad[20:30]] = -rng.integers(1, 9, 10)            # negative counts
    rows[bad[30:35]] = rows[bad[35:40]]                     # duplicate rows
    good = np.setdiff1d(np.arange(n), bad)[:20]
    completed[rows[good[:10]]] = L - 3                      # positions past the table
    completed[rows[good[10:20]]] = -5                       # negative positions
    T = int(np.maximum(counts.astype(np.int64), 0).sum()) + delta
    got, want = compare_with_oracle(rows, counts, completed, tok, T=T)
    assert want["status"] != 0


def test_wide_saturating_prefix_sum():
    """Counts whose sum passes INT32_MAX: query_start_loc saturates, and T (the
    host's count) disagrees, as the oracle has it."""
    n = 1200
    rng = np.random.default_rng(7400)
    R = 2 * n
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = np.ones(n, np.int32)
    counts[:3] = 1 << 30                                    # 3 * 2^30 > INT32_MAX
    completed = np.zeros(R, np.int32)
    tok = np.zeros((R, 4), np.int32)
    T = 2000                                                # only the first tokens are real
    compare_with_oracle(rows, counts, completed, tok, T=T)


@pytest.mark.parametrize("n", [1025, 2048])
def test_wide_whole_step(n):
    """A wide batch through pkv_step (past the one-launch limit: the separate
    kernels), slots, visible pages and the K/V scatter against the oracle."""
    rng = np.random.default_rng(7500 + n)
    R, L, bs = 2 * n, 96, 16
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = rng.integers(0, 6, n).astype(np.int32)
    counts[rng.random(n) < 0.6] = 1
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 80, n)
    MB = L // bs
    need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                   for r, c in zip(rows, counts)))
    NB = need + 9
    bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
    T = int(counts.sum())
    k = rng.integers(0, 65535, (T, 1, 64), dtype=np.uint16)
    v = rng.integers(0, 65535, (T, 1, 64), dtype=np.uint16)
    b = workloads.Batch(f"wide_step_{n}", 7500 + n, rows, counts, completed,
                        rng.integers(0, 1 << 20, (R, L), dtype=np.int32),
                        [workloads.KVGroup(bs, NB, MB, bt, 1, 64, "fp16", k, v)])
    run_and_compare(b, mode="fused")


@pytest.mark.parametrize("n,mean,delta", [(16, 2048, 0), (16, 2048, -1000), (20, 750, 0),
                                          (40, 300, 7), (100, 200, 0), (300, 40, -5)])
def test_requests_per_workgroup(n, mean, delta):
    """Batches whose tokens per request select 1, 2, 4, 8 and 16 requests per
    workgroup (about 2048 tokens per workgroup: means of 2048, 750, 300, 200
    and 40 tokens), with the host's token count equal to, above and below the
    counts' sum (the cut falling inside a request)."""
    rng = np.random.default_rng(7600 + n + delta)
    R, L = 2 * n, 4 * mean + 64
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = rng.integers(1, 2 * mean, n).astype(np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 2 * mean, n)
    tok = rng.integers(0, 1 << 20, (R, L), dtype=np.int32)
    T = int(counts.sum()) + delta
    compare_with_oracle(rows, counts, completed, tok, T=T)


@pytest.mark.parametrize("T", [0, 5000])
def test_no_requests(T):
    """n = 0: query_start_loc = [0]; with T > 0 every token gets position -1
    and input id -1, and TOKEN_SUM is flagged."""
    rows = np.zeros(0, np.int32)
    tok = np.arange(4 * 8, dtype=np.int32).reshape(4, 8)
    got, want = compare_with_oracle(rows, rows.copy(), np.zeros(4, np.int32), tok, T=T)
    assert got["query_start_loc"].tolist() == [0]
    assert (got["status"] != 0) == (T > 0)
