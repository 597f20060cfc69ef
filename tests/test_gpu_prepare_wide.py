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
                                          (40, 300, 7), (100, 200, 0), (300, 40, -5),
                                          (16, 12000, 5), (4, 20000, 0), (2, 60000, -7)])
def test_requests_per_workgroup(n, mean, delta):
    """Batches whose tokens per request select 1, 2, 4, 8 and 16 requests per
    workgroup (about 2048 tokens per workgroup: means of 2048, 750, 300, 200
    and 40 tokens), and requests so long that several workgroups split one
    request's tokens (means of 12000 to 60000), with the host's token count
    equal to, above and below the counts' sum (the cut falling inside a
    request)."""
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


def _random_wide(seed, n_lo=513, n_hi=1600):
    """A seeded random step past the one-launch step's 512 requests: counts
    with ties and zeros, 1-4 groups with block sizes 1-64 (3 included) and
    rows of 16 B to 1 KiB."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(n_lo, n_hi))
    R = n + int(rng.integers(0, n + 1))
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = np.where(rng.random(n) < 0.6, 1, rng.integers(0, 20, n)).astype(np.int32)
    L = 64 + 24
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 64, n)
    T = int(counts.sum())
    groups = []
    for _ in range(int(rng.integers(1, 5))):
        bs = int(rng.choice([1, 3, 4, 8, 16, 32, 64]))
        MB = -(-L // bs)
        need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                       for r, c in zip(rows, counts)))
        NB = need + int(rng.integers(1, 64))
        bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
        H, D = [(1, 8), (2, 64), (4, 32), (1, 512)][int(rng.integers(0, 4))]
        k = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        v = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        groups.append(workloads.KVGroup(bs, NB, MB, bt, H, D, "fp16", k, v))
    tok = rng.integers(0, 1 << 20, (R, L), dtype=np.int32)
    return workloads.Batch(f"wide_sweep_{seed}", seed, rows, counts, completed, tok, groups)


@pytest.mark.parametrize("seed", range(8))
def test_wide_step_random_groups(seed):
    """pkv_step past 512 requests with 1-4 groups: the batch, every group's
    slots and visible pages in one launch, then the scatters; bit-exact."""
    run_and_compare(_random_wide(7700 + seed), mode="fused")


def test_wide_step_data_errors():
    """pkv_step past 512 requests with bad rows, negative counts, missing and
    out-of-pool blocks, logical blocks past the table and a host token count
    above the counts' sum: same outputs, caches and status bits as the oracle."""
    import torch
    from paged_kv_input_amd.step import DeviceStep, GroupSpec
    from gpu_util import SENTINEL16

    b = _random_wide(7800, 900, 901)
    rng = np.random.default_rng(7801)
    n, R = b.n, b.completed.shape[0]
    bad = rng.choice(n, 30, replace=False)
    b.sched_rows[bad[:8]] = -3
    b.sched_rows[bad[8:14]] = R + 2
    b.num_scheduled[bad[14:20]] = -2
    g0 = b.groups[0]
    bt = g0.block_table
    live = np.flatnonzero((bt >= 0).any(axis=1))
    bt[live[:6], 0] = -1                                     # missing blocks
    bt[live[6:12], 0] = g0.num_blocks + 5                    # blocks past the pool
    b.completed[b.sched_rows[bad[20:30]]] = g0.max_blocks * g0.block_size + 1   # past the table
    T = int(np.maximum(b.num_scheduled.astype(np.int64), 0).sum()) + 17
    for g in b.groups:                                       # K/V rows: exactly T
        g.k = np.resize(g.k, (T,) + g.k.shape[1:])
        g.v = np.resize(g.v, (T,) + g.v.shape[1:])
    say(f"[case] wide step errors n={n} T={T} groups={len(b.groups)}")
    step = DeviceStep(b.sched_rows, b.num_scheduled, b.completed, b.token_ids,
                      [GroupSpec(g.block_table, g.block_size, g.num_blocks, g.k, g.v)
                       for g in b.groups],
                      cache_fill=SENTINEL16, ibt_fill=oracle.IBT_UNWRITTEN, num_tokens=T)
    step.run_fused()
    torch.cuda.synchronize()
    prep = oracle.prepare_batch(b.sched_rows, b.num_scheduled, b.completed, b.token_ids, T=T)
    want = prep["status"]
    for key in ("index_mapping", "query_start_loc", "seq_lens", "positions", "input_ids"):
        assert_equal(key, step.host(key), prep[key])
    for gi, g in enumerate(b.groups):
        sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                         prep["seq_lens"], prep["positions"], g.block_table,
                                         g.block_size, g.num_blocks)
        kc = np.full((g.num_slots, g.num_heads, g.head_dim), 0xFFFF, np.uint16)
        vc = kc.copy()
        rc, sst = oracle.scatter_kv(g.k, g.v, kc, vc, sm["slot_mapping"])
        want |= sm["status"] | sst
        assert_equal(f"g{gi} slots", step.host("slot_mapping", gi), sm["slot_mapping"])
        assert_equal(f"g{gi} pages", step.host("input_block_tables", gi),
                     sm["input_block_tables"])
        assert_equal(f"g{gi} k_cache", step.host("k_cache", gi).view(np.uint16), kc)
        assert_equal(f"g{gi} v_cache", step.host("v_cache", gi).view(np.uint16), vc)
    assert step.status_bits() == want, (step.status_bits(), want)
    assert (want & 0x3F) == 0x3F            # every data error above was hit


@pytest.mark.parametrize("W", [1, 37, 300])
def test_wide_step_window(W):
    """pkv_step past 512 requests with two sliding-window groups: blocks behind
    every window freed first (the -1 holes), then the step's pages and slots
    against the oracle's."""
    from test_gpu_alloc import check_free
    from paged_kv_input_amd.step import DeviceStep, GroupSpec
    from gpu_util import SENTINEL16
    import torch

    b = _random_wide(7900 + W, 700, 701)
    while len(b.groups) < 2:
        b = _random_wide(b.seed + 1000, 700, 701)
    b.groups = b.groups[:2]
    tables, specs = [], []
    for gi, g in enumerate(b.groups):
        bt = check_free(b.sched_rows, b.completed, g.block_table, g.block_size, W, f"g{gi}")
        tables.append(bt)
        specs.append(GroupSpec(bt, g.block_size, g.num_blocks, g.k, g.v, sliding_window=W))
    say(f"[case] wide step window W={W} n={b.n} T={b.T}")
    step = DeviceStep(b.sched_rows, b.num_scheduled, b.completed, b.token_ids, specs,
                      cache_fill=SENTINEL16, ibt_fill=oracle.IBT_UNWRITTEN)
    step.run_fused()
    torch.cuda.synchronize()
    prep = oracle.prepare_batch(b.sched_rows, b.num_scheduled, b.completed, b.token_ids)
    status = prep["status"]
    for gi, (g, bt) in enumerate(zip(b.groups, tables)):
        sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                         prep["seq_lens"], prep["positions"], bt, g.block_size,
                                         g.num_blocks, sliding_window=W)
        status |= sm["status"]
        assert_equal(f"g{gi} slots", step.host("slot_mapping", gi), sm["slot_mapping"])
        assert_equal(f"g{gi} pages", step.host("input_block_tables", gi),
                     sm["input_block_tables"])
    assert step.status_bits() == status == 0


def test_wide_step_long_requests():
    """pkv_step past 512 requests with about 3000 tokens per request (1.8 M
    tokens): two workgroups split each group of requests' tokens and pages."""
    rng = np.random.default_rng(7950)
    n, L, bs = 600, 4100, 64
    R = 2 * n
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = rng.integers(2500, 3501, n).astype(np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 500, n)
    MB = L // bs + 1
    need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                   for r, c in zip(rows, counts)))
    NB = need + 9
    bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
    T = int(counts.sum())
    k = rng.integers(0, 65535, (T, 1, 8), dtype=np.uint16)
    v = rng.integers(0, 65535, (T, 1, 8), dtype=np.uint16)
    b = workloads.Batch("wide_long", 7950, rows, counts, completed,
                        rng.integers(0, 1 << 20, (R, L), dtype=np.int32),
                        [workloads.KVGroup(bs, NB, MB, bt, 1, 8, "fp16", k, v)])
    run_and_compare(b, mode="fused")


@pytest.mark.parametrize("n,extra", [(257, 0), (384, 0), (512, 0), (384, 1152), (300, 901)])
def test_decode_like_batches(n, extra):
    """Decode-like batches past 256 requests, with 1-4 tokens per request (the
    request-ranked single launch); each against the oracle, caches included."""
    rng = np.random.default_rng(8100 + n + extra)
    R, L, bs = 3 * n, 512, 16
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = np.full(n, 1 + extra // n, np.int32)
    counts[rng.choice(n, extra % n, replace=False)] += 1     # T = n + extra
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 400, n)
    MB = L // bs
    need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                   for r, c in zip(rows, counts)))
    NB = need + 13
    bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
    T = int(counts.sum())
    k = rng.integers(0, 65535, (T, 2, 64), dtype=np.uint16)
    v = rng.integers(0, 65535, (T, 2, 64), dtype=np.uint16)
    b = workloads.Batch(f"decode_like_{n}_{extra}", 8100 + n, rows, counts, completed,
                        rng.integers(0, 1 << 20, (R, L), dtype=np.int32),
                        [workloads.KVGroup(bs, NB, MB, bt, 2, 64, "fp16", k, v)])
    step, _, _ = run_and_compare(b, mode="fused")
    from paged_kv_input_amd import api

    # which plan ran (the same rule pkv_step routes by; pinned on the CPU in
    # test_step_plan.py): past 256 requests with up to 16 tokens each, the
    # request-ranked single launch
    assert step.fused_path() == (api.STEP_RANKED_ONE_LAUNCH if T <= 16 * n
                                 else api.STEP_ONE_LAUNCH)
