"""pkv_step's request-ranked single launch (batches of at least 32 requests
with a few tokens each) against the CPU oracle, element by element: random
batches of 32 to 4096 requests with 1-4 groups (block sizes 1 to 64, rows of
16 B to 3 KiB, chunk counts that are not powers of two), sliding-window
groups with holes, data errors, K/V views with a token stride, and a cache
shorter than its pool.  Every case asserts that the ranked plan is the one that
ran."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import SENTINEL16, assert_equal, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_input_amd  # noqa: F401  (raises if the library is missing)
    yield
    torch.cuda.synchronize()


ROWS = [(1, 8), (3, 8), (2, 64), (8, 128), (12, 128)]     # 16 B, 48 B, 256 B, 2 KiB, 3 KiB


def ranked_batch(seed):
    """A seeded batch inside the ranked plan: n >= 32, T <= 8 n (16 n past 256)."""
    rng = np.random.default_rng(seed)
    n = [32, 33, 63, 100, 255, 256, 257, 500, 512, 1000, 2048, 4096][seed % 12]
    R = n + int(rng.integers(0, n + 1))
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    base = int(rng.choice([0, 1, 2, 4]))
    hi = 9 if n <= 256 else 17
    counts = np.where(rng.random(n) < 0.5, base, rng.integers(0, hi, n)).astype(np.int32)
    counts = np.minimum(counts, 8 if n <= 256 else 16)
    L = 64 + 20
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 64, n)
    T = int(counts.sum())
    groups, windows = [], []
    for _ in range(int(rng.integers(1, 5))):
        bs = int(rng.choice([1, 3, 4, 8, 16, 32, 64]))
        MB = -(-L // bs)
        need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                       for r, c in zip(rows, counts)))
        NB = need + int(rng.integers(1, 64))
        bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
        H, D = ROWS[int(rng.integers(0, 3 if n > 1000 else len(ROWS)))]
        k = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        v = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        W = int(rng.choice([0, 0, int(rng.integers(1, 3 * bs + 5))]))
        if W:
            # the blocks behind each window are freed first (-1 holes)
            bt = bt.copy()
            assert oracle.window_free(rows, completed, bt, bs, W)["rc"] == 0
        groups.append(workloads.KVGroup(bs, NB, MB, bt, H, D, "fp16", k, v))
        windows.append(W)
    tok = rng.integers(0, 1 << 20, (R, L), dtype=np.int32)
    return workloads.Batch(f"ranked_{seed}", seed, rows, counts, completed, tok, groups), windows


def run_ranked(b, windows, num_tokens=None, with_ids=True, with_pages=True):
    import torch
    from paged_kv_input_amd import api
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    T = b.T if num_tokens is None else num_tokens
    say(f"[case] {b.name} n={b.n} T={T} groups={[(g.block_size, g.row_bytes) for g in b.groups]} "
        f"windows={windows}")
    specs = [GroupSpec(g.block_table, g.block_size, g.num_blocks, g.k, g.v, sliding_window=W)
             for g, W in zip(b.groups, windows)]
    step = DeviceStep(b.sched_rows, b.num_scheduled, b.completed, b.token_ids, specs,
                      cache_fill=SENTINEL16, ibt_fill=oracle.IBT_UNWRITTEN, num_tokens=T,
                      with_input_ids=with_ids, with_block_tables=with_pages)
    assert step.fused_path() == api.STEP_RANKED_ONE_LAUNCH
    step.run_fused()
    torch.cuda.synchronize()
    prep = oracle.prepare_batch(b.sched_rows, b.num_scheduled, b.completed, b.token_ids, T=T)
    keys = ("index_mapping", "query_start_loc", "seq_lens", "positions") + \
        (("input_ids",) if with_ids else ())
    for key in keys:
        assert_equal(key, step.host(key), prep[key])
    status = prep["status"]
    for gi, (g, W) in enumerate(zip(b.groups, windows)):
        sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                         prep["seq_lens"], prep["positions"], g.block_table,
                                         g.block_size, g.num_blocks, sliding_window=W)
        kc = np.full((g.num_slots, g.num_heads, g.head_dim), 0xFFFF, np.uint16)
        vc = kc.copy()
        rc, sst = oracle.scatter_kv(g.k, g.v, kc, vc, sm["slot_mapping"])
        assert_equal(f"g{gi} slot_mapping", step.host("slot_mapping", gi), sm["slot_mapping"])
        if with_pages:
            assert_equal(f"g{gi} input_block_tables", step.host("input_block_tables", gi),
                         sm["input_block_tables"])
        assert_equal(f"g{gi} k_cache", step.host("k_cache", gi).view(np.uint16), kc)
        assert_equal(f"g{gi} v_cache", step.host("v_cache", gi).view(np.uint16), vc)
        status |= sm["status"] | sst
    if with_ids:
        assert step.status_bits() == status, (step.status_bits(), status)
    return step


@pytest.mark.parametrize("seed", range(24))
def test_ranked_random(seed):
    b, windows = ranked_batch(5000 + seed)
    run_ranked(b, windows, with_pages=seed % 5 != 4)


def test_ranked_without_input_ids():
    b, windows = ranked_batch(5100)
    run_ranked(b, windows, with_ids=False)


def test_ranked_error_inputs():
    """40 requests: rows outside [0, R), negative and zero counts, positions
    past the token table and below zero, blocks missing (-1) or past the pool,
    logical blocks past the table; T larger than the counts' sum (tokens past
    the last request) and smaller (tokens dropped).  Written slots stay
    unique, so the caches are compared whole."""
    rng = np.random.default_rng(77)
    n, R, L, bs, NB = 40, 64, 24, 4, 160
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = rng.integers(1, 5, n).astype(np.int32)
    counts[[11, 12]] = 0
    completed = rng.integers(0, 14, R).astype(np.int32)
    completed[rows[20]] = L - 2                       # positions past the token table
    completed[rows[22]] = 27                          # logical blocks past the narrowed table
    wide = -(-(L + 8) // bs)
    bt = workloads._block_table(rng, R, wide, NB, bs, rows, counts, completed)
    MB = 7                                            # positions >= 28 have no table entry
    bt = np.ascontiguousarray(bt[:, :MB])
    bt[rows[25], :] = -1                              # blocks missing
    bt[rows[26], :] = NB + 3                          # blocks past the pool
    completed[rows[21]] = -6                          # negative positions
    rows = rows.copy()
    rows[[3, 17]] = [R + 5, -2]                       # rows outside [0, R)
    counts[[5, 9]] = [-3, -1]                         # negative counts
    tok = (np.arange(R)[:, None] * 1000 + np.arange(L)[None, :]).astype(np.int32)
    total = int(np.maximum(counts, 0).sum())
    for T in (total + 7, total, total - 9):
        k = rng.integers(0, 65000, (T, 1, 8), dtype=np.uint16)
        v = rng.integers(0, 65000, (T, 1, 8), dtype=np.uint16)
        b = workloads.Batch(f"ranked_errors_T{T}", 77, rows, counts, completed, tok,
                            [workloads.KVGroup(bs, NB, MB, bt, 1, 8, "fp16", k, v)])
        step = run_ranked(b, [0], num_tokens=T)
        bits = step.status_bits()
        for name in ("BAD_ROW", "BAD_COUNT", "POS_OOR", "LB_OOR", "BLOCK_OOR"):
            assert bits & getattr(oracle, "ST_" + name), name
        assert bool(bits & oracle.ST_TOKEN_SUM) == (T != total)


def test_ranked_strided_kv_and_short_cache():
    """K and V as views into a fused per-token buffer (token stride 3 rows), and
    a cache shorter than the pool (slots past it flag SLOT_OOR, no write)."""
    import torch
    from paged_kv_input_amd import api

    rng = np.random.default_rng(91)
    n, R, L, bs = 64, 200, 40, 8
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = rng.integers(1, 5, n).astype(np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 30, n)
    MB = -(-L // bs)
    need = int(sum(-(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs
                   for r, c in zip(rows, counts)))
    NB = need + 4
    bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
    T = int(counts.sum())
    H, D = 2, 24                                      # 96 B rows: 6 chunks
    fused = torch.from_numpy(rng.integers(-30000, 30000, (T, 3, H, D), dtype=np.int16)).cuda()
    k, v = fused[:, 1], fused[:, 2]
    short = NB * bs - 3 * bs                          # the last three blocks have no cache rows
    kc = torch.full((short, H, D), SENTINEL16, dtype=torch.int16, device="cuda")
    vc = torch.full_like(kc, SENTINEL16)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = dict(index_mapping=torch.empty(n, **i32), query_start_loc=torch.empty(n + 1, **i32),
                seq_lens=torch.empty(n, **i32), positions=torch.empty(T, **i32),
                input_ids=torch.empty(T, **i32))
    sm = torch.empty(T, **i32)
    ibt = torch.full((n, MB), oracle.IBT_UNWRITTEN, **i32)
    st = torch.zeros(1, **i32)
    tok = rng.integers(0, 1 << 20, (R, L), dtype=np.int32)
    launch = api.prepared_step(d(rows), d(counts), d(completed), d(tok), T,
                               [dict(block_table=d(bt), block_size=bs, num_blocks=NB,
                                     slot_mapping=sm, input_block_tables=ibt, k=k, v=v,
                                     k_cache=kc, v_cache=vc)], status=st, **outs)
    assert launch.path == api.STEP_RANKED_ONE_LAUNCH
    launch()
    torch.cuda.synchronize()
    prep = oracle.prepare_batch(rows, counts, completed, tok, T=T)
    want = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                       prep["seq_lens"], prep["positions"], bt, bs, NB)
    ko = np.full((short, H, D), -1, np.int16)
    vo = ko.copy()
    rc, sst = oracle.scatter_kv(k.cpu().numpy(), v.cpu().numpy(), ko, vo, want["slot_mapping"])
    assert sst == oracle.ST_SLOT_OOR                  # some slots fall past the cache
    assert_equal("slot_mapping", sm.cpu().numpy(), want["slot_mapping"])
    assert_equal("input_block_tables", ibt.cpu().numpy(), want["input_block_tables"])
    assert_equal("k_cache", kc.cpu().numpy(), ko)
    assert_equal("v_cache", vc.cpu().numpy(), vo)
    assert int(st.item()) == prep["status"] | want["status"] | sst


@pytest.mark.parametrize("extra_groups", [0, 3])
def test_ranked_maximum_batch(extra_groups):
    """The plan's largest case: 4096 requests of 16 tokens each (T = 16 n,
    65536 tokens, the ranked rule's edge) in 1 or 4 groups with block sizes 16,
    1, 64 and 3 and rows of 256, 16, 48 and 256 bytes; histories up to 4000
    tokens, so block-table rows of up to 4016 entries at block size 1."""
    rng = np.random.default_rng(4242 + extra_groups)
    n, R = 4096, 6000
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = np.full(n, 16, np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 4000, n)
    T = int(counts.sum())
    L = 4016
    groups = []
    for bs, (H, D) in [(16, (1, 128)), (1, (1, 8)), (64, (3, 8)), (3, (2, 64))][:1 + extra_groups]:
        MB = -(-L // bs)
        need = int(sum(-(-(int(completed[r]) + 16) // bs) - int(completed[r]) // bs for r in rows))
        NB = need + 17
        bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
        k = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        v = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        groups.append(workloads.KVGroup(bs, NB, MB, bt, H, D, "bf16", k, v))
    tok = rng.integers(0, 1 << 20, (R, L), dtype=np.int32)
    b = workloads.Batch(f"ranked_max_{1 + extra_groups}g", 4242, rows, counts, completed, tok,
                        groups)
    run_ranked(b, [0] * len(groups))
