"""The paged K/V read (pkv_gather_kv) on the GPU against the CPU oracle.

Caches start from a seeded pattern (identical bits on both sides), so the
history a request reads is not just the sentinel; after a step's scatter the
read must return every row, kv_start and status word bit for bit.
"""
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


def pattern(num_slots, row_shape, salt):
    """Seeded slot- and word-dependent 16-bit words: (device int16 tensor, the
    same bits as a host uint16 array).  Built on the GPU with torch, since the
    full-size caches are gigabytes (input plumbing, not the method)."""
    import torch

    words = int(np.prod(row_shape))
    s = torch.arange(num_slots, dtype=torch.int64, device="cuda")
    base = ((s * 2654435761 + salt * 97 + 1) >> 9) & 0xFFFF
    w = ((torch.arange(words, dtype=torch.int64, device="cuda") * 40503) >> 3) & 0xFFFF
    x = (base.to(torch.int32)[:, None] ^ w.to(torch.int32)[None, :])
    dev = (x - (x >= 32768).to(torch.int32) * 65536).to(torch.int16).view(num_slots, *row_shape)
    del x
    return dev, dev.cpu().numpy().view(np.uint16)


def device_gather(seq_lens, ibt, bs, nb, kc, vc, out_tokens, fill=SENTINEL16):
    import torch
    from paged_kv_input_amd import api

    dev = kc.device
    k_out = torch.full((out_tokens, *kc.shape[1:]), fill, dtype=kc.dtype, device=dev)
    v_out = torch.full((out_tokens, *kc.shape[1:]), fill, dtype=kc.dtype, device=dev)
    kv_start = torch.full((seq_lens.shape[0] + 1,), -7, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    api.gather_kv(seq_lens, ibt, bs, nb, kc, vc, k_out=k_out, v_out=v_out, kv_start=kv_start,
                  status=status)
    torch.cuda.synchronize()
    return (k_out.cpu().numpy().view(np.uint16), v_out.cpu().numpy().view(np.uint16),
            kv_start.cpu().numpy(), int(status.item()) & 0xFFFFFFFF)


def step_then_gather(batch, mode="fused", out_extra=0, rows=None, patterned=True):
    """Step on the GPU from patterned caches, then read every group back; the
    oracle does the same from the same pattern.  rows: compare only these
    batch rows (the oracle reads just them).  patterned=False (a step with no
    history, so every row read was written by the step): caches start
    unfilled on the GPU and as lazily mapped zeros in the oracle."""
    import torch
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    say(f"[case] gather after step {batch.name} seed={batch.seed} n={batch.n} T={batch.T} "
        f"mode={mode} rows={'all' if rows is None else len(rows)}")
    if patterned:
        pats = [(pattern(g.num_slots, (g.num_heads, g.head_dim), 2 * i),
                 pattern(g.num_slots, (g.num_heads, g.head_dim), 2 * i + 1))
                for i, g in enumerate(batch.groups)]
        dev_caches = [(kp[0], vp[0]) for kp, vp in pats]
        host = [(kp[1], vp[1]) for kp, vp in pats]
    else:
        assert not batch.completed.any(), "unpatterned caches need a step with no history"
        host = [(np.zeros((g.num_slots, g.num_heads, g.head_dim), np.uint16),
                 np.zeros((g.num_slots, g.num_heads, g.head_dim), np.uint16))
                for g in batch.groups]
        dev_caches = None
    step = DeviceStep(batch.sched_rows, batch.num_scheduled, batch.completed, batch.token_ids,
                      [GroupSpec(g.block_table, g.block_size, g.num_blocks, g.k, g.v)
                       for g in batch.groups], ibt_fill=oracle.IBT_UNWRITTEN, caches=dev_caches)
    step.run_fused() if mode == "fused" else step.run()
    prep, groups_o = oracle.run_chain(batch, caches=host)
    for gi, (g, go) in enumerate(zip(batch.groups, groups_o)):
        sl = prep["seq_lens"]
        total = int(np.maximum(sl.astype(np.int64), 0).sum())
        got = device_gather(step.seq_lens, step.groups[gi]["input_block_tables"], g.block_size,
                            g.num_blocks, step.groups[gi]["k_cache"], step.groups[gi]["v_cache"],
                            total + out_extra)
        if rows is None:
            want = oracle.gather_kv(sl, go["input_block_tables"], g.block_size, g.num_blocks,
                                    go["k_cache"], go["v_cache"], total + out_extra)
            assert_equal(f"g{gi} kv_start", got[2], want["kv_start"])
            assert got[3] == want["status"], (gi, got[3], want["status"])
            assert_equal(f"g{gi} k_out", got[0], want["k"])
            assert_equal(f"g{gi} v_out", got[1], want["v"])
        else:
            want = oracle.gather_kv(sl[rows], go["input_block_tables"][rows], g.block_size,
                                    g.num_blocks, go["k_cache"], go["v_cache"])
            full_start = np.concatenate([[0], np.cumsum(np.maximum(sl.astype(np.int64), 0))])
            assert_equal(f"g{gi} kv_start", got[2], full_start)
            assert got[3] == want["status"] == 0
            for i, b in enumerate(rows):
                lo, hi = int(full_start[b]), int(full_start[b + 1])
                wl, wh = int(want["kv_start"][i]), int(want["kv_start"][i + 1])
                assert_equal(f"g{gi} k_out of batch row {b}", got[0][lo:hi], want["k"][wl:wh])
                assert_equal(f"g{gi} v_out of batch row {b}", got[1][lo:hi], want["v"][wl:wh])
    return step


def test_pages_example_read_back():
    """The kongchang.com example: B's row 31 is slot 207 (the token just
    written), A's rows 16..23 are slots 704..711."""
    b = workloads.pages_example()
    step_then_gather(b)


@pytest.mark.parametrize("name", ["seeded_16req", "seeded_16req_decode50", "decode_256x1",
                                  "mixed_8192", "prefill_16x2048", "two_groups_512req"])
def test_reduced_configs(name):
    step_then_gather(workloads.make(name, reduced=True), mode="calls")


@pytest.mark.parametrize("seed", range(24))
def test_random_tiny_after_step(seed):
    step_then_gather(workloads.random_tiny(seed, zero_counts=(seed % 4 == 3)),
                     mode=["calls", "fused"][seed % 2], out_extra=seed % 3)


def _direct_case(seed):
    """Random pages (bad ones included), negative and zero seq_lens, outputs
    shorter or longer than the sum, block sizes 1..32, rows of 1..130 chunks."""
    rng = np.random.default_rng(6100 + seed)
    n = int(rng.integers(0, 300)) if seed % 5 else int(rng.integers(0, 4))
    bs = int(rng.choice([1, 3, 4, 16, 32]))
    MB = int(rng.integers(0, 9))
    NB = int(rng.integers(1, 64))
    chunks = int(rng.choice([1, 2, 3, 8, 128, 130]))
    sl = rng.integers(-2, MB * bs + 3, n).astype(np.int32)
    ibt = rng.integers(0, NB, (n, MB)).astype(np.int32)
    if n and MB:
        bad = rng.random((n, MB)) < 0.05
        ibt[bad] = rng.choice([-1, NB, NB + 9], int(bad.sum()))
    total = int(np.maximum(sl.astype(np.int64), 0).sum())
    out_tokens = max(0, total + int(rng.integers(-5, 4)))
    return sl, ibt, bs, NB, (chunks * 8,), out_tokens


@pytest.mark.parametrize("seed", range(40))
def test_direct_random(seed):
    import torch

    sl, ibt, bs, NB, row, out_tokens = _direct_case(seed)
    say(f"[case] gather direct seed={seed} n={sl.size} MB={ibt.shape[1]} bs={bs} NB={NB} "
        f"row={row} out={out_tokens}")
    (kd, kc), (vd, vc) = pattern(NB * bs, row, 5 + seed), pattern(NB * bs, row, 105 + seed)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    got = device_gather(up(sl), up(ibt), bs, NB, kd, vd, out_tokens)
    want = oracle.gather_kv(sl, ibt, bs, NB, kc, vc, out_tokens)
    assert_equal("kv_start", got[2], want["kv_start"])
    assert got[3] == want["status"], (got[3], want["status"])
    assert_equal("k_out", got[0], want["k"])
    assert_equal("v_out", got[1], want["v"])


def test_max_batch_and_empty():
    """PKV_MAX_BATCH rows (the scan's full width), then n = 0 (kv_start = [0])."""
    import torch

    rng = np.random.default_rng(8)
    n, bs, MB, NB = 4096, 4, 3, 500
    sl = rng.integers(0, MB * bs + 1, n).astype(np.int32)
    ibt = rng.integers(0, NB, (n, MB)).astype(np.int32)
    kd, kc = pattern(NB * bs, (8,), 1)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    total = int(sl.sum())
    got = device_gather(up(sl), up(ibt), bs, NB, kd, kd, total)
    want = oracle.gather_kv(sl, ibt, bs, NB, kc, kc, total)
    assert_equal("kv_start", got[2], want["kv_start"])
    assert got[3] == want["status"] == 0
    assert_equal("k_out", got[0], want["k"])
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    got = device_gather(e, e.view(0, 3), bs, NB, kd, kd, 0)
    assert got[2].tolist() == [0] and got[3] == 0


def test_strided_outputs():
    """Output rows with a larger token stride (e.g. one buffer holding K and V)."""
    import torch
    from paged_kv_input_amd import api

    rng = np.random.default_rng(12)
    n, bs, MB, NB, H, D = 20, 16, 4, 60, 2, 32
    sl = rng.integers(0, MB * bs + 1, n).astype(np.int32)
    ibt = rng.integers(0, NB, (n, MB)).astype(np.int32)
    (kd, kc), (vd, vc) = pattern(NB * bs, (H, D), 3), pattern(NB * bs, (H, D), 4)
    total = int(sl.sum())
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    both = torch.full((total, 2, H, D), SENTINEL16, dtype=torch.int16, device="cuda")
    api.gather_kv(up(sl), up(ibt), bs, NB, kd, vd, k_out=both[:, 0], v_out=both[:, 1])
    torch.cuda.synchronize()
    want = oracle.gather_kv(sl, ibt, bs, NB, kc, vc)
    got = both.cpu().numpy().view(np.uint16)
    assert_equal("K half", got[:, 0], want["k"])
    assert_equal("V half", got[:, 1], want["v"])


def test_full_size_decode_sampled_rows():
    """The 256-request decode step at full size (about a million history rows
    per cache): every kv_start, and the rows of 12 sampled requests against
    the oracle reading just those requests."""
    b = workloads.make("decode_256x1")
    rows = sorted(np.random.default_rng(3).choice(b.n, 12, replace=False).tolist())
    step_then_gather(b, rows=rows)


def test_full_size_prefill():
    """The 32k-token prefill at full size, every row compared (no history:
    every row read is one the step wrote)."""
    step_then_gather(workloads.make("prefill_16x2048"), patterned=False)


@pytest.mark.parametrize("chunks,window", [(128, 0), (130, 0), (128, 2000), (130, 2000), (24, 0)])
def test_long_reads(chunks, window):
    """Reads long enough for tiles of several copy rounds, which move all of K,
    then all of V (about 130k rows of 2 KiB, or 2080 B, plus a read of 384-byte
    rows whose tiles stay one round): every row against the oracle, with and
    without a sliding window (query counts of 1-40 tokens, holes before the
    window's pages)."""
    import torch

    rng = np.random.default_rng(7300 + chunks + window)
    n, bs = 64, 16
    sl = rng.integers(1000, 3100, n).astype(np.int32)
    MB = int(sl.max()) // bs + 1
    NB = n * MB + 5
    ibt = rng.permutation(NB)[: n * MB].reshape(n, MB).astype(np.int32)
    counts = rng.integers(1, 41, n).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    if window:
        first = np.maximum(0, sl.astype(np.int64) - counts - window + 1) // bs
        for b in range(n):
            ibt[b, : first[b]] = -1                   # blocks freed behind the window
    row = (chunks * 8,)
    (kd, kc), (vd, vc) = pattern(NB * bs, row, 21 + chunks), pattern(NB * bs, row, 121 + chunks)
    want = oracle.gather_kv(sl, ibt, bs, NB, kc, vc, query_start_loc=qsl, sliding_window=window)
    rows = int(want["kv_start"][-1])
    say(f"[case] gather long chunks={chunks} window={window} rows={rows}")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    k_out = torch.full((rows, *row), SENTINEL16, dtype=torch.int16, device="cuda")
    v_out = torch.full_like(k_out, SENTINEL16)
    kv_start = torch.full((n + 1,), -7, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    from paged_kv_input_amd import api
    api.gather_kv(up(sl), up(ibt), bs, NB, kd, vd, k_out=k_out, v_out=v_out, kv_start=kv_start,
                  status=status, query_start_loc=up(qsl), sliding_window=window)
    torch.cuda.synchronize()
    assert_equal("kv_start", kv_start.cpu().numpy(), want["kv_start"])
    assert int(status.item()) == want["status"] == 0
    assert_equal("k_out", k_out.cpu().numpy().view(np.uint16), want["k"])
    assert_equal("v_out", v_out.cpu().numpy().view(np.uint16), want["v"])
