"""HIP path against the CPU oracle, element by element, on seeded inputs.

Index tensors and caches must be bit-exact: the path is integer index
arithmetic plus a bit copy, so there is no tolerance anywhere.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (SENTINEL16, assert_equal, compare_caches_at_slots, compare_caches_full,
                      compare_indices, device_step, oracle_chain, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_input_amd  # noqa: F401  (raises if the library is missing)
    yield
    torch.cuda.synchronize()


MODES = ["calls", "fused"]


def run_and_compare(batch, full_cache=True, mode="calls"):
    import torch

    say(f"[case] {batch.name} seed={batch.seed} n={batch.n} T={batch.T} mode={mode} "
        f"groups={[(g.block_size, g.num_blocks) for g in batch.groups]}")
    step = device_step(batch)
    if mode == "fused":
        step.run_fused()
    else:
        step.run()
    torch.cuda.synchronize()
    prep, groups_o = oracle_chain(batch, lazy_caches=not full_cache)
    compare_indices(step, prep, groups_o)
    want = prep["status"]
    for go in groups_o:
        want |= go["status"] | go["scatter_status"]
    assert step.status_bits() == want, (step.status_bits(), want)
    if full_cache:
        compare_caches_full(step, groups_o)
    else:
        compare_caches_at_slots(step, batch, groups_o)
    return step, prep, groups_o


@pytest.mark.parametrize("mode", MODES)
def test_pages_example(mode):
    b = workloads.pages_example()
    step, prep, go = run_and_compare(b, mode=mode)
    # the values the article prints, read straight off the GPU
    assert step.host("query_start_loc").tolist() == [0, 1, 9]
    assert step.host("positions").tolist() == [31] + list(range(16, 24))
    assert int(step.host("slot_mapping", 0)[0]) == 207
    assert step.host("slot_mapping", 0)[1:].tolist() == list(range(704, 712))


@pytest.mark.parametrize("maker", [workloads.prefix_reuse_example, workloads.budget_tie_example],
                         ids=["prefix_reuse", "budget_tie"])
@pytest.mark.parametrize("mode", MODES)
def test_page_examples_other(maker, mode):
    run_and_compare(maker(), mode=mode)


@pytest.mark.parametrize("name", ["seeded_16req", "seeded_16req_decode50"])
@pytest.mark.parametrize("mode", MODES)
def test_seeded_small(name, mode):
    run_and_compare(workloads.make(name), mode=mode)


@pytest.mark.parametrize("name", ["decode_256x1", "mixed_8192", "prefill_16x2048",
                                  "prefill_16x2048_tp8", "two_groups_512req"])
@pytest.mark.parametrize("mode", MODES)
def test_reduced(name, mode):
    run_and_compare(workloads.make(name, reduced=True), full_cache=False, mode=mode)


@pytest.mark.parametrize("seed", range(32))
@pytest.mark.parametrize("mode", MODES)
def test_tiny_random(seed, mode):
    b = workloads.random_tiny(1000 + seed, zero_counts=(seed % 4 == 3))
    run_and_compare(b, mode=mode)


@pytest.mark.parametrize("name", ["decode_256x1", "mixed_8192", "prefill_16x2048",
                                  "two_groups_512req", "decode_4096x1"])
@pytest.mark.parametrize("mode", MODES)
def test_full_size(name, mode):
    """Full configuration sizes, the launch configuration the benchmark times."""
    import torch

    b = workloads.make(name)
    run_and_compare(b, full_cache=False, mode=mode)
    torch.cuda.empty_cache()


def test_shuffled_schedule_same_outputs():
    b = workloads.make("mixed_8192", reduced=True)
    s1 = device_step(b)
    s1.run()
    perm = np.random.default_rng(9).permutation(b.n)
    b.sched_rows, b.num_scheduled = b.sched_rows[perm], b.num_scheduled[perm]
    s2 = device_step(b)
    s2.run()
    for key in ("index_mapping", "query_start_loc", "seq_lens", "positions", "input_ids"):
        assert_equal(key, s2.host(key), s1.host(key))
    assert_equal("slot_mapping", s2.host("slot_mapping", 0), s1.host("slot_mapping", 0))


@pytest.mark.parametrize("mode", MODES)
def test_max_batch(mode):
    """n = PKV_MAX_BATCH requests (the keys held in LDS), counts 0..3, ties galore;
    in fused mode this exceeds the one-launch limit and takes the separate kernels."""
    import paged_kv_input_amd as pkv

    rng = np.random.default_rng(21)
    n, R, L, bs = pkv.MAX_BATCH, pkv.MAX_BATCH + 100, 64, 16
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    counts = rng.integers(0, 4, n).astype(np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 60, n)
    MB = L // bs
    need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                   for r, c in zip(rows, counts)))
    NB = need + 7
    bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
    T = int(counts.sum())
    k = rng.integers(0, 65535, (T, 1, 8), dtype=np.uint16)
    v = rng.integers(0, 65535, (T, 1, 8), dtype=np.uint16)
    b = workloads.Batch("max_batch", 21, rows, counts, completed,
                        rng.integers(0, 1000, (R, L), dtype=np.int32),
                        [workloads.KVGroup(bs, NB, MB, bt, 1, 8, "fp16", k, v)])
    run_and_compare(b, mode=mode)


def test_empty_and_degenerate():
    import torch
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    # n = 0, T = 0: only query_start_loc[0] = 0 is produced
    bt = np.full((4, 2), -1, np.int32)
    g = GroupSpec(bt, 16, 8, np.zeros((0, 1, 8), np.uint16), np.zeros((0, 1, 8), np.uint16))
    s = DeviceStep(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(4, np.int32),
                   np.zeros((4, 8), np.int32), [g], cache_fill=SENTINEL16)
    s.query_start_loc.fill_(77)
    s.run()
    torch.cuda.synchronize()
    assert s.host("query_start_loc").tolist() == [0]
    assert s.status_bits() == 0
    # every request with an empty run: rows ordered, no tokens, nothing written
    b = workloads.random_tiny(5)
    b.num_scheduled[:] = 0
    for gg in b.groups:
        gg.k, gg.v = gg.k[:0], gg.v[:0]
    run_and_compare(b)


def test_strided_kv_and_payload_widths():
    """K/V as views into a fused per-token buffer; 1-, 2- and 4-byte payloads;
    a row of 48 chunks (not a power of two) and a block size of 3."""
    import torch
    import paged_kv_input_amd as pkv

    rng = np.random.default_rng(33)
    for dtype, H, D, bs in ((torch.int8, 2, 64, 16), (torch.int16, 3, 128, 3),
                            (torch.int32, 4, 32, 64)):
        T = 300
        NB = -(-400 // bs)
        num_slots = NB * bs
        say(f"[case] strided dtype={dtype} H={H} D={D} bs={bs}")
        fused = torch.randint(-100, 100, (T, 3, H, D), dtype=torch.int32).to(dtype).cuda()
        k, v = fused[:, 1], fused[:, 2]
        slots = rng.choice(num_slots, T, replace=False).astype(np.int32)
        slots[::17] = -1                             # padding tokens
        kc = torch.zeros((num_slots, H, D), dtype=dtype, device="cuda")
        vc = torch.zeros_like(kc)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        pkv.scatter_kv(k, v, kc, vc, torch.from_numpy(slots).cuda(), status=st)
        torch.cuda.synchronize()
        ko = np.zeros((num_slots, H, D), dtype=kc.cpu().numpy().dtype)
        vo = np.zeros_like(ko)
        rc, ost = oracle.scatter_kv(k.cpu().numpy(), v.cpu().numpy(), ko, vo, slots)
        assert rc == 0 and ost == 0 and int(st.item()) == 0
        assert_equal("k_cache", kc.cpu().numpy(), ko)
        assert_equal("v_cache", vc.cpu().numpy(), vo)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 511, 512, 513])
def test_fused_batch_sizes(n):
    """Batch sizes around the one-wave sort's lane multiples and the fused limit."""
    rng = np.random.default_rng(100 + n)
    R, L, bs = n + 37, 96, 16
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    # n > 64 sorts with every wavefront of the workgroup, n > 512 takes the
    # separate kernels; short runs keep the large cases quick
    counts = rng.integers(0, 40 if n < 256 else 3, n).astype(np.int32)
    counts[rng.random(n) < 0.4] = 1
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 50, n)
    MB = L // bs
    need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                   for r, c in zip(rows, counts)))
    NB = need + 11
    bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
    T = int(counts.sum())
    k = rng.integers(0, 65535, (T, 2, 64), dtype=np.uint16)
    v = rng.integers(0, 65535, (T, 2, 64), dtype=np.uint16)
    b = workloads.Batch(f"fused_n{n}", 100 + n, rows, counts, completed,
                        rng.integers(0, 1000, (R, L), dtype=np.int32),
                        [workloads.KVGroup(bs, NB, MB, bt, 2, 64, "fp16", k, v)])
    run_and_compare(b, mode="fused")


def _random_batch(seed):
    """A seeded random step across the batch-size regimes of the fused step
    (1-64, 65-128, 129-256 and 257-512 requests): counts with many ties and
    some zeros, 1-3 groups with block sizes from 1 to 64 (3 included), rows of
    16 B to 2 KiB."""
    rng = np.random.default_rng(seed)
    lo, hi = [(1, 65), (65, 129), (129, 257), (257, 513)][seed % 4]
    n = int(rng.integers(lo, hi))
    R = n + int(rng.integers(0, 2 * n + 1))
    rows = rng.choice(R, n, replace=False).astype(np.int32)
    base = rng.choice([1, 2, 3, 7, 16])
    counts = np.where(rng.random(n) < 0.5, base, rng.integers(0, 24, n)).astype(np.int32)
    L = 64 + 24
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 64, n)
    T = int(counts.sum())
    groups = []
    for _ in range(int(rng.integers(1, 4))):
        bs = int(rng.choice([1, 3, 4, 8, 16, 32, 64]))
        MB = -(-L // bs)
        need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                       for r, c in zip(rows, counts)))
        NB = need + int(rng.integers(1, 64))
        bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
        H, D = [(1, 8), (2, 64), (8, 128), (4, 32)][int(rng.integers(0, 4))]
        k = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        v = rng.integers(0, 65535, (T, H, D), dtype=np.uint16)
        groups.append(workloads.KVGroup(bs, NB, MB, bt, H, D, "fp16", k, v))
    tok = rng.integers(0, 1 << 20, (R, L), dtype=np.int32)
    return workloads.Batch(f"sweep_{seed}", seed, rows, counts, completed, tok, groups)


@pytest.mark.parametrize("seed", range(24))
def test_fused_random_sweep(seed):
    run_and_compare(_random_batch(1000 + seed), mode="fused")


@pytest.mark.parametrize("wide", [False, True])
def test_fused_many_state_rows(wide):
    """100 requests among 2^20 state rows (rows 0 and 2^20 - 1 included), counts
    up to 30, and with one count of 31: the fused step against the oracle."""
    rng = np.random.default_rng(4242 + wide)
    n, R, L, bs = 100, 1 << 20, 64, 16
    rows = rng.choice(R - 2, n, replace=False).astype(np.int32) + 1
    rows[3], rows[50] = 0, R - 1
    counts = rng.integers(1, 31, n).astype(np.int32)
    counts[rng.random(n) < 0.3] = 1
    if wide:
        counts[17] = 31
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, L - 31, n)
    MB = L // bs
    need = int(sum(max(0, -(-(int(completed[r]) + int(c)) // bs) - int(completed[r]) // bs)
                   for r, c in zip(rows, counts)))
    NB = need + 5
    bt = workloads._block_table(rng, R, MB, NB, bs, rows, counts, completed)
    T = int(counts.sum())
    k = rng.integers(0, 65535, (T, 1, 64), dtype=np.uint16)
    v = rng.integers(0, 65535, (T, 1, 64), dtype=np.uint16)
    tok = np.zeros((R, L), np.int32)
    tok[rows] = rng.integers(0, 1 << 20, (n, L), dtype=np.int32)
    b = workloads.Batch(f"rows2e20_{int(wide)}", 4242 + wide, rows, counts,
                        completed, tok, [workloads.KVGroup(bs, NB, MB, bt, 1, 64, "fp16", k, v)])
    run_and_compare(b, mode="fused")


@pytest.mark.parametrize("groups", [4, 5, 7])
def test_fused_group_counts(groups):
    """pkv_step with up to the kernel's group limit in one launch, and past it
    (the separate kernels); mixed block sizes and row widths."""
    b = workloads.random_tiny(900 + groups, max_n=8, max_T=64, groups=groups)
    run_and_compare(b, mode="fused")


@pytest.mark.parametrize("mode", MODES)
def test_error_inputs_match_oracle(mode):
    """Bad rows, negative counts, a token-sum mismatch, positions past the table,
    missing blocks and a short cache: same outputs and status bits as the oracle,
    and nothing written out of bounds (every access is bounds-checked)."""
    R, L, MB, bs, NB = 6, 10, 3, 4, 8
    completed = np.array([0, 2, 3, 9, -1, 5], np.int32)
    tok = (np.arange(R)[:, None] * 100 + np.arange(L)[None, :]).astype(np.int32)
    rows = np.array([1, 9, 2, 3, 4], np.int32)
    counts = np.array([2, 1, -2, 3, 1], np.int32)
    bt = np.array([[0, 1, 2], [3, -1, 9], [4, 5, 6], [7, -1, -1], [2, 2, 2], [1, 1, 1]], np.int32)
    T = 9
    rng = np.random.default_rng(4)
    k = rng.integers(0, 65000, (T, 1, 8), dtype=np.uint16)
    v = rng.integers(0, 65000, (T, 1, 8), dtype=np.uint16)
    import torch
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    # T is the host's count, deliberately larger than the counts' sum (7)
    step = DeviceStep(rows, counts, completed, tok, [GroupSpec(bt, bs, NB, k, v)],
                      cache_fill=SENTINEL16, ibt_fill=oracle.IBT_UNWRITTEN, num_tokens=T)
    if mode == "fused":
        step.run_fused()
    else:
        step.run()
    torch.cuda.synchronize()
    prep = oracle.prepare_batch(rows, counts, completed, tok, T=T)
    go = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                     prep["seq_lens"], prep["positions"], bt, bs, NB)
    kc = np.full((NB * bs, 1, 8), 0xFFFF, np.uint16)
    vc = kc.copy()
    rc, sst = oracle.scatter_kv(k, v, kc, vc, go["slot_mapping"])
    for key in ("index_mapping", "query_start_loc", "seq_lens", "positions", "input_ids"):
        assert_equal(key, step.host(key), prep[key])
    assert_equal("slot_mapping", step.host("slot_mapping", 0), go["slot_mapping"])
    assert_equal("input_block_tables", step.host("input_block_tables", 0),
                 go["input_block_tables"])
    assert_equal("k_cache", step.host("k_cache", 0).view(np.uint16), kc)
    assert_equal("v_cache", step.host("v_cache", 0).view(np.uint16), vc)
    assert step.status_bits() == prep["status"] | go["status"] | sst, \
        (step.status_bits(), prep["status"], go["status"], sst)


def test_scatter_skips_negative_and_flags_out_of_range_slots():
    import torch
    import paged_kv_input_amd as pkv

    rng = np.random.default_rng(8)
    T, H, D, num_slots = 40, 2, 16, 64
    k = torch.from_numpy(rng.integers(-30000, 30000, (T, H, D), dtype=np.int16)).cuda()
    v = torch.from_numpy(rng.integers(-30000, 30000, (T, H, D), dtype=np.int16)).cuda()
    slots = rng.choice(num_slots, T, replace=False).astype(np.int32)
    slots[3], slots[11], slots[20] = -1, num_slots, num_slots + 1000
    kc = torch.zeros((num_slots, H, D), dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.scatter_kv(k, v, kc, vc, torch.from_numpy(slots).cuda(), status=st)
    torch.cuda.synchronize()
    ko = np.zeros((num_slots, H, D), np.int16)
    vo = np.zeros_like(ko)
    rc, ost = oracle.scatter_kv(k.cpu().numpy(), v.cpu().numpy(), ko, vo, slots)
    assert rc == 0 and ost == oracle.ST_SLOT_OOR == int(st.item())
    assert_equal("k_cache", kc.cpu().numpy(), ko)
    assert_equal("v_cache", vc.cpu().numpy(), vo)


@pytest.mark.parametrize("name", ["seeded_16req", "mixed_8192", "two_groups_512req"])
def test_later_layers_reuse_slot_mapping(name):
    """One model step over four layers: pkv_step writes layer 0 and produces
    each group's slot_mapping; layers 1-3 scatter their own K/V with
    pkv_scatter_kv into their own caches through those slots.  Every layer's
    rows at the oracle's slots hold that layer's payload, and no other row of
    its caches was written (the payload never holds the 0xFFFF sentinel)."""
    import torch
    from paged_kv_input_amd import api

    b = workloads.make(name, reduced=True) if name != "seeded_16req" else workloads.make(name)
    step, prep, groups_o = run_and_compare(b, full_cache=False, mode="fused")
    rng = np.random.default_rng(4040)
    for layer in range(1, 4):
        for gi, (g, go) in enumerate(zip(b.groups, groups_o)):
            say(f"[case] {b.name} layer {layer} group {gi}")
            k = rng.integers(0, 65535, (b.T, g.num_heads, g.head_dim), dtype=np.uint16)
            v = rng.integers(0, 65535, (b.T, g.num_heads, g.head_dim), dtype=np.uint16)
            shape = (g.num_slots, g.num_heads, g.head_dim)
            kc = torch.full(shape, SENTINEL16, dtype=torch.int16, device="cuda")
            vc = torch.full(shape, SENTINEL16, dtype=torch.int16, device="cuda")
            st = torch.zeros(1, dtype=torch.int32, device="cuda")
            api.scatter_kv(torch.from_numpy(k.view(np.int16)).cuda(),
                           torch.from_numpy(v.view(np.int16)).cuda(), kc, vc,
                           step.groups[gi]["slot_mapping"], status=st)
            torch.cuda.synchronize()
            assert int(st.item()) == 0
            slots = np.asarray(go["slot_mapping"])
            tok = np.flatnonzero(slots >= 0)
            idx = torch.from_numpy(slots[tok].astype(np.int64)).cuda()
            for key, cache, pay in (("k", kc, k), ("v", vc, v)):
                got = cache.index_select(0, idx).cpu().numpy().view(np.uint16)
                assert_equal(f"layer {layer} g{gi} {key} rows", got, pay[tok])
                written = int((cache != SENTINEL16).flatten(1).any(dim=1).sum().item())
                assert written == tok.size, (key, written, tok.size)
