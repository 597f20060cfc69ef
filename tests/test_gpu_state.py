"""Persistent request-state updates on the GPU against the CPU oracle.

add_requests, append_blocks and advance_state run through the C ABI on a
DeviceState; the oracle runs the same calls on host arrays.  After every call
all four state arrays and the status word must agree bit for bit.  The last
tests close a decode loop on the device: state updates and pkv_step alternate
with no host copy of the state in between, and every step's outputs, the
caches and the state match the oracle's loop; in the serving loop requests
arrive and finish, and rows and blocks are recycled through the row pool.
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


def new_state(R, L, MB):
    from paged_kv_input_amd.state import DeviceState

    return DeviceState(R, L, MB), oracle.empty_state(R, L, MB)


def compare_state(ds, st, what):
    got = ds.host()
    for key in ("completed", "token_ids", "block_table", "row_blocks"):
        assert_equal(f"{what}: {key}", got[key], st[key])


def take_status(ds):
    bits = ds.status_bits()
    ds.status.zero_()
    return bits


def test_pages_example_rebuilt_on_device():
    """The kongchang.com example's state, registered with add_request on the GPU."""
    ref = workloads.pages_example()
    ds, st = new_state(ref.R, ref.L, ref.groups[0].max_blocks)
    rows, done = [7, 6], [31, 16]
    prompts = [ref.token_ids[7, :32].tolist(), ref.token_ids[6, :24].tolist()]
    blocks = [[37, 12], [81, 44]]
    ds.add_requests(rows, done, prompts, blocks)
    rc, want = oracle.add_requests(st, rows, done, prompts, blocks)
    assert rc == 0 and take_status(ds) == want == 0
    compare_state(ds, st, "pages example")
    assert_equal("block_table", ds.block_table.cpu().numpy(), ref.groups[0].block_table)


def test_prefix_example_append_on_device():
    """caffein.top: P1, P2 reused at registration, B3 appended -> [P1][P2][B3]."""
    ds, st = new_state(4, 12, 3)
    ds.add_requests([1], [8], [list(range(12, 22))], [[5, 9]])
    oracle.add_requests(st, [1], [8], [list(range(12, 22))], [[5, 9]])
    ds.append_blocks([1], [[2]])
    oracle.append_blocks(st, [1], [[2]])
    assert take_status(ds) == 0
    compare_state(ds, st, "prefix example")
    assert ds.block_table[1].tolist() == [5, 9, 2]


def _maybe_corrupt(rng, lists, p=0.15):
    """CSR triple of the lists, sometimes with one range pushed outside the flat
    array or reversed (the request must be skipped and BAD_RANGE raised)."""
    start, flat, total = oracle.csr(lists)
    if len(lists) and rng.random() < p:
        i = int(rng.integers(len(lists)))
        kind = int(rng.integers(3))
        if kind == 0:
            start[i + 1] = total + int(rng.integers(1, 50))
        elif kind == 1:
            start[i] = -int(rng.integers(1, 50))
        else:
            start[i], start[i + 1] = start[i] + 3, start[i]
    return start, flat, total


SHAPES = {
    # R, L, MB, longest prompt, most blocks: small, then large enough that the
    # copies span several 1024-element rounds with a ragged tail, then prompts
    # of 4500 tokens on average (the registration's wider workgroups, several
    # 4096-token rounds)
    "small": (6, 12, 4, 14, 6),
    "large": (300, 3000, 300, 3300, 320),
    "long": (64, 9000, 600, 9000, 620),
}


@pytest.mark.parametrize("shape", list(SHAPES))
def test_random_state_sequences(shape):
    R, L, MB, max_prompt, max_blocks = SHAPES[shape]
    seeds = range(40) if shape == "small" else range(6)
    for seed in seeds:
        say(f"[case] state sequence shape={shape} seed={seed}")
        rng = np.random.default_rng(9000 + seed)
        ds, st = new_state(R, L, MB)
        for op_i in range(10):
            m = int(rng.integers(0, min(R, 40) + 1))
            rows = rng.choice(R, m, replace=False).astype(np.int32)
            if m and rng.random() < 0.2:
                rows[int(rng.integers(m))] = int(rng.choice([-1, R, R + 7]))
            op = int(rng.integers(3))
            if op == 0:
                done = rng.integers(0, L, m).astype(np.int32)
                prompts = [rng.integers(0, 1 << 20, int(rng.integers(0, max_prompt + 1))).tolist()
                           for _ in range(m)]
                blocks = [rng.integers(0, 1 << 16, int(rng.integers(0, max_blocks + 1))).tolist()
                          for _ in range(m)]
                p, b = _maybe_corrupt(rng, prompts), _maybe_corrupt(rng, blocks)
                ds.add_requests(rows, done, p, b)
                rc, want = oracle.add_requests(st, rows, done, p, b)
            elif op == 1:
                blocks = [rng.integers(0, 1 << 16, int(rng.integers(0, max_blocks // 4 + 2))).tolist()
                          for _ in range(m)]
                b = _maybe_corrupt(rng, blocks)
                ds.append_blocks(rows, b)
                rc, want = oracle.append_blocks(st, rows, b)
            else:
                seq = rng.integers(-2, L + 3, m).astype(np.int32)
                sampled = rng.integers(-2, 1 << 20, m).astype(np.int32)
                use_sampled = rng.random() < 0.8
                ds.advance(rows, seq, sampled if use_sampled else None)
                rc, want = oracle.advance_state(st, rows, seq, sampled if use_sampled else None)
            assert rc == 0
            got = take_status(ds)
            assert got == want, (seed, op_i, op, got, want)
            compare_state(ds, st, f"seed {seed} op {op_i} ({op})")


def test_state_errors_match_oracle():
    """The oracle pins' error cases (bad row, prompt past L, blocks past MB,
    full row, bad CSR ranges, sampled -1, position past L) on the device."""
    ds, st = new_state(3, 4, 2)
    args = ([5, 1], [0, 2], [[1], [9, 8, 7, 6, 5, 4]], [[1], [3, 4, 5]])
    ds.add_requests(*args)
    _, want = oracle.add_requests(st, *args)
    assert take_status(ds) == want == (oracle.ST_BAD_ROW | oracle.ST_POS_OOR | oracle.ST_LB_OOR)
    compare_state(ds, st, "add")
    ds.append_blocks([1, -1], [[7], [8]])
    _, want = oracle.append_blocks(st, [1, -1], [[7], [8]])
    assert take_status(ds) == want == (oracle.ST_LB_OOR | oracle.ST_BAD_ROW)
    compare_state(ds, st, "append to a full row")
    ds.advance([1, 2, 7], [4, 1, 0], [5, -1, 3])
    _, want = oracle.advance_state(st, [1, 2, 7], [4, 1, 0], [5, -1, 3])
    assert take_status(ds) == want == (oracle.ST_POS_OOR | oracle.ST_BAD_ROW)
    compare_state(ds, st, "advance")
    ds2, st2 = new_state(3, 4, 2)
    p = (np.array([0, 3, 9], np.int32), np.array([4, 5, 6, 7], np.int32), 4)
    b = (np.array([0, 1, 2], np.int32), np.array([8, 9], np.int32), 2)
    ds2.add_requests([0, 1], [1, 1], p, b)
    _, want = oracle.add_requests(st2, [0, 1], [1, 1], p, b)
    assert take_status(ds2) == want == oracle.ST_BAD_RANGE
    compare_state(ds2, st2, "bad prompt range")


def test_empty_calls():
    ds, st = new_state(4, 8, 2)
    ds.add_requests([], [], [], [])
    ds.append_blocks([], [])
    ds.advance([], [], [])
    assert take_status(ds) == 0
    compare_state(ds, st, "empty")


@pytest.mark.parametrize("mode", ["calls", "fused"])
def test_device_decode_loop(mode):
    """Chunked prefill then decode, with the state kept only on the device:
    per step append_blocks, the step itself, then advance_state with sampled
    tokens (-1 for a prompt chunk that does not end its prompt)."""
    import torch
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    rng = np.random.default_rng(4242)
    R, L, MB, bs, NB, H, D = 64, 2048, 128, 16, 4096, 2, 64
    chunk, steps, m = 96, 14, 40
    ds, st = new_state(R, L, MB)
    pool = rng.permutation(NB).tolist()
    rows = rng.choice(R, m, replace=False).tolist()
    plen = rng.integers(1, 300, m).tolist()
    prompts = [rng.integers(0, 1 << 20, p).tolist() for p in plen]
    first = [[pool.pop() for _ in range(-(-min(p, chunk) // bs))] for p in plen]
    ds.add_requests(rows, [0] * m, prompts, first)
    oracle.add_requests(st, rows, [0] * m, prompts, first)
    kc_o = np.full((NB * bs, H, D), 0xFFFF, np.uint16)
    vc_o = np.full((NB * bs, H, D), 0xFFFF, np.uint16)
    caches = None
    for s in range(steps):
        done = st["completed"][rows]
        counts = [min(p - d, chunk) if d < p else 1 for p, d in zip(plen, done)]
        need = []
        for r, c in zip(rows, counts):
            want_blocks = -(-(int(st["completed"][r]) + c) // bs)
            need.append([pool.pop() for _ in range(max(0, want_blocks - int(st["row_blocks"][r])))])
        say(f"[case] device decode loop mode={mode} step={s} T={sum(counts)}")
        ds.append_blocks(rows, need)
        oracle.append_blocks(st, rows, need)
        T = int(sum(counts))
        k = rng.integers(-30000, 30000, (T, H, D)).astype(np.int16)
        v = rng.integers(-30000, 30000, (T, H, D)).astype(np.int16)
        step = DeviceStep(rows, counts, ds.completed, ds.token_ids,
                          [GroupSpec(ds.block_table, bs, NB, k, v)],
                          cache_fill=SENTINEL16 if caches is None else None,
                          ibt_fill=oracle.IBT_UNWRITTEN, caches=caches)
        caches = [(step.groups[0]["k_cache"], step.groups[0]["v_cache"])]
        step.run_fused() if mode == "fused" else step.run()
        prep = oracle.prepare_batch(rows, counts, st["completed"], st["token_ids"])
        sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                         prep["seq_lens"], prep["positions"], st["block_table"],
                                         bs, NB)
        rc, sst = oracle.scatter_kv(k.view(np.uint16), v.view(np.uint16), kc_o, vc_o,
                                    sm["slot_mapping"])
        assert prep["status"] == sm["status"] == sst == 0
        assert step.status_bits() == 0
        for key in ("index_mapping", "query_start_loc", "seq_lens", "positions", "input_ids"):
            assert_equal(f"step {s} {key}", step.host(key), prep[key])
        assert_equal(f"step {s} slot_mapping", step.host("slot_mapping", 0), sm["slot_mapping"])
        assert_equal(f"step {s} input_block_tables", step.host("input_block_tables", 0),
                     sm["input_block_tables"])
        # sampled in batch order: none for a chunk that leaves part of its prompt
        sampled = rng.integers(0, 1 << 20, m).astype(np.int32)
        for b_, r in enumerate(prep["index_mapping"].tolist()):
            if prep["seq_lens"][b_] < plen[rows.index(r)]:
                sampled[b_] = -1
        ds.advance(step.index_mapping, step.seq_lens, sampled)
        oracle.advance_state(st, prep["index_mapping"], prep["seq_lens"], sampled)
        assert take_status(ds) == 0
        compare_state(ds, st, f"step {s}")
    torch.cuda.synchronize()
    assert_equal("k_cache", caches[0][0].cpu().numpy().view(np.uint16), kc_o)
    assert_equal("v_cache", caches[0][1].cpu().numpy().view(np.uint16), vc_o)
    assert all(int(st["completed"][r]) > plen[i] for i, r in enumerate(rows))


def test_device_serving_loop_with_row_pool():
    """Requests arrive and finish: rows come from the library's RowPool (and
    match the oracle's pool), finished rows and their blocks are recycled to
    later requests, and the device state, step outputs and caches stay
    bit-exact with the oracle's loop throughout."""
    import torch
    from paged_kv_input_amd import RowPool
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    rng = np.random.default_rng(5151)
    R, L, MB, bs, NB, H, D = 24, 512, 32, 16, 600, 1, 64
    chunk, steps = 64, 40
    ds, st = new_state(R, L, MB)
    pool, pool_o = RowPool(R), oracle.RowPool(R)
    free_blocks = rng.permutation(NB).tolist()
    active = {}                          # row -> [prompt_len, total_len, blocks]
    kc_o = np.full((NB * bs, H, D), 0xFFFF, np.uint16)
    vc_o = np.full((NB * bs, H, D), 0xFFFF, np.uint16)
    caches, used_rows, recycled = None, set(), 0
    for s in range(steps):
        arrive = int(rng.integers(0, 4)) if len(active) < 16 else 0
        if arrive:
            rows = pool.acquire(arrive)
            rc, rows_o = pool_o.acquire(arrive)
            assert rc == 0 and rows == rows_o
            plens = rng.integers(1, 150, arrive).tolist()
            prompts = [rng.integers(0, 1 << 20, p).tolist() for p in plens]
            blocks = [[free_blocks.pop() for _ in range(-(-min(p, chunk) // bs))] for p in plens]
            ds.add_requests(rows, [0] * arrive, prompts, blocks)
            oracle.add_requests(st, rows, [0] * arrive, prompts, blocks)
            for r, p, b in zip(rows, plens, blocks):
                recycled += r in used_rows
                used_rows.add(r)
                active[r] = [p, p + int(rng.integers(1, 40)), list(b)]
        rows = list(active)
        if not rows:
            continue
        counts = [min(active[r][0] - int(st["completed"][r]), chunk)
                  if st["completed"][r] < active[r][0] else 1 for r in rows]
        need = []
        for r, c in zip(rows, counts):
            want_blocks = -(-(int(st["completed"][r]) + c) // bs)
            nb = [free_blocks.pop() for _ in range(max(0, want_blocks - int(st["row_blocks"][r])))]
            active[r][2] += nb
            need.append(nb)
        ds.append_blocks(rows, need)
        oracle.append_blocks(st, rows, need)
        T = int(sum(counts))
        say(f"[case] serving loop step={s} n={len(rows)} T={T} free_rows={pool.num_free}")
        k = rng.integers(-30000, 30000, (T, H, D)).astype(np.int16)
        v = rng.integers(-30000, 30000, (T, H, D)).astype(np.int16)
        step = DeviceStep(rows, counts, ds.completed, ds.token_ids,
                          [GroupSpec(ds.block_table, bs, NB, k, v)],
                          cache_fill=SENTINEL16 if caches is None else None,
                          ibt_fill=oracle.IBT_UNWRITTEN, caches=caches)
        caches = [(step.groups[0]["k_cache"], step.groups[0]["v_cache"])]
        step.run_fused()
        prep = oracle.prepare_batch(rows, counts, st["completed"], st["token_ids"])
        sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                         prep["seq_lens"], prep["positions"], st["block_table"],
                                         bs, NB)
        oracle.scatter_kv(k.view(np.uint16), v.view(np.uint16), kc_o, vc_o, sm["slot_mapping"])
        assert prep["status"] == sm["status"] == step.status_bits() == 0
        for key in ("index_mapping", "seq_lens", "positions", "input_ids"):
            assert_equal(f"step {s} {key}", step.host(key), prep[key])
        assert_equal(f"step {s} slot_mapping", step.host("slot_mapping", 0), sm["slot_mapping"])
        sampled = rng.integers(0, 1 << 20, len(rows)).astype(np.int32)
        for b_, r in enumerate(prep["index_mapping"].tolist()):
            if prep["seq_lens"][b_] < active[r][0]:
                sampled[b_] = -1
        ds.advance(step.index_mapping, step.seq_lens, sampled)
        oracle.advance_state(st, prep["index_mapping"], prep["seq_lens"], sampled)
        assert take_status(ds) == 0
        compare_state(ds, st, f"step {s}")
        done = [r for r in rows if st["completed"][r] >= active[r][1]]
        if done:
            pool.release(done)
            assert pool_o.release(done) == 0
            for r in done:
                free_blocks.extend(active.pop(r)[2])
        assert pool.num_free == pool_o.free == R - len(active)
    torch.cuda.synchronize()
    assert_equal("k_cache", caches[0][0].cpu().numpy().view(np.uint16), kc_o)
    assert_equal("v_cache", caches[0][1].cpu().numpy().view(np.uint16), vc_o)
    assert recycled > 0, "no row was recycled: the loop is too short"


def test_second_group_registration():
    """A second KV-cache group: the same requests registered again with that
    group's block table and empty prompts leaves the tokens alone."""
    import torch

    rng = np.random.default_rng(77)
    R, L = 16, 200
    ds, st = new_state(R, L, 12)
    rows = rng.choice(R, 6, replace=False).tolist()
    done = rng.integers(0, 100, 6).tolist()
    prompts = [rng.integers(0, 1000, int(rng.integers(1, 200))).tolist() for _ in rows]
    ds.add_requests(rows, done, prompts, [[1, 2]] * 6)
    oracle.add_requests(st, rows, done, prompts, [[1, 2]] * 6)
    # group 1: its own table (width 5) and block counts
    bt1 = torch.full((R, 5), -1, dtype=torch.int32, device=ds.device)
    rb1 = torch.zeros(R, dtype=torch.int32, device=ds.device)
    st1 = {"completed": st["completed"], "token_ids": st["token_ids"],
           "block_table": np.full((R, 5), -1, np.int32), "row_blocks": np.zeros(R, np.int32)}
    blocks1 = [rng.integers(0, 50, int(rng.integers(0, 6))).tolist() for _ in rows]
    from paged_kv_input_amd import api
    from paged_kv_input_amd.state import pack_csr

    ps, pt, _ = pack_csr([[] for _ in rows])
    bs_, bl, bt = pack_csr(blocks1)
    up = ds._up
    api.add_requests(up(rows), up(done), up(ps), up(pt)[:0], up(bs_), up(bl)[:bt],
                     completed=ds.completed, token_ids=ds.token_ids, block_table=bt1,
                     row_blocks=rb1, status=ds.status)
    rc, want = oracle.add_requests(st1, rows, done, [[] for _ in rows], blocks1)
    assert rc == 0 and take_status(ds) == want
    compare_state(ds, st, "group 0 after group 1's registration")
    assert_equal("group 1 block_table", bt1.cpu().numpy(), st1["block_table"])
    assert_equal("group 1 row_blocks", rb1.cpu().numpy(), st1["row_blocks"])
