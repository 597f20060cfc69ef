"""Prefix-cache block hashes and the prefix index on the GPU against the CPU
oracle: hashes bit for bit; the index compared by what it means (the live
hash -> block entries and the set of known hashes), since the slot a hash
lands in depends on the order concurrent registrations claim slots."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_equal, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_input_amd  # noqa: F401  (raises if the library is missing)
    yield
    torch.cuda.synchronize()


def up(a, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(dtype)).cuda()


def status_tensor():
    import torch

    return torch.zeros(1, dtype=torch.int32, device="cuda")


def device_hash(flat, total, starts, lengths, bs, MB):
    import torch
    from paged_kv_input_amd import api

    m = len(lengths)
    hashes = torch.zeros((m, MB), dtype=torch.int64, device="cuda")
    nf = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    st = status_tensor()
    api.hash_blocks(up(flat if len(flat) else np.zeros(1, np.int32)), up(np.asarray(starts, np.int64)),
                    up(np.asarray(lengths, np.int32)), bs, hashes=hashes, num_full=nf, status=st)
    torch.cuda.synchronize()
    return hashes.cpu().numpy().view(np.uint64), nf.cpu().numpy(), int(st.item())


def check_hash_case(flat, total, starts, lengths, bs, MB):
    got_h, got_nf, got_st = device_hash(flat, total, starts, lengths, bs, MB)
    want = oracle.hash_blocks(block_size=bs, MB=MB, views=(flat if len(flat) else np.zeros(1, np.int32),
                                                           total, starts, lengths))
    assert got_st == want["status"], (got_st, want["status"])
    assert_equal("num_full", got_nf, want["num_full"])
    assert_equal("hashes", got_h, want["hashes"])


@pytest.mark.parametrize("seed", range(30))
def test_hash_random_lists(seed):
    """Random lists over one flat array; block sizes 1..64 (3 included); long
    lists span several 256-block chunks; some views are bad (negative start,
    past the array, negative length) and some lists have more blocks than MB."""
    rng = np.random.default_rng(4400 + seed)
    bs = int(rng.choice([1, 3, 4, 16, 32, 64]))
    m = int(rng.integers(1, 40))
    total = int(rng.integers(0, 3000)) if seed % 3 else int(rng.integers(600, 1200))
    flat = rng.integers(-2**31, 2**31, total).astype(np.int32)
    starts = rng.integers(0, max(total, 1), m).astype(np.int64)
    lengths = np.array([int(rng.integers(0, total - s + 1)) if total > s else 0 for s in starts],
                       np.int32)
    if seed % 4 == 1 and m > 2:
        starts[0], lengths[1], starts[2] = -5, -3, total - 1
        lengths[2] = 7
    MB = int(rng.integers(0, 1 + (lengths.max() // bs if m else 0) + 2))
    say(f"[case] hash seed={seed} bs={bs} m={m} total={total} MB={MB}")
    check_hash_case(flat, total, starts, lengths, bs, MB)


def test_hash_token_table_rows():
    """Lists read straight from the persistent token table: starts = row * stride."""
    rng = np.random.default_rng(3)
    R, stride, bs = 50, 1030, 16
    table = rng.integers(0, 128256, (R, stride)).astype(np.int32)
    rows = rng.choice(R, 20, replace=False)
    lengths = rng.integers(0, stride, 20).astype(np.int32)
    starts = (rows * stride).astype(np.int64)
    check_hash_case(table.reshape(-1), table.size, starts, lengths, bs, stride // bs)


def test_hash_long_chain():
    """Block size 1 and 5000 tokens: 20 chunks of 256 blocks chained by the carry."""
    rng = np.random.default_rng(4)
    flat = rng.integers(0, 1000, 5000).astype(np.int32)
    check_hash_case(flat, 5000, [0, 17, 4999], [5000, 4000, 1], 1, 5000)


def make_index(cap):
    import torch
    from paged_kv_input_amd import api

    keys = torch.full((cap,), 12345, dtype=torch.int64, device="cuda")   # garbage before clear
    vals = torch.full((cap,), 7, dtype=torch.int32, device="cuda")
    api.prefix_clear(keys, vals)
    return keys, vals


def live_entries(keys, vals):
    k = keys.cpu().numpy().view(np.uint64)
    v = vals.cpu().numpy()
    return ({int(a): int(b) for a, b in zip(k, v) if a != 0 and b != oracle.NO_BLOCK},
            {int(a) for a in k if a != 0})


def test_cf_example_on_device():
    """caffein.top: A's blocks registered as P1, P2 (and its own third block);
    B hashes its two full blocks and hits P1, P2: 8 tokens computed."""
    import torch
    from paged_kv_input_amd import api

    P1, P2 = 5, 9
    system = [101, 102, 103, 104, 105, 106, 107, 108]
    a, b = system + [201, 202, 203, 204], system + [301, 302]
    flat = np.array(a + b, np.int32)
    h, nf, st = device_hash(flat, flat.size, [0, len(a)], [len(a), len(b)], 4, 3)
    assert st == 0 and nf.tolist() == [3, 2]
    keys, vals = make_index(64)
    bt = up(np.array([[P1, P2, 40]], np.int32))
    hd = up(h.view(np.int64))
    status = status_tensor()
    api.prefix_insert(hd[:1], up(np.array([0], np.int32)), up(np.array([3], np.int32)),
                      up(np.array([0], np.int32)), bt, keys, vals, status=status)
    nc = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    hits = torch.full((1, 3), -7, dtype=torch.int32, device="cuda")
    api.prefix_lookup(hd[1:], up(np.array([len(b)], np.int32)), 4, keys, vals, num_computed=nc,
                      hit_blocks=hits, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert nc.tolist() == [8]
    assert hits.tolist() == [[P1, P2, -7]]


@pytest.mark.parametrize("seed", range(30))
def test_index_random_sequences(seed):
    """Inserts, evictions and lookups with repeated hashes, against the oracle's
    index after every call.  At most `capacity` distinct hashes are used, so
    which registrations find room never depends on their order.  Block tables of
    8 entries, and (seeds 20-29) of 100 to 1500, so that every workgroup width
    the kernels choose from the table width (64 to 1024 threads, and more blocks
    than threads) runs."""
    import torch
    from paged_kv_input_amd import api

    rng = np.random.default_rng(5200 + seed)
    cap = int(rng.choice([16, 64, 1024]))
    MB, R = (8 if seed < 20 else [100, 200, 300, 700, 1500][seed % 5]), 12
    alphabet = rng.integers(1, 2**63, min(cap, 40)).astype(np.uint64)
    keys, vals = make_index(cap)
    ref = oracle.PrefixIndex(cap)
    say(f"[case] index seed={seed} cap={cap} MB={MB}")
    for op_i in range(15):
        m = int(rng.integers(1, 8))
        hashes = alphabet[rng.integers(0, alphabet.size, (m, MB))]
        hd = up(hashes.view(np.int64))
        status = status_tensor()
        op = int(rng.integers(3))
        if op == 0:
            bt = rng.integers(-1, 500, (R, MB)).astype(np.int32)
            rows = rng.choice(R, m, replace=False).astype(np.int32)
            if rng.random() < 0.2:
                rows[0] = -1
            lo = rng.integers(-1, MB + 1, m).astype(np.int32)
            hi = (lo + rng.integers(-1, 6 if MB == 8 else MB // 2, m)).astype(np.int32)
            api.prefix_insert(hd, up(lo), up(hi), up(rows), up(bt), keys, vals, status=status)
            rc, want = ref.insert(hashes, lo, hi, rows, bt)
            torch.cuda.synchronize()
            assert int(status.item()) == want, (seed, op_i, int(status.item()), want)
        elif op == 1:
            # most evictions name the entry's current block, some another one
            live = ref.live()
            blocks = np.array([live.get(int(k), 0) if rng.random() < 0.6 else int(rng.integers(500))
                               for k in hashes.reshape(-1)], np.int32)
            api.prefix_evict(hd.view(-1), up(blocks), keys, vals)
            ref.evict(hashes.reshape(-1), blocks)
        else:
            lens = rng.integers(-1, MB * 4 + 3, m).astype(np.int32)
            nc = torch.full((m,), -7, dtype=torch.int32, device="cuda")
            hits = torch.full((m, MB), -7, dtype=torch.int32, device="cuda")
            api.prefix_lookup(hd, up(lens), 4, keys, vals, num_computed=nc, hit_blocks=hits,
                              status=status)
            want = ref.lookup(hashes, lens, 4)
            torch.cuda.synchronize()
            assert int(status.item()) == want["status"]
            assert_equal("num_computed", nc.cpu().numpy(), want["num_computed"])
            assert_equal("hit_blocks", hits.cpu().numpy(), want["hit_blocks"])
        live, known = live_entries(keys, vals)
        assert live == ref.live(), (seed, op_i)
        assert known == ref.known(), (seed, op_i)


def test_index_full():
    """A full index refuses new hashes (TABLE_FULL) and still updates known ones:
    four hashes fill a 4-slot index, two more are refused, then two of the
    first four get smaller blocks."""
    import torch
    from paged_kv_input_amd import api

    cap = 4
    keys, vals = make_index(cap)
    ref = oracle.PrefixIndex(cap)
    hashes = np.arange(1, 7, dtype=np.uint64).reshape(1, 6) * np.uint64(0x9E3779B97F4A7C15)
    bt = np.array([[10, 11, 12, 13, 14, 15]], np.int32)
    for lo, hi, table, full in ((0, 4, bt, False), (4, 6, bt, True), (0, 2, bt - 5, False)):
        status = status_tensor()
        api.prefix_insert(up(hashes.view(np.int64)), up(np.array([lo], np.int32)),
                          up(np.array([hi], np.int32)), up(np.array([0], np.int32)), up(table),
                          keys, vals, status=status)
        rc, want = ref.insert(hashes, [lo], [hi], [0], table)
        torch.cuda.synchronize()
        assert int(status.item()) == want
        assert bool(want & oracle.ST_TABLE_FULL) == full
        live, known = live_entries(keys, vals)
        assert live == ref.live() and known == ref.known()
    assert sorted(ref.live().values()) == [5, 6, 12, 13]


def test_shared_prefix_batch():
    """A batch whose requests share system prompts of several lengths: hash,
    look up in an empty index (no hits), register every full block, look up
    again (each request hits its cap), all against the oracle."""
    import torch
    from paged_kv_input_amd import api

    rng = np.random.default_rng(6)
    bs, m = 16, 96
    prompts = [rng.integers(0, 128256, int(L)).tolist() for L in (40, 300, 1000, 2500)]
    lists = []
    for i in range(m):
        p = prompts[i % len(prompts)]
        lists.append(p + rng.integers(0, 128256, int(rng.integers(0, 200))).tolist())
    lengths = np.array([len(x) for x in lists], np.int32)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    flat = np.array([t for x in lists for t in x], np.int32)
    MB = int(lengths.max()) // bs + 1
    h, nf, st = device_hash(flat, flat.size, starts, lengths, bs, MB)
    want = oracle.hash_blocks(lists, bs, MB)
    assert_equal("hashes", h, want["hashes"])
    keys, vals = make_index(1 << 14)
    ref = oracle.PrefixIndex(1 << 14)
    hd = up(h.view(np.int64))
    bt = np.arange(m * MB, dtype=np.int32).reshape(m, MB)
    rows = np.arange(m, dtype=np.int32)
    for phase in range(2):
        nc = torch.full((m,), -7, dtype=torch.int32, device="cuda")
        hits = torch.full((m, MB), -7, dtype=torch.int32, device="cuda")
        status = status_tensor()
        api.prefix_lookup(hd, up(lengths), bs, keys, vals, num_computed=nc, hit_blocks=hits,
                          status=status)
        look = ref.lookup(want["hashes"], lengths, bs)
        torch.cuda.synchronize()
        assert_equal(f"phase {phase} num_computed", nc.cpu().numpy(), look["num_computed"])
        assert_equal(f"phase {phase} hit_blocks", hits.cpu().numpy(), look["hit_blocks"])
        if phase == 0:
            assert not look["num_computed"].any()
            api.prefix_insert(hd, up(np.zeros(m, np.int32)), up(nf), up(rows), up(bt), keys,
                              vals, status=status)
            ref.insert(want["hashes"], np.zeros(m, np.int32), want["num_full"], rows, bt)
            torch.cuda.synchronize()
            assert int(status.item()) == 0
    assert_equal("hits at the cap", look["num_computed"], ((lengths - 1) // bs) * bs)
    live, known = live_entries(keys, vals)
    assert live == ref.live() and known == ref.known()
