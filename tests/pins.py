"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` function takes a loaded oracle library (the real one, or a copy
with a planted mistake) and raises AssertionError when the oracle disagrees
with: the values the pages print for their worked examples (golden files under
tests/golden/), brute force on tiny batches, NumPy library routines, closed
forms, or invariants.  test_oracle_pins.py runs them on the oracle;
test_oracle_mutants.py checks that each planted mistake fails at least one.
"""
import json
import os
import struct

import numpy as np

import oracle
import workloads
from bruteforce import chain as brute_chain
from bruteforce import gather_slots as brute_gather_slots

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _eq(a, b, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape and np.array_equal(a, b), f"{what}: {a.tolist()} != {b.tolist()}"


# ---------------------------------------------------------------------------
# the pages' worked examples
# ---------------------------------------------------------------------------

def pin_pages_example(lib):
    """Printed and derived values of the kongchang.com worked example."""
    g = _golden("pages_example.json")
    b = workloads.pages_example()
    prep, groups = oracle.run_chain(b, lib=lib)
    assert prep["rc"] == 0 and prep["status"] == 0
    _eq(prep["query_start_loc"], g["printed"]["query_start_loc"], "query_start_loc")
    _eq(prep["positions"], g["printed"]["positions"], "positions")
    first = g["printed"]["first_token_of_B"]
    t = first["flat_token_index"]
    gr = groups[0]
    assert gr["rc"] == 0 and gr["status"] == 0
    assert int(prep["positions"][t]) == first["position"]
    bs = b.groups[0].block_size
    assert int(prep["positions"][t]) // bs == first["logic_block"]
    assert int(prep["positions"][t]) % bs == first["offset"]
    assert int(gr["slot_mapping"][t]) == first["slot_id"]
    assert int(gr["slot_mapping"][t]) // bs == first["physical_block_id"]
    d = g["derived"]
    _eq(prep["index_mapping"], d["index_mapping"], "index_mapping")
    _eq(prep["seq_lens"], d["seq_lens"], "seq_lens")
    _eq(gr["slot_mapping"], d["slot_mapping"], "slot_mapping")
    _eq(gr["input_block_tables"], d["input_block_tables"], "input_block_tables")
    _eq(prep["input_ids"], d["input_ids_identity_code"], "input_ids")
    k, v = b.groups[0].k, b.groups[0].v
    kc, vc = gr["k_cache"], gr["v_cache"]
    _eq(kc[207], k[0], "K at slot 207")
    _eq(vc[207], v[0], "V at slot 207")
    for i in range(8):
        _eq(kc[704 + i], k[1 + i], f"K at slot {704 + i}")
        _eq(vc[704 + i], v[1 + i], f"V at slot {704 + i}")
    written = np.any(kc != 0xFFFF, axis=(1, 2))
    assert int(written.sum()) == 9


def pin_prefix_example(lib):
    """The caffein.top prefix-reuse example: [P1][P2][B3], 8 reused + 2 new tokens."""
    g = _golden("prefix_reuse_example.json")
    inst = g["inputs"]["instantiate"]
    b = workloads.prefix_reuse_example(inst["P1"], inst["P2"], inst["B3"])
    prep, groups = oracle.run_chain(b, lib=lib)
    e = g["expected"]
    _eq(prep["index_mapping"], e["index_mapping"], "index_mapping")
    _eq(prep["query_start_loc"], e["query_start_loc"], "query_start_loc")
    _eq(prep["seq_lens"], e["seq_lens"], "seq_lens")
    _eq(prep["positions"], e["positions"], "positions")
    bs = g["inputs"]["block_size"]
    _eq(prep["positions"] // bs, e["logic_block"], "logic_block")
    b3 = inst["B3"]
    _eq(groups[0]["slot_mapping"], [bs * b3, bs * b3 + 1], "slot_mapping")
    _eq(groups[0]["input_block_tables"], [[inst["P1"], inst["P2"], b3]], "input_block_tables")


def pin_budget_tie_example(lib):
    """The caffein.top budget example: equal counts, order fixed by the tie-break."""
    g = _golden("budget_tie_example.json")
    b = workloads.budget_tie_example()
    prep, _ = oracle.run_chain(b, lib=lib)
    e = g["expected"]
    for key in ("index_mapping", "query_start_loc", "seq_lens", "positions"):
        _eq(prep[key], e[key], key)


# ---------------------------------------------------------------------------
# brute force on tiny batches
# ---------------------------------------------------------------------------

def pin_bruteforce(lib, seeds=range(200)):
    for seed in seeds:
        b = workloads.random_tiny(seed, zero_counts=(seed % 5 == 4))
        prep, groups = oracle.run_chain(b, lib=lib)
        bf = brute_chain(b.sched_rows, b.num_scheduled, b.completed, b.token_ids,
                         [(g.block_table.tolist(), g.block_size) for g in b.groups])
        for key in ("index_mapping", "query_start_loc", "seq_lens", "positions", "input_ids"):
            _eq(prep[key], bf[key], f"seed {seed} {key}")
        assert prep["status"] == 0, f"seed {seed} status {prep['status']}"
        for gi, (g, gr, bg) in enumerate(zip(b.groups, groups, bf["groups"])):
            _eq(gr["slot_mapping"], bg["slot_mapping"], f"seed {seed} g{gi} slot_mapping")
            for bi, vis in enumerate(bg["input_block_tables"]):
                row = gr["input_block_tables"][bi]
                _eq(row[:len(vis)], vis, f"seed {seed} g{gi} ibt row {bi}")
                assert np.all(row[len(vis):] == oracle.IBT_UNWRITTEN), f"seed {seed} ibt tail"
            assert gr["status"] == 0
            # scatter: NumPy fancy-index assignment of the brute-force slots
            kc = np.full_like(gr["k_cache"], 0xFFFF)
            vc = np.full_like(gr["v_cache"], 0xFFFF)
            s = np.asarray(bg["slot_mapping"], np.int64)
            kc[s] = g.k
            vc[s] = g.v
            _eq(gr["k_cache"], kc, f"seed {seed} g{gi} k_cache")
            _eq(gr["v_cache"], vc, f"seed {seed} g{gi} v_cache")


# ---------------------------------------------------------------------------
# library routines and closed forms on seeded configs
# ---------------------------------------------------------------------------

def _library_chain(b):
    """The same outputs from NumPy routines: lexsort, cumsum, repeat, searchsorted."""
    order = np.lexsort((b.sched_rows, b.num_scheduled))
    im = b.sched_rows[order]
    counts = b.num_scheduled[order].astype(np.int64)
    qsl = np.concatenate([[0], np.cumsum(counts)])
    T = int(qsl[-1])
    owner = np.repeat(np.arange(im.size), counts)
    assert np.array_equal(owner, np.searchsorted(qsl, np.arange(T), side="right") - 1)
    pos = b.completed[im][owner] + (np.arange(T) - qsl[owner])
    ids = b.token_ids[im[owner], pos]
    seq = b.completed[im] + counts
    return im, qsl, seq, pos, ids, owner


def pin_library_routines(lib, names=("seeded_16req", "seeded_16req_decode50")):
    for name in names:
        b = workloads.make(name)
        prep, groups = oracle.run_chain(b, lib=lib)
        im, qsl, seq, pos, ids, owner = _library_chain(b)
        _eq(prep["index_mapping"], im, f"{name} index_mapping")
        _eq(prep["query_start_loc"], qsl, f"{name} query_start_loc")
        _eq(prep["seq_lens"], seq, f"{name} seq_lens")
        _eq(prep["positions"], pos, f"{name} positions")
        _eq(prep["input_ids"], ids, f"{name} input_ids")
        for g, gr in zip(b.groups, groups):
            bt = g.block_table
            bs = g.block_size
            blk = bt[im[owner], pos // bs]
            _eq(gr["slot_mapping"], blk * bs + pos % bs, f"{name} slot_mapping")
            kc = np.full_like(gr["k_cache"], 0xFFFF)
            kc[gr["slot_mapping"]] = g.k
            _eq(gr["k_cache"], kc, f"{name} k_cache")


def pin_closed_forms(lib):
    """Identity token table and a contiguous block table (the textbook
    unpaged cache: request r owns slots [r*MB*bs, (r+1)*MB*bs))."""
    rng = np.random.default_rng(7)
    for bs in (1, 3, 16):
        R, n, L = 12, 9, 40
        MB = -(-L // bs)
        rows = rng.choice(R, n, replace=False).astype(np.int32)
        counts = rng.integers(0, 7, n).astype(np.int32)
        completed = np.zeros(R, np.int32)
        completed[rows] = rng.integers(0, L - 7, n)
        tok = (np.arange(R)[:, None] * L + np.arange(L)[None, :]).astype(np.int32)
        prep = oracle.prepare_batch(rows, counts, completed, tok, lib=lib)
        im, qsl = prep["index_mapping"], prep["query_start_loc"]
        pos, ids = prep["positions"], prep["input_ids"]
        T = int(qsl[-1])
        assert T == int(counts.sum())
        owner = np.searchsorted(qsl, np.arange(T), side="right") - 1
        _eq(ids // L, im[owner], f"bs {bs} input_ids row code")
        _eq(ids % L, pos, f"bs {bs} input_ids position code")
        bt = (np.arange(R)[:, None] * MB + np.arange(MB)[None, :]).astype(np.int32)
        sm = oracle.compute_slot_mapping(im, qsl, prep["seq_lens"], pos, bt, bs, R * MB, lib=lib)
        _eq(sm["slot_mapping"], im[owner].astype(np.int64) * MB * bs + pos, f"bs {bs} contiguous")
        if bs == 1:
            _eq(sm["slot_mapping"], bt[im[owner], pos], "bs 1: slot = block_table[row][pos]")


def pin_invariants(lib, names=("seeded_16req", "seeded_16req_decode50")):
    for name in names:
        b = workloads.make(name)
        prep, groups = oracle.run_chain(b, lib=lib)
        im, qsl, pos = prep["index_mapping"], prep["query_start_loc"], prep["positions"]
        counts = np.diff(qsl)
        assert sorted(im.tolist()) == sorted(b.sched_rows.tolist()), "permutation"
        assert np.all(np.diff(counts) >= 0), "counts non-decreasing along the batch"
        assert qsl[0] == 0 and qsl[-1] == b.T
        # independent of the order the host lists the schedule in
        perm = np.random.default_rng(3).permutation(b.n)
        p2 = oracle.prepare_batch(b.sched_rows[perm], b.num_scheduled[perm], b.completed,
                                  b.token_ids, lib=lib)
        for key in ("index_mapping", "query_start_loc", "seq_lens", "positions", "input_ids"):
            _eq(p2[key], prep[key], f"{name} shuffled {key}")
        for bb in range(b.n):
            seg = pos[qsl[bb]:qsl[bb + 1]]
            _eq(seg, b.completed[im[bb]] + np.arange(counts[bb]), f"{name} run {bb}")
        for g, gr in zip(b.groups, groups):
            s = gr["slot_mapping"]
            bs = g.block_size
            assert np.unique(s).size == s.size, "slots unique"
            _eq(s % bs, pos % bs, "offset kept")
            owner = np.searchsorted(qsl, np.arange(b.T), side="right") - 1
            for t in range(b.T):
                vis = -(-int(prep["seq_lens"][owner[t]]) // bs)
                assert s[t] // bs in g.block_table[im[owner[t]], :vis], "slot in a visible block"
            _eq(gr["k_cache"][s], g.k, "gather by slot reproduces K")
            _eq(gr["v_cache"][s], g.v, "gather by slot reproduces V")
            nonsent = np.any(gr["k_cache"] != 0xFFFF, axis=(1, 2))
            assert int(nonsent.sum()) == b.T, "no stray writes"


def pin_error_semantics(lib):
    """Data errors give the documented outputs and status bits (the readings of
    what the pages leave open), and nothing is written for them."""
    R, L, MB, bs, NB = 6, 10, 3, 4, 8
    completed = np.array([0, 2, 3, 9, -1, 5], np.int32)
    tok = (np.arange(R)[:, None] * 100 + np.arange(L)[None, :]).astype(np.int32)
    # row 9 is out of range; count -2 reads as 0; row 3 runs past L; row 4 starts negative
    rows = np.array([1, 9, 2, 3, 4], np.int32)
    counts = np.array([2, 1, -2, 3, 1], np.int32)
    prep = oracle.prepare_batch(rows, counts, completed, tok, T=9, lib=lib)
    st = prep["status"]
    assert st == (oracle.ST_BAD_ROW | oracle.ST_BAD_COUNT | oracle.ST_TOKEN_SUM | oracle.ST_POS_OOR), st
    # order by (count, row): (0,2) (1,4) (1,9) (2,1) (3,3)
    _eq(prep["index_mapping"], [2, 4, 9, 1, 3], "index_mapping")
    _eq(prep["query_start_loc"], [0, 0, 1, 2, 4, 7], "query_start_loc")
    _eq(prep["seq_lens"], [3, 0, -1, 4, 12], "seq_lens")
    _eq(prep["positions"], [-1, -1, 2, 3, 9, 10, 11, -1, -1], "positions")
    _eq(prep["input_ids"], [-1, -1, 102, 103, 309, -1, -1, -1, -1], "input_ids")
    bt = np.array([[0, 1, 2], [3, -1, 9], [4, 5, 6], [7, -1, -1], [2, 2, 2], [1, 1, 1]], np.int32)
    sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                     prep["seq_lens"], prep["positions"], bt, bs, NB, lib=lib)
    # token 0: row 4, position -1 -> POS_OOR; token 1: row 9 -> BAD_ROW;
    # tokens 2,3: row 1 positions 2,3 -> block 3 -> slots 14, 15;
    # token 4: row 3 position 9 -> logic block 2 -> block -1 -> BLOCK_OOR;
    # tokens 5,6: positions 10, 11 -> logic block 2 -> BLOCK_OOR; tokens 7, 8: no request
    _eq(sm["slot_mapping"], [-1, -1, 14, 15, -1, -1, -1, -1, -1], "slot_mapping")
    assert sm["status"] == (oracle.ST_BAD_ROW | oracle.ST_POS_OOR | oracle.ST_BLOCK_OOR), sm["status"]
    # visible blocks: row 2 seq 3 -> 1: [4]; row 4 seq 0 -> none; row 9 skipped;
    # row 1 seq 4 -> 1: [3]; row 3 seq 12 -> 3: [7, -1, -1] (BLOCK_OOR)
    U = oracle.IBT_UNWRITTEN
    _eq(sm["input_block_tables"], [[4, U, U], [U, U, U], [U, U, U], [3, U, U], [7, -1, -1]], "ibt")
    # logic block beyond the table and seq_len beyond MB*bs
    sm2 = oracle.compute_slot_mapping(np.array([2], np.int32), np.array([0, 1], np.int32),
                                      np.array([13], np.int32), np.array([12], np.int32),
                                      bt, bs, NB, lib=lib)
    _eq(sm2["slot_mapping"], [-1], "lb >= MB")
    assert sm2["status"] == oracle.ST_LB_OOR
    _eq(sm2["input_block_tables"], [[4, 5, 6]], "ibt cut to MB")
    # scatter: slot beyond the cache is flagged and skipped, negative slot skipped silently
    k = np.arange(4 * 8, dtype=np.uint16).reshape(4, 8)
    v = k + 1000
    kc = np.zeros((5, 8), np.uint16)
    vc = np.zeros((5, 8), np.uint16)
    rc, st = oracle.scatter_kv(k, v, kc, vc, np.array([4, -1, 5, 0], np.int32), lib=lib)
    assert rc == 0 and st == oracle.ST_SLOT_OOR
    _eq(kc[4], k[0], "k slot 4")
    _eq(kc[0], k[3], "k slot 0")
    _eq(vc[0], v[3], "v slot 0")
    assert not kc[1:4].any() and not vc[1:4].any()
    # without a token table the width L bounds nothing: only negative positions flag
    p3 = oracle.prepare_batch(np.array([3], np.int32), np.array([3], np.int32), completed, tok,
                              T=3, lib=lib, with_input_ids=False)
    assert p3["status"] == 0, p3["status"]
    _eq(p3["positions"], [9, 10, 11], "positions without input_ids")
    # argument errors
    assert oracle.prepare_batch(rows, counts, completed, tok, T=-1, lib=lib)["rc"] == oracle.EINVAL
    assert oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                       prep["seq_lens"], prep["positions"], bt, 0, NB,
                                       lib=lib)["rc"] == oracle.EINVAL


def pin_strided_kv(lib):
    """K/V as strided views of a wider per-token buffer (e.g. a fused QKV output)."""
    rng = np.random.default_rng(5)
    T, H, D = 7, 2, 8
    qkv = rng.integers(0, 65535, size=(T, 3, H, D), dtype=np.uint16)
    k, v = qkv[:, 1], qkv[:, 2]
    slots = np.array([3, 0, 9, 4, 7, 1, 2], np.int32)
    kc = np.zeros((10, H, D), np.uint16)
    vc = np.zeros((10, H, D), np.uint16)
    rc, st = oracle.scatter_kv(k, v, kc, vc, slots, lib=lib)
    assert rc == 0 and st == 0
    _eq(kc[slots], k, "strided K")
    _eq(vc[slots], v, "strided V")


ALL_PINS = [pin_pages_example, pin_prefix_example, pin_budget_tie_example, pin_bruteforce,
            pin_library_routines, pin_closed_forms, pin_invariants, pin_error_semantics,
            pin_strided_kv]


# ---------------------------------------------------------------------------
# paged K/V read (the gather through visible pages)
# ---------------------------------------------------------------------------

def pin_gather_pages_example(lib):
    """Reading back the kongchang.com example after its step: B's history runs
    0..31 over blocks 37 and 12, so its row 31 is slot 207, the token just
    written; A's rows 16..23 are slots 704..711.  kv_start = [0, 32, 56]."""
    g = _golden("pages_example.json")
    b = workloads.pages_example()
    prep, groups = oracle.run_chain(b, lib=lib)
    gr = groups[0]
    out = oracle.gather_kv(prep["seq_lens"], gr["input_block_tables"], 16, b.groups[0].num_blocks,
                           gr["k_cache"], gr["v_cache"], lib=lib)
    assert out["rc"] == 0 and out["status"] == 0
    sl = g["derived"]["seq_lens"]
    _eq(out["kv_start"], [0, sl[0], sl[0] + sl[1]], "kv_start")
    k, v = b.groups[0].k, b.groups[0].v
    _eq(out["k"][31], k[0], "B's row 31")
    _eq(out["v"][31], v[0], "B's row 31 (V)")
    _eq(out["k"][32 + 16:32 + 24], k[1:9], "A's rows 16..23")
    _eq(out["v"][32 + 16:32 + 24], v[1:9], "A's rows 16..23 (V)")
    # everything else is history the step did not write: still the sentinel
    assert int(np.any(out["k"] != 0xFFFF, axis=(1, 2)).sum()) == 9


def pin_gather_inverse_of_scatter(lib, names=("seeded_16req", "seeded_16req_decode50")):
    """Invariant: after a step, reading request b's positions completed ..
    seq_len-1 gives back exactly the K/V rows of its tokens this step."""
    for name in names:
        b = workloads.make(name)
        prep, groups = oracle.run_chain(b, lib=lib)
        for g, gr in zip(b.groups, groups):
            out = oracle.gather_kv(prep["seq_lens"], gr["input_block_tables"], g.block_size,
                                   g.num_blocks, gr["k_cache"], gr["v_cache"], lib=lib)
            assert out["rc"] == 0 and out["status"] == 0
            qsl, ks = prep["query_start_loc"], out["kv_start"]
            for bi in range(b.n):
                cnt = int(qsl[bi + 1] - qsl[bi])
                end = int(ks[bi + 1])
                _eq(out["k"][end - cnt:end], g.k[qsl[bi]:qsl[bi + 1]], f"{name} K of request {bi}")
                _eq(out["v"][end - cnt:end], g.v[qsl[bi]:qsl[bi + 1]], f"{name} V of request {bi}")


def pin_gather_bruteforce(lib, seeds=range(150)):
    """Random caches and visible pages (bad pages included): every output row
    equals the cache row at the slot found by enumerating the request's
    address space, by NumPy fancy indexing; unreadable rows keep the fill."""
    for seed in seeds:
        rng = np.random.default_rng(1300 + seed)
        n = int(rng.integers(0, 7))
        bs = int(rng.choice([1, 2, 3, 4, 16]))
        MB = int(rng.integers(1, 6))
        NB = int(rng.integers(1, 12))
        sl = rng.integers(0, MB * bs + 1, n).astype(np.int32)
        ibt = rng.integers(0, NB, (n, MB)).astype(np.int32)
        if n and seed % 4 == 3:
            ibt[rng.integers(n), rng.integers(MB)] = int(rng.choice([-1, NB, NB + 3]))
        kc = rng.integers(0, 1 << 16, (NB * bs, 2, 3)).astype(np.uint16)
        vc = rng.integers(0, 1 << 16, (NB * bs, 2, 3)).astype(np.uint16)
        out = oracle.gather_kv(sl, ibt, bs, NB, kc, vc, lib=lib)
        slots = np.asarray(brute_gather_slots(sl.tolist(), ibt.tolist(), bs), np.int64)
        slots[(slots < 0) | (slots >= NB * bs)] = -1
        good = slots >= 0
        assert out["rc"] == 0
        _eq(out["k"][good], kc[slots[good]], f"seed {seed} K")
        _eq(out["v"][good], vc[slots[good]], f"seed {seed} V")
        assert np.all(out["k"][~good] == 0xFFFF), f"seed {seed} unread rows"
        want = oracle.ST_BLOCK_OOR if (~good).any() else 0
        assert out["status"] == want, (seed, out["status"])
        _eq(out["kv_start"], np.concatenate([[0], np.cumsum(sl)]), f"seed {seed} kv_start")


def pin_gather_closed_forms(lib):
    """Contiguous pages (page i of request b is block b*MB + i): each request's
    rows are one contiguous slice of the cache.  Block size 1: row p is the
    cache row named by page p."""
    rng = np.random.default_rng(91)
    n, MB, bs = 5, 4, 8
    kc = rng.integers(0, 1 << 16, (n * MB * bs, 4)).astype(np.uint16)
    sl = np.array([0, 1, 8, 9, 32], np.int32)
    ibt = (np.arange(n)[:, None] * MB + np.arange(MB)[None, :]).astype(np.int32)
    out = oracle.gather_kv(sl, ibt, bs, n * MB, kc, kc, lib=lib)
    ks = out["kv_start"]
    for b_ in range(n):
        base = b_ * MB * bs
        _eq(out["k"][ks[b_]:ks[b_ + 1]], kc[base:base + sl[b_]], f"contiguous request {b_}")
    ibt1 = rng.permutation(40)[:24].reshape(3, 8).astype(np.int32)
    kc1 = rng.integers(0, 1 << 16, (40, 2)).astype(np.uint16)
    sl1 = np.array([8, 3, 5], np.int32)
    out = oracle.gather_kv(sl1, ibt1, 1, 40, kc1, kc1, lib=lib)
    want = np.concatenate([kc1[ibt1[i, :sl1[i]]] for i in range(3)])
    _eq(out["k"], want, "block size 1")


def pin_gather_errors(lib):
    """R15: negative seq_len (0 rows, BAD_COUNT), a position past MB pages
    (LB_OOR), a bad page (BLOCK_OOR), an output too small (TOKEN_SUM)."""
    kc = np.arange(40, dtype=np.uint16).reshape(20, 2)
    ibt = np.array([[0, 1], [2, 9], [3, 4]], np.int32)      # block 9 is outside 5 blocks
    out = oracle.gather_kv([-3, 9, 5], ibt, 4, 5, kc, kc, out_tokens=14, lib=lib)
    assert out["rc"] == 0
    assert out["status"] == (oracle.ST_BAD_COUNT | oracle.ST_BLOCK_OOR | oracle.ST_LB_OOR), \
        hex(out["status"])
    _eq(out["kv_start"], [0, 0, 9, 14], "kv_start")
    _eq(out["k"][0:4], kc[8:12], "request 1, page 0 (block 2)")
    assert np.all(out["k"][4:9] == 0xFFFF), "bad page and past-MB rows unread"
    _eq(out["k"][9:13], kc[12:16], "request 2, page 0 (block 3)")
    _eq(out["k"][13], kc[16], "request 2, page 1, first slot")
    out = oracle.gather_kv([-3, 9, 5], ibt, 4, 5, kc, kc, out_tokens=13, lib=lib)
    assert out["status"] & oracle.ST_TOKEN_SUM
    _eq(out["kv_start"], [0, 0, 9, 14], "kv_start past the output")
    _eq(out["k"][9:13], kc[12:16], "rows before the cut")
    out = oracle.gather_kv([4, 4], ibt[:2], 4, 5, kc, kc, out_tokens=6, lib=lib)
    assert out["status"] == oracle.ST_TOKEN_SUM
    _eq(out["k"][4:6], kc[8:10], "cut at out_tokens")


GATHER_PINS = [pin_gather_pages_example, pin_gather_inverse_of_scatter, pin_gather_bruteforce,
               pin_gather_closed_forms, pin_gather_errors]
ALL_PINS += GATHER_PINS


# ---------------------------------------------------------------------------
# persistent request state: add_request, update_request, the after-step advance
# ---------------------------------------------------------------------------

def pin_state_pages_example(lib):
    """Rebuild the kongchang.com example's state from nothing with add_request
    (rows 7 and 6, 31 and 16 tokens done, blocks [37, 12] and [81, 44]); the
    chain on it then gives the printed values."""
    g = _golden("pages_example.json")
    ref = workloads.pages_example()
    R, L, MB = ref.R, ref.L, ref.groups[0].max_blocks
    st = oracle.empty_state(R, L, MB)
    rows = [7, 6]
    prompts = [ref.token_ids[7, :32].tolist(), ref.token_ids[6, :24].tolist()]
    rc, status = oracle.add_requests(st, rows, [31, 16], prompts, [[37, 12], [81, 44]], lib=lib)
    assert rc == 0 and status == 0
    _eq(st["completed"], ref.completed, "completed")
    _eq(st["block_table"], ref.groups[0].block_table, "block_table")
    _eq(st["row_blocks"][[7, 6]], [2, 2], "row_blocks")
    _eq(st["token_ids"][7, :32], ref.token_ids[7, :32], "tokens of B")
    _eq(st["token_ids"][6, :24], ref.token_ids[6, :24], "tokens of A")
    prep = oracle.prepare_batch(ref.sched_rows, ref.num_scheduled, st["completed"],
                                st["token_ids"], lib=lib)
    sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                     prep["seq_lens"], prep["positions"], st["block_table"], 16,
                                     ref.groups[0].num_blocks, lib=lib)
    _eq(prep["query_start_loc"], g["printed"]["query_start_loc"], "query_start_loc")
    _eq(sm["slot_mapping"], g["derived"]["slot_mapping"], "slot_mapping")
    # after the step both requests have computed their scheduled tokens
    rc, status = oracle.advance_state(st, prep["index_mapping"], prep["seq_lens"], lib=lib)
    _eq(st["completed"][[7, 6]], g["derived"]["seq_lens"], "completed after the step")


def pin_state_prefix_example(lib):
    """The caffein.top example: B reuses cached P1, P2 (8 tokens computed),
    then B3 is newly allocated and appended: the table reads [P1][P2][B3]."""
    g = _golden("prefix_reuse_example.json")
    inst = g["inputs"]["instantiate"]
    st = oracle.empty_state(4, 12, 3)
    prompt = (np.arange(10) + 12).tolist()                # identity code of row 1
    rc, status = oracle.add_requests(st, [1], [8], [prompt], [[inst["P1"], inst["P2"]]], lib=lib)
    assert rc == 0 and status == 0
    _eq(st["block_table"][1], [inst["P1"], inst["P2"], -1], "after reuse")
    _eq(st["row_blocks"][1], 2, "row_blocks after reuse")
    rc, status = oracle.append_blocks(st, [1], [[inst["B3"]]], lib=lib)
    assert rc == 0 and status == 0
    _eq(st["block_table"][1], [inst["P1"], inst["P2"], inst["B3"]], "[P1][P2][B3]")
    _eq(st["row_blocks"][1], 3, "row_blocks after append")
    prep = oracle.prepare_batch([1], [2], st["completed"], st["token_ids"], lib=lib)
    sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                     prep["seq_lens"], prep["positions"], st["block_table"], 4, 16,
                                     lib=lib)
    e = g["expected"]
    _eq(prep["positions"], e["positions"], "positions")
    _eq(sm["slot_mapping"], [4 * inst["B3"], 4 * inst["B3"] + 1], "slots")


class StateModel:
    """Pure-Python model of the state: per row a token list, a block list and a
    computed count (lists instead of arrays, no -1 padding)."""

    def __init__(self, R, L, MB):
        self.R, self.L, self.MB = R, L, MB
        self.tokens = {r: {} for r in range(R)}
        self.blocks = {r: [] for r in range(R)}
        self.done = {r: 0 for r in range(R)}

    def add(self, r, done, prompt, blocks):
        self.done[r] = done
        for p, t in enumerate(prompt[:self.L]):
            self.tokens[r][p] = t
        self.blocks[r] = list(blocks[:self.MB])

    def append(self, r, blocks):
        self.blocks[r] = (self.blocks[r] + list(blocks))[:self.MB]

    def advance(self, r, seq_len, sampled):
        self.done[r] = seq_len
        if sampled is not None and sampled >= 0 and 0 <= seq_len < self.L:
            self.tokens[r][seq_len] = sampled

    def check(self, st, token_fill=-1):
        for r in range(self.R):
            assert st["completed"][r] == self.done[r], (r, "completed")
            row = [-1] * self.MB
            row[:len(self.blocks[r])] = self.blocks[r]
            assert st["block_table"][r].tolist() == row, (r, "block_table")
            assert st["row_blocks"][r] == len(self.blocks[r]), (r, "row_blocks")
            want = [self.tokens[r].get(p, token_fill) for p in range(self.L)]
            assert st["token_ids"][r].tolist() == want, (r, "token_ids")


def pin_state_bruteforce(lib, seeds=range(60)):
    """Random sequences of add / append / advance against the Python model."""
    for seed in seeds:
        rng = np.random.default_rng(500 + seed)
        R, L, MB = 6, 12, 4
        st = oracle.empty_state(R, L, MB)
        model = StateModel(R, L, MB)
        for _ in range(8):
            op = rng.integers(3)
            rows = rng.choice(R, int(rng.integers(1, 4)), replace=False).tolist()
            if op == 0:
                done = rng.integers(0, 8, len(rows)).tolist()
                prompts = [rng.integers(0, 1000, int(rng.integers(0, 14))).tolist() for _ in rows]
                blocks = [rng.integers(0, 50, int(rng.integers(0, 6))).tolist() for _ in rows]
                oracle.add_requests(st, rows, done, prompts, blocks, lib=lib)
                for r, d, p, b in zip(rows, done, prompts, blocks):
                    model.add(r, d, p, b)
            elif op == 1:
                blocks = [rng.integers(0, 50, int(rng.integers(0, 3))).tolist() for _ in rows]
                oracle.append_blocks(st, rows, blocks, lib=lib)
                for r, b in zip(rows, blocks):
                    model.append(r, b)
            else:
                seq = rng.integers(0, 14, len(rows)).tolist()
                sampled = rng.integers(-1, 1000, len(rows)).tolist()
                oracle.advance_state(st, rows, seq, sampled, lib=lib)
                for r, q, s in zip(rows, seq, sampled):
                    model.advance(r, q, s)
            model.check(st)


def pin_state_multistep(lib, steps=24):
    """A decode loop closed on the state: each step appends a block to rows
    whose next token starts a new one, runs the chain, and advances the state
    with a sampled token; positions then walk on by one per step."""
    rng = np.random.default_rng(77)
    R, L, MB, bs, NB = 10, 64, 16, 4, 200
    st = oracle.empty_state(R, L, MB)
    model = StateModel(R, L, MB)
    pool = rng.permutation(NB).tolist()
    rows = rng.choice(R, 6, replace=False).tolist()
    prompts = [rng.integers(0, 1000, int(rng.integers(1, 9))).tolist() for _ in rows]
    blocks = [[pool.pop() for _ in range(-(-len(p) // bs))] for p in prompts]
    oracle.add_requests(st, rows, [0] * len(rows), prompts, blocks, lib=lib)
    for r, p, b in zip(rows, prompts, blocks):
        model.add(r, 0, p, b)
    counts = [len(p) for p in prompts]                    # first step: the whole prompt
    seen = set()
    for step in range(steps):
        need = []
        for r, c in zip(rows, counts):
            have = int(st["row_blocks"][r])
            want = -(-(int(st["completed"][r]) + c) // bs)
            need.append([pool.pop() for _ in range(max(0, want - have))])
        oracle.append_blocks(st, rows, need, lib=lib)
        for r, b in zip(rows, need):
            model.append(r, b)
        prep = oracle.prepare_batch(rows, counts, st["completed"], st["token_ids"], lib=lib)
        assert prep["status"] == 0
        sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                         prep["seq_lens"], prep["positions"], st["block_table"],
                                         bs, NB, lib=lib)
        assert sm["status"] == 0 and (sm["slot_mapping"] >= 0).all()
        for s in sm["slot_mapping"].tolist():
            assert s not in seen, "a slot is written twice across steps"
            seen.add(s)
        # every scheduled position holds a known token (prompt or sampled)
        for b_, r in enumerate(prep["index_mapping"].tolist()):
            for t in range(prep["query_start_loc"][b_], prep["query_start_loc"][b_ + 1]):
                assert prep["input_ids"][t] == model.tokens[r][prep["positions"][t]]
        sampled = rng.integers(0, 1000, len(rows)).tolist()
        oracle.advance_state(st, prep["index_mapping"], prep["seq_lens"], sampled, lib=lib)
        for r, q, s_ in zip(prep["index_mapping"].tolist(), prep["seq_lens"].tolist(), sampled):
            model.advance(r, q, s_)
        model.check(st)
        counts = [1] * len(rows)


def pin_state_errors(lib):
    st = oracle.empty_state(3, 4, 2)
    rc, status = oracle.add_requests(st, [5, 1], [0, 2], [[1], [9, 8, 7, 6, 5, 4]],
                                     [[1], [3, 4, 5]], lib=lib)
    assert rc == 0 and status == (oracle.ST_BAD_ROW | oracle.ST_POS_OOR | oracle.ST_LB_OOR), status
    _eq(st["token_ids"][1], [9, 8, 7, 6], "prompt cut at L")
    _eq(st["block_table"][1], [3, 4], "blocks cut at MB")
    _eq(st["row_blocks"][1], 2, "row_blocks cut at MB")
    rc, status = oracle.append_blocks(st, [1, -1], [[7], [8]], lib=lib)
    assert status == (oracle.ST_LB_OOR | oracle.ST_BAD_ROW), status
    _eq(st["block_table"][1], [3, 4], "full row unchanged")
    # CSR ranges outside the flat array: the request is skipped and flagged
    st2 = oracle.empty_state(3, 4, 2)
    rc, status = oracle.add_requests(
        st2, [0, 1], [1, 1], (np.array([0, 3, 9], np.int32), np.array([4, 5, 6, 7], np.int32), 4),
        (np.array([0, 1, 2], np.int32), np.array([8, 9], np.int32), 2), lib=lib)
    assert rc == 0 and status == oracle.ST_BAD_RANGE, status
    _eq(st2["completed"], [1, 0, 0], "second request skipped")
    _eq(st2["token_ids"][0, :3], [4, 5, 6], "first request's prompt")
    rc, status = oracle.append_blocks(st2, [0, 2], (np.array([0, 1, 0], np.int32),
                                                    np.array([7], np.int32), 1), lib=lib)
    assert status == oracle.ST_BAD_RANGE, status
    _eq(st2["block_table"][0], [8, 7], "first append kept")
    rc, status = oracle.advance_state(st, [1, 2, 7], [4, 1, 0], [5, -1, 3], lib=lib)
    assert status == (oracle.ST_POS_OOR | oracle.ST_BAD_ROW), status
    _eq(st["completed"], [0, 4, 1], "completed")
    _eq(st["token_ids"][2], [-1, -1, -1, -1], "no token for sampled -1")


def pin_pool_model(lib, seeds=range(40)):
    """The row pool against a Python list used as a stack (rows 0, 1, ... on
    top at the start; acquire pops, release pushes in order), with its
    all-or-nothing failures, on random sequences; plus the invariants: no row
    is handed out twice, and free plus handed-out rows make up every row."""
    for seed in seeds:
        rng = np.random.default_rng(700 + seed)
        R = int(rng.integers(0, 12))
        pool = oracle.RowPool(R, lib=lib)
        stack = list(range(R - 1, -1, -1))
        out = set()
        for _ in range(30):
            if rng.random() < 0.5:
                m = int(rng.integers(0, R + 3))
                rc, rows = pool.acquire(m)
                if m > len(stack):
                    assert rc == oracle.ENOROWS and rows == [], (seed, m)
                else:
                    want = [stack.pop() for _ in range(m)]
                    assert rc == 0 and rows == want, (seed, rows, want)
                    assert not (set(rows) & out), "row handed out twice"
                    out |= set(rows)
            else:
                cand = sorted(out) * 2 + list(range(R)) + [-1, R, R + 5]
                k = int(rng.integers(0, 4))
                rows = [int(x) for x in rng.choice(cand, k)] if k else []
                ok = len(set(rows)) == len(rows) and all(r in out for r in rows)
                rc = pool.release(rows)
                if ok:
                    assert rc == 0, (seed, rows)
                    stack.extend(rows)
                    out -= set(rows)
                else:
                    assert rc == oracle.EINVAL, (seed, rows)
            assert pool.free == len(stack) and pool.free + len(out) == R
            assert pool.free_rows[:pool.free].tolist() == stack
            assert sorted(np.flatnonzero(pool.in_use[:R]).tolist()) == sorted(out)


def pin_pool_recycles_into_state(lib):
    """A completed request's row goes back to the pool and the next request
    gets it; add_request then leaves nothing of the old request's blocks."""
    pool = oracle.RowPool(4, lib=lib)
    st = oracle.empty_state(4, 8, 3)
    rc, (a, b) = pool.acquire(2)
    assert (a, b) == (0, 1)
    oracle.add_requests(st, [a, b], [0, 0], [[1, 2, 3], [4]], [[5, 6, 7], [8]], lib=lib)
    assert pool.release([a]) == 0
    rc, (c,) = pool.acquire(1)
    assert c == a
    oracle.add_requests(st, [c], [0], [[9]], [[2]], lib=lib)
    _eq(st["block_table"][c], [2, -1, -1], "recycled row's blocks")
    _eq(st["row_blocks"][c], 1, "recycled row's block count")


STATE_PINS = [pin_state_pages_example, pin_state_prefix_example, pin_state_bruteforce,
              pin_state_multistep, pin_state_errors, pin_pool_model,
              pin_pool_recycles_into_state]
ALL_PINS += STATE_PINS


# ---------------------------------------------------------------------------
# prefix-cache block hashes and the prefix index
# ---------------------------------------------------------------------------

# FNV-1a 64-bit test vectors published with the FNV specification (Fowler,
# Noll, Vo; IETF draft-eastlake-fnv): the empty string, "a" and "foobar".
FNV1A64_VECTORS = [(b"", 0xcbf29ce484222325), (b"a", 0xaf63dc4c8601ec8c),
                   (b"foobar", 0x85944171f73967e8)]
FNV_PRIME64 = 1099511628211


def pin_fnv_vectors(lib):
    for data, want in FNV1A64_VECTORS:
        assert oracle.fnv1a64(data, lib=lib) == want, data


def pin_hash_closed_form(lib, seeds=range(30)):
    """The chain written as a sum: s_i = sum_j c_j * P^(i-j) (mod 2^64), with
    c_j the FNV-1a of block j's little-endian bytes and h_i the FNV-1a of s_i's
    8 little-endian bytes (0 -> 1); Python integers, not the oracle's loop."""
    for seed in seeds:
        rng = np.random.default_rng(1700 + seed)
        bs = int(rng.choice([1, 2, 4, 16, 32]))
        lists = [rng.integers(-2**31, 2**31, int(rng.integers(0, 7 * bs))).tolist()
                 for _ in range(int(rng.integers(1, 5)))]
        MB = 6
        out = oracle.hash_blocks(lists, bs, MB, lib=lib)
        assert out["rc"] == 0 and out["status"] == 0
        for b, toks in enumerate(lists):
            full = len(toks) // bs
            assert out["num_full"][b] == full
            c = [oracle.fnv1a64(struct.pack(f"<{bs}i", *toks[j * bs:(j + 1) * bs]), lib=lib)
                 for j in range(full)]
            for i in range(full):
                s_i = sum(c[j] * pow(FNV_PRIME64, i - j, 2**64) for j in range(i + 1)) % 2**64
                h = oracle.fnv1a64(struct.pack("<Q", s_i), lib=lib) or 1
                assert int(out["hashes"][b, i]) == h, (seed, b, i)
            assert np.all(out["hashes"][b, full:] == 0), "blocks past the full ones are not written"


def pin_hash_prefix_context(lib):
    """Equal prefixes give equal hashes; changing one token of block j changes
    the hashes of blocks j, j+1, ... and no earlier one; a partial last block
    is not hashed."""
    rng = np.random.default_rng(5)
    bs = 4
    base = rng.integers(0, 1000, 6 * bs).tolist()
    for j in range(6):
        for t in range(bs):
            other = list(base)
            other[j * bs + t] += 1
            out = oracle.hash_blocks([base, other, base[:-1]], bs, 6, lib=lib)
            h = out["hashes"]
            assert np.array_equal(h[0, :j], h[1, :j])
            assert np.all(h[0, j:] != h[1, j:]), (j, t)
            assert out["num_full"].tolist() == [6, 6, 5]
            assert np.array_equal(h[2, :5], h[0, :5])


def pin_prefix_cf_example(lib):
    """caffein.top: block size 4, A and B share an 8-token system prompt.  A's
    full blocks are registered (P1, P2, A's own third block); B (10 tokens)
    hashes its two full blocks, hits P1 and P2, and has 8 tokens computed."""
    g = _golden("prefix_reuse_example.json")
    inst = g["inputs"]["instantiate"]
    P1, P2 = inst["P1"], inst["P2"]
    system = [101, 102, 103, 104, 105, 106, 107, 108]
    a = system + [201, 202, 203, 204]
    b = system + [301, 302]
    ha = oracle.hash_blocks([a], 4, 3, lib=lib)["hashes"]
    hb = oracle.hash_blocks([b], 4, 3, lib=lib)
    assert hb["num_full"].tolist() == [2]
    idx = oracle.PrefixIndex(16, lib=lib)
    bt = np.array([[P1, P2, 40]], np.int32)
    rc, st = idx.insert(ha, [0], [3], [0], bt)
    assert rc == 0 and st == 0
    look = idx.lookup(hb["hashes"], [len(b)], 4)
    assert look["num_computed"].tolist() == [g["inputs"]["completed"]]      # 8 reused tokens
    _eq(look["hit_blocks"][0, :2], [P1, P2], "B reuses P1, P2")
    assert look["hit_blocks"][0, 2] == -7, "nothing written past the hit"


def pin_prefix_hit_cap(lib):
    """A hit never covers the last token: a prompt of exactly two cached full
    blocks (8 tokens, block size 4) hits one block; with a ninth token, two."""
    toks = list(range(9))
    h = oracle.hash_blocks([toks], 4, 3, lib=lib)["hashes"]
    idx = oracle.PrefixIndex(8, lib=lib)
    idx.insert(h, [0], [2], [0], np.array([[7, 9, -1]], np.int32))
    assert idx.lookup(h, [8], 4)["num_computed"].tolist() == [4]
    assert idx.lookup(h, [9], 4)["num_computed"].tolist() == [8]
    assert idx.lookup(h, [1], 4)["num_computed"].tolist() == [0]
    assert idx.lookup(h, [0], 4)["num_computed"].tolist() == [0]


class IndexModel:
    """Python dict model of the prefix index."""

    def __init__(self, capacity):
        self.capacity = capacity
        self.entries = {}                       # hash -> block or None

    def insert(self, key, block):
        if key == 0:
            return 0
        if key not in self.entries:
            if len(self.entries) == self.capacity:
                return oracle.ST_TABLE_FULL
            self.entries[key] = None
        cur = self.entries[key]
        self.entries[key] = block if cur is None else min(cur, block)
        return 0

    def evict(self, key, block):
        if self.entries.get(key, "absent") == block:
            self.entries[key] = None

    def lookup(self, hashes, length, bs):
        cap = (length - 1) // bs if length > 0 else 0
        out = []
        for i in range(min(cap, len(hashes))):
            blk = self.entries.get(int(hashes[i]))
            if blk is None:
                break
            out.append(blk)
        return out


def pin_prefix_model(lib, seeds=range(40)):
    """Random inserts, evictions and lookups against the dict model, with a
    small hash alphabet (many repeats) and a capacity that fills up."""
    for seed in seeds:
        rng = np.random.default_rng(2300 + seed)
        cap = int(rng.integers(1, 12))
        MB = 5
        alphabet = rng.integers(1, 2**63, 10).astype(np.uint64)
        idx, model = oracle.PrefixIndex(cap, lib=lib), IndexModel(cap)
        for _ in range(12):
            m = int(rng.integers(1, 4))
            hashes = alphabet[rng.integers(0, 10, (m, MB))]
            op = int(rng.integers(3))
            if op == 0:
                R = 4
                bt = rng.integers(-1, 30, (R, MB)).astype(np.int32)
                rows = rng.choice(R, m, replace=False)
                lo = rng.integers(0, MB + 1, m)
                hi = np.minimum(lo + rng.integers(0, 4, m), MB)
                rc, st = idx.insert(hashes, lo, hi, rows, bt)
                want = 0
                for b in range(m):
                    for i in range(lo[b], hi[b]):
                        blk = int(bt[rows[b], i])
                        if blk < 0:
                            want |= oracle.ST_BLOCK_OOR
                            continue
                        want |= model.insert(int(hashes[b, i]), blk)
                assert rc == 0 and st == want, (seed, st, want)
            elif op == 1:
                blocks = rng.integers(0, 30, m * MB)
                idx.evict(hashes.reshape(-1), blocks)
                for k, blk in zip(hashes.reshape(-1).tolist(), blocks.tolist()):
                    model.evict(int(k), int(blk))
            else:
                lens = rng.integers(0, MB * 4 + 3, m)
                look = idx.lookup(hashes, lens, 4)
                for b in range(m):
                    want = model.lookup(hashes[b], int(lens[b]), 4)
                    assert look["num_computed"][b] == 4 * len(want), (seed, b)
                    _eq(look["hit_blocks"][b, :len(want)], want, f"seed {seed} hits")
            assert idx.live() == {k: v for k, v in model.entries.items() if v is not None}
            assert idx.known() == set(model.entries)


PREFIX_PINS = [pin_fnv_vectors, pin_hash_closed_form, pin_hash_prefix_context,
               pin_prefix_cf_example, pin_prefix_hit_cap, pin_prefix_model]
ALL_PINS += PREFIX_PINS


# ---------------------------------------------------------------------------
# sliding-window holes and speculative lookahead
# ---------------------------------------------------------------------------

def _needed_positions(prep, bi, W):
    """Brute force: every position some new token of batch row bi attends with
    window W (token at p attends p-W+1 .. p), as a sorted list."""
    need = set()
    for t in range(int(prep["query_start_loc"][bi]), int(prep["query_start_loc"][bi + 1])):
        p = int(prep["positions"][t])
        need.update(q for q in range(p - W + 1, p + 1) if q >= 0)
    return sorted(need)


def pin_window_bruteforce(lib, seeds=range(80)):
    """Sliding windows on tiny random batches: the blocks window_free releases
    are exactly those wholly before every position the step's tokens attend
    (found by enumeration, no division); after freeing, the visible pages copy
    the holes unflagged while full attention flags them; the windowed read
    returns exactly the attended positions, request after request."""
    for seed in seeds:
        b = workloads.random_tiny(seed)
        g = b.groups[0]
        bs = g.block_size
        W = int(np.random.default_rng(seed).integers(1, 3 * bs + 5))
        bt = g.block_table.copy()
        fr = oracle.window_free(b.sched_rows, b.completed, bt, bs, W, lib=lib)
        assert fr["rc"] == 0 and fr["status"] == 0
        prep = oracle.prepare_batch(b.sched_rows, b.num_scheduled, b.completed, b.token_ids, lib=lib)
        order = prep["index_mapping"].tolist()
        for i, r in enumerate(b.sched_rows.tolist()):
            bi = order.index(r)
            need = _needed_positions(prep, bi, W)
            first_need = need[0] if need else int(b.completed[r])
            # wholly before: every slot position of the block is below first_need
            gone = [blk for blk_i, blk in enumerate(g.block_table[r])
                    if blk >= 0 and all(blk_i * bs + o < first_need for o in range(bs))
                    and int(b.completed[r]) - W + 1 > 0]
            _eq(fr["freed"][i, :fr["num_freed"][i]], gone, f"seed {seed} freed of row {r}")
            for blk_i in range(g.max_blocks):
                want = -1 if g.block_table[r, blk_i] in gone and g.block_table[r, blk_i] >= 0 \
                    and all(blk_i * bs + o < first_need for o in range(bs)) else g.block_table[r, blk_i]
                assert bt[r, blk_i] == want, (seed, r, blk_i)
        full = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                           prep["seq_lens"], prep["positions"], bt, bs,
                                           g.num_blocks, lib=lib)
        win = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                          prep["seq_lens"], prep["positions"], bt, bs,
                                          g.num_blocks, sliding_window=W, lib=lib)
        _eq(win["slot_mapping"], full["slot_mapping"], f"seed {seed} slots")
        _eq(win["input_block_tables"], full["input_block_tables"], f"seed {seed} pages")
        assert win["status"] == 0, (seed, win["status"])
        holes_visible = any(
            (full["input_block_tables"][bi, :-(-int(prep["seq_lens"][bi]) // bs)] == -1).any()
            for bi in range(b.n))
        assert bool(full["status"] & oracle.ST_BLOCK_OOR) == holes_visible, seed
        # the windowed read: exactly the attended positions, from a patterned cache
        kc = (np.arange(g.num_slots * 2, dtype=np.uint32) * 2654435761 >> 16).astype(np.uint16)
        kc = kc.reshape(g.num_slots, 2, 1)
        out = oracle.gather_kv(prep["seq_lens"], win["input_block_tables"], bs, g.num_blocks, kc, kc,
                               query_start_loc=prep["query_start_loc"], sliding_window=W, lib=lib)
        assert out["rc"] == 0 and out["status"] == 0, (seed, out["status"])
        rows_want = []
        for bi in range(b.n):
            need = _needed_positions(prep, bi, W)
            assert out["kv_start"][bi + 1] - out["kv_start"][bi] == len(need)
            r = int(prep["index_mapping"][bi])
            for p in need:
                space = [int(x) * bs + o for x in g.block_table[r] for o in range(bs)]
                rows_want.append(kc[space[p]])
        if rows_want:
            _eq(out["k"], np.stack(rows_want), f"seed {seed} windowed read")


def pin_window_zero_is_full_attention(lib):
    """W = 0 frees nothing and reads every position, as without a window."""
    b = workloads.make("seeded_16req")
    g = b.groups[0]
    bt = g.block_table.copy()
    fr = oracle.window_free(b.sched_rows, b.completed, bt, g.block_size, 0, lib=lib)
    assert fr["num_freed"].sum() == 0 and np.array_equal(bt, g.block_table)
    prep, groups = oracle.run_chain(b, lib=lib)
    a = oracle.gather_kv(prep["seq_lens"], groups[0]["input_block_tables"], g.block_size,
                         g.num_blocks, groups[0]["k_cache"], groups[0]["v_cache"], lib=lib)
    w = oracle.gather_kv(prep["seq_lens"], groups[0]["input_block_tables"], g.block_size,
                         g.num_blocks, groups[0]["k_cache"], groups[0]["v_cache"],
                         query_start_loc=prep["query_start_loc"], sliding_window=0, lib=lib)
    _eq(a["k"], w["k"], "W=0 read")


def pin_lookahead(lib, seeds=range(60)):
    """The lookahead slots of a step are the slots the next step would write
    with k new tokens per request (the oracle's slot mapping of that step),
    and by enumeration of each request's address space."""
    for seed in seeds:
        b = workloads.random_tiny(seed)
        g = b.groups[0]
        k = int(np.random.default_rng(seed).integers(0, 5))
        prep = oracle.prepare_batch(b.sched_rows, b.num_scheduled, b.completed, b.token_ids, lib=lib)
        la = oracle.lookahead_slots(prep["index_mapping"], prep["seq_lens"], g.block_table,
                                    g.block_size, g.num_blocks, k, lib=lib)
        assert la["rc"] == 0
        # the following step: completed = seq_len, k tokens each
        comp2 = b.completed.copy()
        comp2[prep["index_mapping"]] = prep["seq_lens"]
        nxt = oracle.prepare_batch(prep["index_mapping"], np.full(b.n, k, np.int32), comp2,
                                   np.zeros((b.R, 0), np.int32), with_input_ids=False, lib=lib)
        sm = oracle.compute_slot_mapping(nxt["index_mapping"], nxt["query_start_loc"],
                                         nxt["seq_lens"], nxt["positions"], g.block_table,
                                         g.block_size, g.num_blocks, with_ibt=False, lib=lib)
        assert la["status"] == sm["status"], (seed, la["status"], sm["status"])
        # the next step orders its batch by row (equal counts): map back
        nxt_rows = nxt["index_mapping"].tolist()
        for bi, r in enumerate(prep["index_mapping"].tolist()):
            j = nxt_rows.index(r)
            q0 = int(nxt["query_start_loc"][j])
            _eq(la["slots"][bi], sm["slot_mapping"][q0:q0 + k], f"seed {seed} row {r}")
            space = [(-1 if x < 0 or x >= g.num_blocks else int(x) * g.block_size + o)
                     for x in g.block_table[r] for o in range(g.block_size)]
            s0 = int(prep["seq_lens"][bi])
            want = [space[p] if p < len(space) else -1 for p in range(s0, s0 + k)]
            _eq(la["slots"][bi], want, f"seed {seed} row {r} by enumeration")


def pin_blocks_needed(lib, seeds=range(60)):
    """caffein.top: B has 8 tokens computed (P1, P2 reused), 2 new, block size
    4 and two blocks: only B3 is new (one block).  Random cases against a count
    of the distinct blocks the positions 0 .. completed+new+k-1 touch."""
    r = oracle.blocks_needed([1], [2], 0, 4, [0, 8], [0, 2], lib=lib)
    assert r["need"].tolist() == [1] and r["status"] == 0
    for seed in seeds:
        rng = np.random.default_rng(900 + seed)
        R, n = 10, int(rng.integers(1, 8))
        rows = rng.choice(R, n, replace=False)
        comp = rng.integers(0, 60, R).astype(np.int32)
        rb = rng.integers(0, 20, R).astype(np.int32)
        new = rng.integers(0, 30, n).astype(np.int32)
        k, bs = int(rng.integers(0, 6)), int(rng.choice([1, 3, 4, 16]))
        got = oracle.blocks_needed(rows, new, k, bs, comp, rb, lib=lib)
        for i, r_ in enumerate(rows):
            touched = {p // bs for p in range(int(comp[r_] + new[i] + k))}
            assert got["need"][i] == max(0, len(touched) - int(rb[r_])), (seed, i)


NEXT4_PINS = [pin_window_bruteforce, pin_window_zero_is_full_attention, pin_lookahead,
              pin_blocks_needed]
ALL_PINS += NEXT4_PINS
