"""CPU oracle of the paged-KV input path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (``paged_kv_input_amd``)
never does, and the two share no code.  The arithmetic lives in ``oracle.c``
(plain C, one thread); this module compiles it with gcc and marshals NumPy
arrays through ctypes.

Sources: "Deep Dive into vLLM's Scheduling Mechanism: The Complete CPU-to-GPU
Mapping Pipeline" (kongchang.com/en, with its Chinese original) for the whole
chain, and "从源码读 vLLM Scheduler" (caffein.top) for the scheduler examples.
Every function is pinned by CPU tests (worked examples, brute force, library
routines, closed forms, invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# Contract values, restated (not shared) from the library's public header.
OK = 0
EINVAL = -1
ENOROWS = -5
ST_BAD_ROW, ST_BAD_COUNT, ST_TOKEN_SUM, ST_POS_OOR = 0x01, 0x02, 0x04, 0x08
ST_LB_OOR, ST_BLOCK_OOR, ST_SLOT_OOR, ST_BAD_RANGE = 0x10, 0x20, 0x40, 0x80
ST_TABLE_FULL = 0x100
NO_BLOCK = 2**31 - 1          # prefix index: an entry without a block

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def build(src: str = _SRC, out: str = _LIB, extra_flags=(), strict: bool = True) -> str:
    """Compile the oracle with gcc into a shared library (always rebuilds)."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", *(["-Werror"] if strict else []),
           "-fPIC", "-shared", *extra_flags, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.orc_prepare_batch.restype = ctypes.c_int
    lib.orc_prepare_batch.argtypes = [_I32, _I32, _P, _P, _P, _I32, _P, _I64, _I32,
                                      _P, _P, _P, _P, _P, _P]
    lib.orc_compute_slot_mapping.restype = ctypes.c_int
    lib.orc_compute_slot_mapping.argtypes = [_I32, _I32, _P, _P, _P, _P, _P, _I32, _I32,
                                             _I32, _I32, _I32, _P, _P, _P]
    lib.orc_scatter_kv.restype = ctypes.c_int
    lib.orc_scatter_kv.argtypes = [_I32, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _P]
    lib.orc_add_requests.restype = ctypes.c_int
    lib.orc_add_requests.argtypes = [_I32, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _P, _P,
                                     _I64, _I32, _P, _I32, _P, _P]
    lib.orc_append_blocks.restype = ctypes.c_int
    lib.orc_append_blocks.argtypes = [_I32, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P]
    lib.orc_advance_state.restype = ctypes.c_int
    lib.orc_advance_state.argtypes = [_I32, _P, _P, _P, _I32, _P, _P, _I64, _I32, _P]
    lib.orc_gather_kv.restype = ctypes.c_int
    lib.orc_gather_kv.argtypes = [_I32, _P, _P, _I32, _P, _I32, _I32, _I32, _I64, _P, _P, _I64,
                                  _P, _I64, _P, _I64, _P, _P]
    lib.orc_window_free.restype = ctypes.c_int
    lib.orc_window_free.argtypes = [_I32, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P]
    lib.orc_lookahead_slots.restype = ctypes.c_int
    lib.orc_lookahead_slots.argtypes = [_I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P]
    lib.orc_blocks_needed.restype = ctypes.c_int
    lib.orc_blocks_needed.argtypes = [_I32, _P, _P, _I32, _I32, _P, _P, _I32, _P, _P]
    lib.orc_fnv1a64.restype = ctypes.c_uint64
    lib.orc_fnv1a64.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
    lib.orc_hash_blocks.restype = ctypes.c_int
    lib.orc_hash_blocks.argtypes = [_I32, _P, _I64, _P, _P, _I32, _I32, _P, _P, _P]
    lib.orc_prefix_lookup.restype = ctypes.c_int
    lib.orc_prefix_lookup.argtypes = [_I32, _P, _I32, _P, _I32, _P, _P, _I64, _P, _P, _P]
    lib.orc_prefix_insert.restype = ctypes.c_int
    lib.orc_prefix_insert.argtypes = [_I32, _P, _I32, _P, _P, _P, _P, _I32, _P, _P, _I64, _P]
    lib.orc_prefix_evict.restype = ctypes.c_int
    lib.orc_prefix_evict.argtypes = [_I32, _P, _P, _P, _P, _I64]
    for name in ("orc_pool_acquire", "orc_pool_release"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [_I32, _P, _P, _P, _I32, _P]
    lib.orc_pool_reset.restype = ctypes.c_int
    lib.orc_pool_reset.argtypes = [_I32, _P, _P, _P]
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library, compiling it first if it is missing or stale."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def prepare_batch(sched_rows, num_scheduled, completed, token_ids, T=None, *, lib=None,
                  with_input_ids=True):
    """Oracle of ``prepare_batch``.  Returns a dict of NumPy outputs plus
    ``status`` (OR of status bits) and ``rc`` (return code)."""
    lib = lib or load()
    rows, counts, comp = _i32(sched_rows), _i32(num_scheduled), _i32(completed)
    tok = _i32(token_ids)
    n = rows.shape[0]
    if T is None:
        T = int(np.maximum(counts.astype(np.int64), 0).sum())
    R = comp.shape[0]
    L = tok.shape[1] if tok.ndim == 2 else 0
    out = {
        "index_mapping": np.full(n, -7, np.int32),
        "query_start_loc": np.full(n + 1, -7, np.int32),
        "seq_lens": np.full(n, -7, np.int32),
        "positions": np.full(max(T, 0), -7, np.int32),
        "input_ids": np.full(max(T, 0), -7, np.int32) if with_input_ids else None,
    }
    st = np.zeros(1, np.uint32)
    rc = lib.orc_prepare_batch(n, T, _ptr(rows), _ptr(counts), _ptr(comp), R, _ptr(tok),
                               tok.strides[0] // 4 if tok.ndim == 2 else 0, L,
                               _ptr(out["index_mapping"]), _ptr(out["query_start_loc"]),
                               _ptr(out["seq_lens"]), _ptr(out["positions"]),
                               _ptr(out["input_ids"]), _ptr(st))
    out["status"], out["rc"] = int(st[0]), int(rc)
    return out


IBT_UNWRITTEN = -9  # fill value of input_block_tables entries the call must not write


def compute_slot_mapping(index_mapping, query_start_loc, seq_lens, positions, block_table,
                         block_size, num_blocks, *, with_ibt=True, sliding_window=0, lib=None):
    """Oracle of ``compute_slot_mapping`` for one KV-cache group (sliding_window
    0 = full attention)."""
    lib = lib or load()
    im, qsl, sl, pos = _i32(index_mapping), _i32(query_start_loc), _i32(seq_lens), _i32(positions)
    bt = _i32(block_table)
    n, T = im.shape[0], pos.shape[0]
    R, MB = bt.shape
    out = {
        "slot_mapping": np.full(T, -7, np.int32),
        "input_block_tables": np.full((n, MB), IBT_UNWRITTEN, np.int32) if with_ibt else None,
    }
    st = np.zeros(1, np.uint32)
    rc = lib.orc_compute_slot_mapping(n, T, _ptr(im), _ptr(qsl), _ptr(sl), _ptr(pos), _ptr(bt),
                                      R, MB, block_size, num_blocks, sliding_window,
                                      _ptr(out["slot_mapping"]),
                                      _ptr(out["input_block_tables"]), _ptr(st))
    out["status"], out["rc"] = int(st[0]), int(rc)
    return out


def scatter_kv(k, v, k_cache, v_cache, slot_mapping, *, lib=None):
    """Oracle of ``scatter_kv``: writes into ``k_cache``/``v_cache`` in place.

    ``k``/``v`` are [T, ...] arrays whose rows may be strided; the caches are
    C-contiguous [num_slots, ...] arrays with the same row size.  Returns
    ``(rc, status)``.
    """
    lib = lib or load()
    sm = _i32(slot_mapping)
    T = sm.shape[0]
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    row_bytes = int(np.prod(k_cache.shape[1:])) * k_cache.itemsize
    num_slots = k_cache.shape[0]
    for a in (k, v):
        assert a.shape[0] == T
        assert int(np.prod(a.shape[1:])) * a.itemsize == row_bytes
        # each row itself must be contiguous: only the token stride may differ
        assert a.shape[0] == 0 or a[0].flags.c_contiguous
    st = np.zeros(1, np.uint32)
    rc = lib.orc_scatter_kv(T, row_bytes, _ptr(k), k.strides[0] if T else row_bytes,
                            _ptr(v), v.strides[0] if T else row_bytes,
                            _ptr(k_cache), _ptr(v_cache), num_slots, _ptr(sm), _ptr(st))
    return int(rc), int(st[0])


def gather_kv(seq_lens, input_block_tables, block_size, num_blocks, k_cache, v_cache,
              out_tokens=None, *, out_fill=0xFFFF, query_start_loc=None, sliding_window=0,
              lib=None):
    """Oracle of the paged K/V read: the rows of every position < seq_len,
    request after request.  ``k_cache``/``v_cache`` are C-contiguous
    [num_blocks * block_size, ...] arrays.  Returns a dict with ``k``, ``v``
    ([out_tokens, ...], filled with ``out_fill`` where nothing is read),
    ``kv_start`` [n+1], ``status`` and ``rc``."""
    lib = lib or load()
    sl, ibt = _i32(seq_lens), _i32(input_block_tables)
    qsl = None if query_start_loc is None else _i32(query_start_loc)
    n = sl.shape[0]
    MB = ibt.shape[1] if ibt.ndim == 2 else 0
    if out_tokens is None:
        lens = np.maximum(sl.astype(np.int64), 0)
        if sliding_window > 0:
            cnt = np.maximum(np.diff(qsl.astype(np.int64)), 0)
            lens = lens - np.maximum(lens - cnt - sliding_window + 1, 0)
        out_tokens = int(lens.sum())
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.shape[0] >= num_blocks * block_size
    row_shape = k_cache.shape[1:]
    row_bytes = int(np.prod(row_shape)) * k_cache.itemsize
    out = {"k": np.full((out_tokens, *row_shape), out_fill, k_cache.dtype),
           "v": np.full((out_tokens, *row_shape), out_fill, v_cache.dtype),
           "kv_start": np.full(n + 1, -7, np.int32)}
    st = np.zeros(1, np.uint32)
    rc = lib.orc_gather_kv(n, _ptr(sl), _ptr(qsl), sliding_window,
                           _ptr(ibt) if MB else None, MB, block_size, num_blocks,
                           row_bytes, _ptr(k_cache), _ptr(v_cache), out_tokens, _ptr(out["k"]),
                           row_bytes, _ptr(out["v"]), row_bytes, _ptr(out["kv_start"]), _ptr(st))
    out["status"], out["rc"] = int(st[0]), int(rc)
    return out


def run_chain(batch, *, caches=None, sentinel=0xFFFF, lib=None):
    """Whole chain on one ``workloads.Batch``: prepare, then per group the slot
    mapping and the scatter into host caches (filled with ``sentinel`` words
    unless ``caches`` is given).  Returns (prep, [per-group dict])."""
    lib = lib or load()
    prep = prepare_batch(batch.sched_rows, batch.num_scheduled, batch.completed,
                         batch.token_ids, batch.T, lib=lib)
    groups = []
    for gi, g in enumerate(batch.groups):
        sm = compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                  prep["seq_lens"], prep["positions"], g.block_table,
                                  g.block_size, g.num_blocks, lib=lib)
        if caches is not None:
            kc, vc = caches[gi]
        else:
            kc = np.full((g.num_slots, g.num_heads, g.head_dim), sentinel, np.uint16)
            vc = np.full((g.num_slots, g.num_heads, g.head_dim), sentinel, np.uint16)
        rc, st = scatter_kv(g.k, g.v, kc, vc, sm["slot_mapping"], lib=lib)
        sm["scatter_rc"], sm["scatter_status"] = rc, st
        sm["k_cache"], sm["v_cache"] = kc, vc
        groups.append(sm)
    return prep, groups


# ---------------------------------------------------------------------------
# persistent request state (updated in place)
# ---------------------------------------------------------------------------

def csr(lists):
    """[list, ...] -> (start[m+1], flat, total) with int32 arrays (flat holds at
    least one element so that its pointer is valid)."""
    start = np.zeros(len(lists) + 1, np.int32)
    start[1:] = np.cumsum([len(x) for x in lists]) if lists else []
    total = int(start[-1])
    flat = np.array([v for x in lists for v in x], np.int32) if total else np.zeros(1, np.int32)
    return start, flat, total


def add_requests(state, rows, num_computed, prompts, blocks, *, lib=None):
    """add_request for each new request, on a state dict with int32 arrays
    completed[R], token_ids[R, L], block_table[R, MB], row_blocks[R] (in place).
    prompts / blocks: one list per request, or (start, flat, total) CSR triples
    (which may hold bad ranges).  Returns (rc, status)."""
    lib = lib or load()
    rows, nc = _i32(rows), _i32(num_computed)
    ps, pt, ptot = prompts if isinstance(prompts, tuple) else csr(prompts)
    bs_, bl, btot = blocks if isinstance(blocks, tuple) else csr(blocks)
    tok, bt = state["token_ids"], state["block_table"]
    st = np.zeros(1, np.uint32)
    # every array passed by address is held in a local for the whole call
    ps, pt, bs_, bl = _i32(ps), _i32(pt), _i32(bs_), _i32(bl)
    rc = lib.orc_add_requests(rows.size, _ptr(rows), _ptr(nc), _ptr(ps), _ptr(pt),
                              ptot, _ptr(bs_), _ptr(bl), btot,
                              state["completed"].size, _ptr(state["completed"]),
                              _ptr(tok), tok.strides[0] // 4, tok.shape[1], _ptr(bt), bt.shape[1],
                              _ptr(state["row_blocks"]), _ptr(st))
    return int(rc), int(st[0])


def append_blocks(state, rows, blocks, *, lib=None):
    """update_request: append each request's newly allocated blocks (in place)."""
    lib = lib or load()
    rows = _i32(rows)
    bs_, bl, btot = blocks if isinstance(blocks, tuple) else csr(blocks)
    bt = state["block_table"]
    st = np.zeros(1, np.uint32)
    bs_, bl = _i32(bs_), _i32(bl)
    rc = lib.orc_append_blocks(rows.size, _ptr(rows), _ptr(bs_), _ptr(bl), btot,
                               bt.shape[0], _ptr(bt), bt.shape[1], _ptr(state["row_blocks"]),
                               _ptr(st))
    return int(rc), int(st[0])


def advance_state(state, index_mapping, seq_lens, sampled=None, *, lib=None):
    """After a step: completed[row] = seq_len, sampled tokens appended (in place)."""
    lib = lib or load()
    im, sl = _i32(index_mapping), _i32(seq_lens)
    sm = None if sampled is None else _i32(sampled)
    tok = state["token_ids"]
    st = np.zeros(1, np.uint32)
    rc = lib.orc_advance_state(im.size, _ptr(im), _ptr(sl), _ptr(sm), state["completed"].size,
                               _ptr(state["completed"]), _ptr(tok), tok.strides[0] // 4,
                               tok.shape[1], _ptr(st))
    return int(rc), int(st[0])


def empty_state(R, L, MB, token_fill=-1):
    """A fresh state: nothing computed, no tokens, no blocks."""
    return {"completed": np.zeros(R, np.int32),
            "token_ids": np.full((R, L), token_fill, np.int32),
            "block_table": np.full((R, MB), -1, np.int32),
            "row_blocks": np.zeros(R, np.int32)}


class RowPool:
    """The oracle's row pool on NumPy arrays (see orc_pool_* in oracle.c)."""

    def __init__(self, R, *, lib=None):
        self.lib = lib or load()
        self.R = int(R)
        self.free_rows = np.zeros(max(self.R, 1), np.int32)
        self.in_use = np.zeros(max(self.R, 1), np.uint8)
        self.num_free = np.zeros(1, np.int32)
        rc = self.lib.orc_pool_reset(self.R, _ptr(self.free_rows), _ptr(self.num_free),
                                     _ptr(self.in_use))
        assert rc == OK

    def acquire(self, m):
        """(rc, rows handed out)"""
        out = np.full(max(int(m), 1), -7, np.int32)
        rc = self.lib.orc_pool_acquire(self.R, _ptr(self.free_rows), _ptr(self.num_free),
                                       _ptr(self.in_use), int(m), _ptr(out))
        return int(rc), (out[:m].tolist() if rc == OK else [])

    def release(self, rows):
        r = _i32(rows) if len(rows) else np.zeros(1, np.int32)
        return int(self.lib.orc_pool_release(self.R, _ptr(self.free_rows), _ptr(self.num_free),
                                             _ptr(self.in_use), len(rows), _ptr(r)))

    @property
    def free(self):
        return int(self.num_free[0])


# ---------------------------------------------------------------------------
# prefix-cache block hashes and the prefix index
# ---------------------------------------------------------------------------

def hash_blocks(token_lists=None, block_size=16, MB=None, *, views=None, lib=None):
    """Hashes of every full block of each token list (see orc_hash_blocks).
    token_lists: list of int sequences, or views=(tokens flat, total, starts
    int64 [m], lengths int32 [m]).  Returns dict(hashes uint64 [m, MB] (0
    where not written), num_full [m], status, rc)."""
    lib = lib or load()
    if views is None:
        lens = [len(t) for t in token_lists]
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64) if lens else \
            np.zeros(0, np.int64)
        flat = np.array([x for t in token_lists for x in t], np.int32)
        total = int(flat.size)
        lengths = np.asarray(lens, np.int32)
        if MB is None:
            MB = max([l // block_size for l in lens] + [0])
    else:
        flat, total, starts, lengths = views
        flat = _i32(flat)
        starts = np.ascontiguousarray(starts, np.int64)
        lengths = _i32(lengths)
    if flat.size == 0:
        flat = np.zeros(1, np.int32)
    m = lengths.size
    out = np.zeros((m, MB), np.uint64)
    nf = np.full(m, -7, np.int32)
    st = np.zeros(1, np.uint32)
    rc = lib.orc_hash_blocks(m, _ptr(flat), total, _ptr(starts), _ptr(lengths), block_size, MB,
                             _ptr(out), _ptr(nf), _ptr(st))
    return {"hashes": out, "num_full": nf, "status": int(st[0]), "rc": int(rc)}


def fnv1a64(data: bytes, *, lib=None) -> int:
    """The oracle's FNV-1a 64-bit hash of a byte string."""
    lib = lib or load()
    return int(lib.orc_fnv1a64(data, len(data)))


class PrefixIndex:
    """The oracle's prefix index: hash -> smallest registered block id, with
    room for ``capacity`` distinct hashes (see orc_prefix_*)."""

    def __init__(self, capacity, *, lib=None):
        self.lib = lib or load()
        self.capacity = int(capacity)
        self.keys = np.zeros(max(self.capacity, 1), np.uint64)
        self.vals = np.full(max(self.capacity, 1), NO_BLOCK, np.int32)

    def lookup(self, hashes, lengths, block_size):
        h = np.ascontiguousarray(hashes, np.uint64)
        m, MB = h.shape
        ln = _i32(lengths)
        hit = np.full((m, MB), -7, np.int32)
        nc = np.full(m, -7, np.int32)
        st = np.zeros(1, np.uint32)
        rc = self.lib.orc_prefix_lookup(m, _ptr(h), MB, _ptr(ln), block_size, _ptr(self.keys),
                                        _ptr(self.vals), self.capacity, _ptr(hit), _ptr(nc),
                                        _ptr(st))
        return {"hit_blocks": hit, "num_computed": nc, "status": int(st[0]), "rc": int(rc)}

    def insert(self, hashes, lo, hi, rows, block_table):
        h = np.ascontiguousarray(hashes, np.uint64)
        m, MB = h.shape
        bt = _i32(block_table)
        st = np.zeros(1, np.uint32)
        lo, hi, rows = _i32(lo), _i32(hi), _i32(rows)        # held for the call
        rc = self.lib.orc_prefix_insert(m, _ptr(h), MB, _ptr(lo), _ptr(hi),
                                        _ptr(rows), _ptr(bt), bt.shape[0], _ptr(self.keys),
                                        _ptr(self.vals), self.capacity, _ptr(st))
        return int(rc), int(st[0])

    def evict(self, hashes, blocks):
        h = np.ascontiguousarray(hashes, np.uint64).reshape(-1)
        bl = _i32(blocks).reshape(-1)
        return int(self.lib.orc_prefix_evict(h.size, _ptr(h), _ptr(bl), _ptr(self.keys),
                                             _ptr(self.vals), self.capacity))

    def live(self):
        """{hash: block} of the entries that hold a block."""
        return {int(k): int(v) for k, v in zip(self.keys[:self.capacity], self.vals[:self.capacity])
                if k != 0 and v != NO_BLOCK}

    def known(self):
        """Every hash that takes room (with or without a block)."""
        return {int(k) for k in self.keys[:self.capacity] if k != 0}


# ---------------------------------------------------------------------------
# sliding-window holes and speculative lookahead
# ---------------------------------------------------------------------------

def window_free(rows, completed, block_table, block_size, sliding_window, *, lib=None):
    """Free the blocks wholly before every window (block_table updated in
    place).  Returns dict(freed [m, MB] (-7 where not written), num_freed [m],
    status, rc)."""
    lib = lib or load()
    rows, comp = _i32(rows), _i32(completed)
    assert block_table.dtype == np.int32 and block_table.flags.c_contiguous
    R, MB = block_table.shape
    m = rows.size
    freed = np.full((m, max(MB, 1)), -7, np.int32)
    nf = np.full(m, -7, np.int32)
    st = np.zeros(1, np.uint32)
    rc = lib.orc_window_free(m, _ptr(rows), _ptr(comp), _ptr(block_table), R, MB, block_size,
                             sliding_window, _ptr(freed), _ptr(nf), _ptr(st))
    return {"freed": freed[:, :MB], "num_freed": nf, "status": int(st[0]), "rc": int(rc)}


def lookahead_slots(index_mapping, seq_lens, block_table, block_size, num_blocks, k, *, lib=None):
    """Slots of the k positions after each request's seq_len."""
    lib = lib or load()
    im, sl, bt = _i32(index_mapping), _i32(seq_lens), _i32(block_table)
    R, MB = bt.shape
    n = im.size
    out = np.full((n, max(k, 1)), -7, np.int32)
    st = np.zeros(1, np.uint32)
    rc = lib.orc_lookahead_slots(n, _ptr(im), _ptr(sl), _ptr(bt), R, MB, block_size, num_blocks,
                                 k, _ptr(out), _ptr(st))
    return {"slots": out[:, :k], "status": int(st[0]), "rc": int(rc)}


def blocks_needed(rows, num_new, k, block_size, completed, row_blocks, *, lib=None):
    """New blocks each request still needs for its new and lookahead tokens."""
    lib = lib or load()
    rows, nn, comp, rb = _i32(rows), _i32(num_new), _i32(completed), _i32(row_blocks)
    n = rows.size
    need = np.full(max(n, 1), -7, np.int32)
    st = np.zeros(1, np.uint32)
    rc = lib.orc_blocks_needed(n, _ptr(rows), _ptr(nn), k, block_size, _ptr(comp), _ptr(rb),
                               comp.size, _ptr(need), _ptr(st))
    return {"need": need[:n], "status": int(st[0]), "rc": int(rc)}
