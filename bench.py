"""Benchmark of the paged-KV input path on one MI355X.

A step is the whole path on one synthetic batch: prepare_batch, then for every
KV-cache group compute_slot_mapping and scatter_kv (one layer), with every
input already resident in HBM.  Default workload: 16 requests x 2048 new
tokens (32768 tokens) from an empty history, block size 32, a 131072-block
pool, K/V of 8 heads x 128 in bf16.

Timing: the step inputs come in ROTATE independent seeded batches of the same
shape (own K/V payload, rows and random block tables; one shared pair of
caches), so consecutive steps never find each other's data in L2 or the
256 MB Infinity Cache (a cycle touches over 1 GB).  W untimed warm-up steps,
then exactly K timed steps back to back, bracketed by torch.cuda.synchronize()
on both sides and by HIP events on the launch stream; ms_per_step is the
event interval / K.  The step runs through pkv_step (one launch whenever
the groups fit: each workgroup ranking its own requests for batches of short
requests, else each workgroup ordering the batch and writing a tile of flat
tokens; past 512 longer requests, the batch with every group's slots and
pages in one launch, then the scatters) and, timed the same way, through the
three separate calls; value is the faster.  Secondary figures: the
per-call split of the three calls, the host wall time of one step with the
schedule uploaded from pinned host memory, flushed single steps (100 of them
whatever K is: a 1 GiB rewrite before each step, events around it; median,
p10, p90 and the fraction of peak at the median), ceilings to
read the step against (a same-byte device copy, the rate at which the host issues one-lane launches), and the
calls around the path: the state updates, the paged K/V read, the
prefix-cache calls and the sliding-window and lookahead variants.

Prints one JSON line (N = 1 only: the benchmark runs on one GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scheduled tokens/sec (prep+slot_mapping+KV scatter); HBM GB/s % of peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
FLUSH_BYTES = 1 << 30
ROTATE = 4
COLD_REPS = 100                # flushed single-step reps, whatever --steps is


def algorithmic_bytes(batch):
    """Bytes the step must move, each required read or write counted once
    (no re-reads of intermediates, no scratch):
      K/V     4 * T * row_bytes per group (read K and V, write both cache rows)
      tokens  T * (4 position write + 4 input-id write + 4 input-id read)
              + 4 * T per group (slot write)
      requests  24 * n + 4 (rows, counts, completed read; index_mapping,
              seq_lens, query_start_loc written)
      table   4 bytes per logical block the new tokens touch, per group
      pages   8 bytes per visible block (read + write), per group
    """
    import numpy as np

    T, n = batch.T, batch.n
    done = batch.completed[batch.sched_rows].astype(np.int64)
    cnt = batch.num_scheduled.astype(np.int64)
    kv = sum(4 * T * g.row_bytes for g in batch.groups)
    tok = T * 12 + sum(4 * T for _ in batch.groups)
    req = 24 * n + 4
    table = pages = 0
    for g in batch.groups:
        bs = g.block_size
        touched = np.where(cnt > 0, (done + cnt - 1) // bs - done // bs + 1, 0)
        table += 4 * int(touched.sum())
        pages += 8 * int((-(-(done + cnt) // bs)).sum())
    return dict(kv=kv, tokens=tok, requests=req, block_table=table, pages=pages,
                total=kv + tok + req + table + pages)


def call_bytes(batch):
    """Algorithmic bytes of each separate call on its own (inputs read once,
    outputs written once):
      prepare_batch         12 n (rows, counts, completed) + 4 T (token table)
                            + 12 n + 4 (index_mapping, seq_lens, query_start_loc)
                            + 8 T (positions, input_ids)
      compute_slot_mapping  per group: 4 T (positions) + 4 T (slots) + 8 n + 4 (index
                            mapping, query_start_loc) + 4 n (seq_lens) + 4 per touched
                            block + 8 per visible block
      scatter_kv            per group: T (4 row_bytes + 4)
    """
    import numpy as np

    T, n = batch.T, batch.n
    done = batch.completed[batch.sched_rows].astype(np.int64)
    cnt = batch.num_scheduled.astype(np.int64)
    prep = 24 * n + 4 + 12 * T
    slots = 0
    for g in batch.groups:
        bs = g.block_size
        touched = np.where(cnt > 0, (done + cnt - 1) // bs - done // bs + 1, 0)
        slots += 8 * T + 12 * n + 4 + 4 * int(touched.sum()) + 8 * int((-(-(done + cnt) // bs)).sum())
    scat = sum(scatter_bytes_per_launch(batch, gi) for gi in range(len(batch.groups)))
    return dict(prepare_batch=prep, compute_slot_mapping=slots, scatter_kv=scat)


def scatter_bytes_per_launch(batch, gi):
    """Algorithmic bytes of one scatter_kv launch: per token, read K and V rows,
    write both cache rows, read the slot (4 * row_bytes + 4)."""
    g = batch.groups[gi]
    return batch.T * (4 * g.row_bytes + 4)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_sources(kernel):
    csrc = os.path.join(ROOT, "paged_kv_input_amd", "csrc")
    files = {"step": ["step.hip", "internal.h", "geometry.h"],
             "ranked_step": ["prepare.hip", "internal.h", "geometry.h"],
             "scatter_kv": ["scatter.hip", "internal.h", "geometry.h"],
             "gather_kv": ["gather.hip", "internal.h", "geometry.h"]}
    return [os.path.join(csrc, f) for f in files[kernel]]


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch of the kernel from the committed rocprofv3 counter
    summary, when it was taken on the kernel's current source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_b) or m_src.group(1) != source_digest(kernel_sources(kernel)):
        return None
    return float(m_b.group(1))


_CPU_BATCH = None     # the batch the forked oracle workers inherit


def _oracle_loop(budget_s):
    """One host thread: the oracle's whole step (prepare, slots and the scatter
    into lazily mapped host caches) on the seeded batch, repeated for about
    budget_s.  Returns (tokens, seconds, repetitions)."""
    import numpy as np
    import oracle

    batch = _CPU_BATCH
    lib = oracle.load()
    caches = [(np.zeros((g.num_slots, g.num_heads, g.head_dim), np.uint16),
               np.zeros((g.num_slots, g.num_heads, g.head_dim), np.uint16)) for g in batch.groups]
    oracle.run_chain(batch, caches=caches, lib=lib)       # first touch of the written pages
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run_chain(batch, caches=caches, lib=lib)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return batch.T * reps, el, reps


def cpu_baseline(workload, seed, budget_s):
    """The CPU oracle, as it stands, on the same step.  Run before the GPU is
    touched: first on one host thread, then as one process per host core (at
    most 16) started together, each forked with the batch already built (so
    the workers run only the oracle's C code), the aggregate being all their
    tokens over the longest of their times."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import oracle
    import workloads

    global _CPU_BATCH
    _CPU_BATCH = workloads.make(workload, seed=seed)
    oracle.load()                                   # built and loaded before the fork
    tok1, el1, reps1 = _oracle_loop(budget_s)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    par_budget = max(1.0, budget_s / 4)
    with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("fork")) as ex:
        runs = list(ex.map(_oracle_loop, [par_budget] * workers))
    _CPU_BATCH = None
    tokens = sum(r[0] for r in runs)
    wall = max(r[1] for r in runs)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), None)
    except OSError:
        pass
    return dict(value=tokens / wall, unit="tokens/s", cores=workers, kind="oracle",
                cpu_model=cpu_model,
                sample=f"the full {workload} step, {workers} processes (one per host core) each "
                       f"repeating it for about {par_budget:.1f} s ({sum(r[2] for r in runs)} steps "
                       f"in all); plain C oracle, gcc -O2",
                one_thread={"value": tok1 / el1, "unit": "tokens/s", "cores": 1,
                            "sample": f"{reps1} steps in {el1:.1f} s on one host thread"})


def state_calls(batch, step, steps, warmup, stream):
    """The persistent-state updates on this batch's shape, each timed back to
    back like the step: registering the batch's requests (add_requests: each
    prompt is the history plus this step's tokens, its blocks are the
    allocated prefix of group 0's block-table row), appending one new block
    per request (append_blocks; the table is widened so that every timed call
    has room) and the after-step advance (advance_state on the step's own
    index_mapping and seq_lens, one sampled token per request).  All three
    move well under 1 MB here, so they are bound by launch and memory
    latency; bytes count each required read or write once."""
    import numpy as np
    import torch

    from paged_kv_input_amd import api
    from paged_kv_input_amd.state import DeviceState, pack_csr

    g = batch.groups[0]
    rows = batch.sched_rows.astype(np.int64)
    plen = np.minimum(batch.completed[rows].astype(np.int64)
                      + np.maximum(batch.num_scheduled, 0), batch.L)
    nblk = np.minimum(-(-plen // g.block_size), g.max_blocks)
    MB = g.max_blocks + warmup + steps
    ds = DeviceState(batch.R, batch.L + 1, MB)     # one spare position for the sampled token
    dev = ds.device

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    ps, pt, _ = pack_csr([batch.token_ids[r, :p] for r, p in zip(rows, plen)])
    bs_, bl, _ = pack_csr([g.block_table[r, :k] for r, k in zip(rows, nblk)])
    ptot, btot = int(plen.sum()), int(nblk.sum())
    rows_d = up(rows)
    add = api.prepared_add_requests(
        rows_d, up(batch.completed[rows]), up(ps), up(pt)[:ptot], up(bs_), up(bl)[:btot],
        completed=ds.completed,
        token_ids=ds.token_ids, block_table=ds.block_table, row_blocks=ds.row_blocks,
        status=ds.status)
    one = pack_csr([[int(b)] for b in np.arange(batch.n) % max(g.num_blocks, 1)])
    app = api.prepared_append_blocks(rows_d, up(one[0]), up(one[1]),
                                     block_table=ds.block_table, row_blocks=ds.row_blocks,
                                     status=ds.status)
    sampled = up(np.arange(batch.n) % 128256)
    adv = api.prepared_advance_state(step.index_mapping, step.seq_lens, sampled,
                                     completed=ds.completed, token_ids=ds.token_ids,
                                     status=ds.status)
    add(stream)

    def timed(fn):
        for _ in range(warmup):
            fn(stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    n = batch.n
    out = {}
    for name, fn, nbytes in (
            ("add_requests", add,
             int((8 * plen + 4 * nblk).sum()) + 4 * MB * n + 24 * n + 8),
            ("append_blocks", app, 24 * n + 4),
            ("advance_state", adv, 20 * n)):
        ms = timed(fn)
        out[name] = {"ms": ms, "algorithmic_bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
                     "bound": "latency"}
    if ds.status_bits() != 0:
        raise RuntimeError(f"state status bits set: {ds.status_bits():#x}")
    out["note"] = (f"{n} requests; add_requests registers {ptot} prompt tokens and {btot} "
                   f"blocks into a {MB}-wide table; append_blocks adds 1 block per request")
    return out


def variant_calls(batch, step, steps, warmup, stream, window=1024, k=4):
    """The allocation-side variants on this batch's shape (group 0): the slots
    of k speculative lookahead positions after every request's seq_len, the
    new blocks each request needs for its new and k lookahead tokens (both
    timed back to back), and the blocks a sliding window of `window` tokens no
    longer needs.  window_free changes the table, so each of its calls runs
    on a fresh copy (restored untimed) with HIP events around the call alone;
    its figure is the median.  Bytes count each required read or write once."""
    import numpy as np
    import torch

    from paged_kv_input_amd import api

    g, gd = batch.groups[0], step.groups[0]
    dev = step.completed.device
    n, bs, MB = batch.n, g.block_size, g.max_blocks

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    rows_d = up(batch.sched_rows)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)     # expected: unallocated lookahead
    look_out = torch.empty((n, k), dtype=torch.int32, device=dev)
    look = api.prepared_lookahead_slots(step.index_mapping, step.seq_lens, gd["block_table"], bs,
                                        g.num_blocks, out=look_out, status=flags)
    row_blocks = up((g.block_table >= 0).sum(axis=1))
    need = torch.empty(n, dtype=torch.int32, device=dev)
    needed = api.prepared_blocks_needed(rows_d, step.num_scheduled, k, bs, step.completed,
                                        row_blocks, need=need, status=flags)

    def timed(fn):
        for _ in range(warmup):
            fn(stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    out = {}
    for name, fn, nbytes in (("lookahead_slots", look, 8 * n + 8 * n * k),
                             ("blocks_needed", needed, 20 * n)):
        ms = timed(fn)
        out[name] = {"ms": ms, "algorithmic_bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
                     "bound": "latency"}

    done = batch.completed[batch.sched_rows].astype(np.int64)
    scan = np.minimum(np.maximum(done - window + 1, 0) // bs, MB)
    freed_n = sum(int((g.block_table[r, :c] >= 0).sum()) for r, c in zip(batch.sched_rows, scan))
    base = gd["block_table"].clone()
    work = base.clone()
    freed = torch.empty((n, MB), dtype=torch.int32, device=dev)
    num_freed = torch.empty(n, dtype=torch.int32, device=dev)
    wf = api.prepared_window_free(rows_d, step.completed, work, bs, window, freed=freed,
                                  num_freed=num_freed, status=flags)
    times = []
    for i in range(warmup + min(steps, 100)):
        work.copy_(base)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        wf(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            times.append(e0.elapsed_time(e1))
    if int(num_freed.sum().item()) != freed_n:
        raise RuntimeError("window_free released an unexpected number of blocks")
    ms = statistics.median(times)
    nbytes = 12 * n + 4 * int(scan.sum()) + 8 * freed_n
    out["window_free"] = {"ms": ms, "algorithmic_bytes": nbytes,
                          "gbs": nbytes / (ms * 1e-3) / 1e9, "bound": "latency",
                          "blocks_freed": freed_n,
                          "timing": "events around single calls (median), table restored untimed"}
    out["note"] = (f"{n} requests, group 0 (block size {bs}); {k} lookahead positions; "
                   f"a {window}-token window")
    return out


def gather_calls(batch, steps_dev, steps, warmup, stream, workload):
    """The paged K/V read on this batch's shape: after the step, every group's
    KV range of every request (history plus new tokens) read through its
    visible pages into a contiguous varlen array; rotating over the same
    seeded batches as the step, timed back to back.  Bytes (averaged over the
    rotation): each K/V row read once and written once, 4 B per visible page
    read, the seq_lens read and kv_start written."""
    import numpy as np
    import torch

    from paged_kv_input_amd import api

    seqs = [np.maximum(st.seq_lens.cpu().numpy().astype(np.int64), 0) for st in steps_dev]
    rows = [int(q.sum()) for q in seqs]
    outs = []
    for g in steps_dev[0].groups:
        kc = g["k_cache"]
        outs.append(tuple(torch.empty((max(rows), *kc.shape[1:]), dtype=kc.dtype,
                                      device=kc.device) for _ in range(2)))
    launches = [[api.prepared_gather_kv(st.seq_lens, g["input_block_tables"], g["block_size"],
                                        g["num_blocks"], g["k_cache"], g["v_cache"],
                                        k_out=o[0][:r], v_out=o[1][:r], status=st.status)
                 for g, o in zip(st.groups, outs)]
                for st, r in zip(steps_dev, rows)]
    per_batch = [sum(4 * r * bg.row_bytes + 4 * int((-(-q // bg.block_size)).sum())
                     + 8 * batch.n + 4 for bg in batch.groups) for q, r in zip(seqs, rows)]
    nbytes = statistics.fmean(per_batch)          # the timed loop cycles through them evenly

    def run(i):
        for fn in launches[i % len(launches)]:
            fn(stream)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    for st in steps_dev:
        if st.status_bits() != 0:
            raise RuntimeError(f"gather status bits set: {st.status_bits():#x}")
    return {"ms": ms, "kv_rows": statistics.fmean(rows), "algorithmic_bytes": nbytes,
            "gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bound": "hbm",
            "kernel": "pkv_gather_kv (k_gather)", "launches_per_step": len(batch.groups),
            "traffic_per_launch": traffic_from_profile("gather_kv", workload)}


def prefix_calls(batch, step, steps, warmup, stream):
    """Prefix-cache work on this batch's shape: every scheduled request's whole
    token list after the step (seq_len tokens, read from the persistent token
    table) hashed block by block (group 0's block size), its full blocks
    registered in an index of twice their number, and the lookup that then
    hits each request's cap; each call timed back to back.  Hashing is bound by
    the FNV-1a multiply chain (ALU), lookup and registration by memory latency."""
    import numpy as np
    import torch

    from paged_kv_input_amd import api

    g = batch.groups[0]
    bs = g.block_size
    rows = batch.sched_rows.astype(np.int64)
    lengths = np.minimum(batch.completed[rows].astype(np.int64)
                         + np.maximum(batch.num_scheduled, 0), batch.L).astype(np.int32)
    full = lengths // bs
    MB = max(int(full.max()), 1)
    dev = step.device
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)   # noqa: E731
    tokens = step.token_ids.view(-1)
    starts = up(rows * batch.L)
    lens = up(lengths)
    m = batch.n
    hashes = torch.zeros((m, MB), dtype=torch.int64, device=dev)
    num_full = torch.empty(m, dtype=torch.int32, device=dev)
    cap = 1 << max(4, int(2 * full.sum()).bit_length())
    keys = torch.empty(cap, dtype=torch.int64, device=dev)
    vals = torch.empty(cap, dtype=torch.int32, device=dev)
    api.prefix_clear(keys, vals)
    table = up(np.arange(m * MB, dtype=np.int32).reshape(m, MB))
    zero, rid = up(np.zeros(m, np.int32)), up(np.arange(m, dtype=np.int32))
    nc = torch.empty(m, dtype=torch.int32, device=dev)
    hits = torch.empty((m, MB), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def hash_():
        api.hash_blocks(tokens, starts, lens, bs, hashes=hashes, num_full=num_full,
                        status=status, stream=stream)

    def insert():
        api.prefix_insert(hashes, zero, num_full, rid, table, keys, vals, status=status,
                          stream=stream)

    def lookup():
        api.prefix_lookup(hashes, lens, bs, keys, vals, num_computed=nc, hit_blocks=hits,
                          status=status, stream=stream)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    out = {}
    tok = int(lengths.sum())
    nblk = int(full.sum())
    for name, fn in (("hash_blocks", hash_), ("prefix_insert", insert),
                     ("prefix_lookup", lookup)):
        ms = timed(fn)
        out[name] = {"ms": ms}
    want = ((np.maximum(lengths, 1) - 1) // bs) * bs
    if status.item() != 0 or not np.array_equal(nc.cpu().numpy(), want):
        raise RuntimeError("prefix calls: unexpected status or hits")
    hs = out["hash_blocks"]
    hs["tokens_per_s"] = tok / (hs["ms"] * 1e-3)
    # FNV-1a over 4 bytes per token, then 8 bytes per block for its hash:
    # one xor and one 64-bit multiply by the prime per byte.
    hs["fnv_bytes_per_s"] = (4 * tok + 8 * nblk) / (hs["ms"] * 1e-3)
    hs["bound"] = "alu"
    out["prefix_insert"]["blocks_per_s"] = nblk / (out["prefix_insert"]["ms"] * 1e-3)
    out["prefix_lookup"]["blocks_per_s"] = nblk / (out["prefix_lookup"]["ms"] * 1e-3)
    out["note"] = (f"{m} requests, {tok} tokens, {nblk} full blocks of {bs}; index of {cap} "
                   "entries; every lookup hits its cap")
    return out


def hip_enum_values(enum, header="/opt/rocm/include/hip/hip_runtime_api.h"):
    """Values of a C enum of the installed HIP header: each enumerator is the
    previous one plus one unless it is assigned a literal or an earlier name."""
    with open(header) as f:
        text = f.read()
    m = re.search(r"typedef\s+enum\s+" + enum + r"\s*\{(.*?)\}", text, re.S)
    if m is None:
        raise ValueError(f"{enum} not found in {header}")
    body = re.sub(r"//[^\n]*|/\*.*?\*/", "", m.group(1), flags=re.S)
    if "#" in body:
        raise ValueError(f"preprocessor lines inside {enum}")
    vals, nxt = {}, 0
    for item in body.split(","):
        item = item.strip()
        if not item:
            continue
        name, _, expr = (x.strip() for x in item.partition("="))
        if expr:
            nxt = vals[expr] if expr in vals else int(expr, 0)
        vals[name] = nxt
        nxt += 1
    return vals


def device_hbm_peak():
    """HBM peak from the device's own figures (HIP's device attributes, read
    through the HIP runtime): bus width x memory clock x transfers per clock.
    HBM3E pins run at four transfers per reported memory clock (8 Gb/s at
    2 GHz), so on MI355X this gives 8192 bits x 2 GHz x 4 / 8 = 8.19 TB/s.
    The attribute numbers come from the installed hip_runtime_api.h."""
    import ctypes

    try:
        hip = ctypes.CDLL("libamdhip64.so")
        attrs = hip_enum_values("hipDeviceAttribute_t")
        bus_attr = attrs["hipDeviceAttributeMemoryBusWidth"]
        clock_attr = attrs["hipDeviceAttributeMemoryClockRate"]
    except (OSError, ValueError, KeyError):
        return None
    vals = []
    for attr in (bus_attr, clock_attr):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) != 0:
            return None
        vals.append(v.value)
    bus_bits, clock_khz = vals
    return {"bus_width_bits": bus_bits, "memory_clock_khz": clock_khz, "transfers_per_clock": 4,
            "gbs": 4.0 * clock_khz * 1e3 * bus_bits / 8 / 1e9}


def context_figures(step_bytes, steps, warmup, stream):
    """Ceilings to read the step against (not targets): a device-to-device copy
    moving the same bytes (half read, half written; torch's copy kernel, four
    rotating buffer pairs, back to back) and the rate at which the host issues
    a one-lane kernel launched back to back."""
    import torch

    half = int(round(step_bytes)) // 2
    src = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(ROTATE)]
    dst = [torch.empty_like(x) for x in src]

    def timed(fn, reps):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    copy_ms = timed(lambda i: dst[i % ROTATE].copy_(src[i % ROTATE]), steps)
    one = torch.zeros(1, device="cuda")
    tiny_ms = timed(lambda i: one.add_(1), max(steps, 1000))
    return {"d2d_copy_same_bytes": {"ms": copy_ms, "bytes": 2 * half,
                                    "gbs": 2 * half / (copy_ms * 1e-3) / 1e9},
            "tiny_kernel_us": tiny_ms * 1e3,
            "hbm_peak_from_device": device_hbm_peak()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_16x2048")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch a plain 256 MiB device copy (for counter calibration)")
    ap.add_argument("--step-only", action="store_true",
                    help="time pkv_step alone (warm-up, then K steps back to back) and print a "
                         "short line; for profiler runs, not a benchmark result")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported", file=sys.stderr, flush=True)
        sys.exit(2)

    import workloads

    default_seed = workloads.CONFIGS[args.workload][1]
    cpu = None
    if not args.no_cpu_baseline:          # before the GPU is touched: the workers are forked
        cpu = cpu_baseline(args.workload, default_seed, args.cpu_seconds)

    import torch

    from paged_kv_input_amd import api
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    torch.cuda.set_device(0)
    batches = [workloads.make(args.workload, seed=default_seed + 1000 * i) for i in range(ROTATE)]
    batch = batches[0]
    steps, caches = [], None
    for b in batches:
        st = DeviceStep(b.sched_rows, b.num_scheduled, b.completed, b.token_ids,
                        [GroupSpec(g.block_table, g.block_size, g.num_blocks, g.k, g.v)
                         for g in b.groups], caches=caches)
        caches = [(g["k_cache"], g["v_cache"]) for g in st.groups]
        steps.append(st)
    stream = torch.cuda.current_stream()
    print(f"[bench] {batch.name}: n={batch.n} T={batch.T} groups={len(batch.groups)} "
          f"rotating {ROTATE} batches", file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    ng = len(batch.groups)
    # Every timed loop cycles through the ROTATE batches evenly, so the tokens
    # and bytes of a step are their means over the rotation (the batches'
    # token counts differ where the workload draws them).
    T = statistics.fmean(b.T for b in batches)
    T = int(T) if T == int(T) else T

    def back_to_back(run):
        for i in range(args.warmup):
            run(steps[i % ROTATE])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        for i in range(args.steps):
            run(steps[i % ROTATE])
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return e0.elapsed_time(e1) / args.steps, wall * 1e3 / args.steps

    fused_ms, fused_wall = back_to_back(lambda s: s.run_fused(stream))
    if args.step_only:
        print(json.dumps({"workload": batch.name, "step_only": True, "steps": args.steps,
                          "ms_per_step": fused_ms, "plan": steps[0].fused_path()}), flush=True)
        return
    calls_ms, calls_wall = back_to_back(lambda s: s.run(stream))

    # The same steps captured once per batch in HIP graphs and replayed back to
    # back: the three calls (three kernels per graph) and pkv_step.
    graphs = {}
    for name, run in (("three_calls", lambda s: s.run()), ("fused", lambda s: s.run_fused())):
        gs = []
        for s_ in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run(s_)
            gs.append(g)
        graphs[name] = gs
    graph_ms = {name: back_to_back(lambda s, gs=gs: gs[steps.index(s)].replay())[0]
                for name, gs in graphs.items()}
    del graphs

    # Per-call split of the three calls (events between the calls add their own
    # overhead; for attribution only).
    split = {"prepare_batch": [], "compute_slot_mapping": [], "scatter_kv": []}
    reps = max(ROTATE, min(args.steps, 60) // ROTATE * ROTATE)   # whole rotations
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for i in range(reps):
        s, e = steps[i % ROTATE], marks[i]
        e[0].record(stream)
        s.prepare(stream)
        e[1].record(stream)
        for gi in range(ng):
            s.slots(gi, stream)
        e[2].record(stream)
        for gi in range(ng):
            s.scatter(gi, stream)
        e[3].record(stream)
    torch.cuda.synchronize()
    for e in marks:
        split["prepare_batch"].append(e[0].elapsed_time(e[1]))
        split["compute_slot_mapping"].append(e[1].elapsed_time(e[2]))
        split["scatter_kv"].append(e[2].elapsed_time(e[3]))

    # Host wall time of one step as a caller sees it: the schedule (rows and
    # counts, n x 8 bytes) copied from pinned host memory, the fused step, a
    # synchronize.  Each iteration starts on an idle GPU.
    s0 = steps[0]
    pin_rows = s0.sched_rows.cpu().pin_memory()
    pin_counts = s0.num_scheduled.cpu().pin_memory()
    upload_wall = []
    for i in range(args.warmup + min(args.steps, 200)):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        s0.sched_rows.copy_(pin_rows, non_blocking=True)
        s0.num_scheduled.copy_(pin_counts, non_blocking=True)
        s0.run_fused(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            upload_wall.append((time.perf_counter() - w0) * 1e6)

    # Flushed single steps: a 1 GiB rewrite (L2 and the 256 MB Infinity Cache
    # hold nothing of the step afterwards), then events around one fused step;
    # COLD_REPS of them whatever --steps is, median and deciles reported.
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(COLD_REPS)]
    for i in range(COLD_REPS):
        flush.fill_(1)
        cev[i][0].record(stream)
        steps[i % ROTATE].run_fused(stream)
        cev[i][1].record(stream)
    torch.cuda.synchronize()
    cold = [e[0].elapsed_time(e[1]) for e in cev]
    # The same protocol around a one-element torch kernel: the event and
    # dispatch latency that every flushed rep above also carries.
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(COLD_REPS)]
    for i in range(COLD_REPS):
        flush.fill_(1)
        lev[i][0].record(stream)
        one.add_(1)
        lev[i][1].record(stream)
    torch.cuda.synchronize()
    lone = [e[0].elapsed_time(e[1]) for e in lev]
    del flush, one

    for s in steps:
        if s.status_bits() != 0:
            raise RuntimeError(f"device status bits set: {s.status_bits():#x}")
    state = state_calls(batch, steps[0], args.steps, args.warmup, stream)
    variants = variant_calls(batch, steps[0], args.steps, args.warmup, stream)
    gather = gather_calls(batch, steps, args.steps, args.warmup, stream, args.workload)
    prefix = prefix_calls(batch, steps[0], args.steps, args.warmup, stream)

    ab = {"total": statistics.fmean(algorithmic_bytes(b)["total"] for b in batches)}
    cbs = [call_bytes(b) for b in batches]
    cb = {k: statistics.fmean(c[k] for c in cbs) for k in cbs[0]}
    # The launch plan pkv_step takes for this batch, as the library decides it
    # (pkv_step_path): one launch (k_step), or the batch with every group's
    # slots and pages then the scatters, or the separate kernels.
    plan = steps[0].fused_path()
    one_launch = plan in (api.STEP_ONE_LAUNCH, api.STEP_RANKED_ONE_LAUNCH)
    use_fused = fused_ms <= calls_ms
    ms = fused_ms if use_fused else calls_ms
    if use_fused and plan == api.STEP_RANKED_ONE_LAUNCH:
        path = "pkv_step (one launch, each workgroup ranking its own requests)"
    elif use_fused and one_launch:
        path = "pkv_step (one launch)"
    elif use_fused and plan == api.STEP_BATCH_THEN_SCATTER:
        path = "pkv_step (batch with slots and pages, then the scatters)"
    elif use_fused:
        path = "pkv_step (the separate kernels)"
    else:
        path = "three calls"
    context = context_figures(ab["total"], args.steps, args.warmup, stream)
    context["step_vs_copy"] = context["d2d_copy_same_bytes"]["ms"] / ms
    if use_fused and plan == api.STEP_RANKED_ONE_LAUNCH:
        kernel, launch_ms, kbytes, prof_key = ("pkv_step (k_prepare with the K/V write)", fused_ms,
                                               ab["total"], "ranked_step")
    elif use_fused and one_launch:
        kernel, launch_ms, kbytes, prof_key = "pkv_step (k_step)", fused_ms, ab["total"], "step"
    else:
        kernel = "scatter_kv (k_scatter)"
        launch_ms = statistics.fmean(split["scatter_kv"]) / ng
        kbytes = statistics.fmean(scatter_bytes_per_launch(b, gi) for b in batches
                                  for gi in range(ng))
        prof_key = "scatter_kv"
    achieved = kbytes / (launch_ms * 1e-3) / 1e9


    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic (seeded NumPy generator; K/V N(0,1) rounded to bf16)",
        "config": {
            "workload": batch.name, "requests": batch.n, "tokens": T,
            "block_size": [g.block_size for g in batch.groups],
            "num_blocks": [g.num_blocks for g in batch.groups],
            "kv_row": [f"{g.num_heads}x{g.head_dim} {g.dtype}" for g in batch.groups],
            "kv_groups": ng, "layers": 1, "rotating_batches": ROTATE,
        },
        "step": {
            "path": path,
            "algorithmic_bytes": ab["total"],
            "hbm_gbs": ab["total"] / (ms * 1e-3) / 1e9,
            "frac_of_peak": ab["total"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "wall_ms_per_step": fused_wall if use_fused else calls_wall,
        },
        "fused": {"ms_per_step": fused_ms, "tokens_per_s": T / (fused_ms * 1e-3)},
        "three_calls": {
            "ms_per_step": calls_ms, "tokens_per_s": T / (calls_ms * 1e-3),
            "per_call": {
                k: {"ms": statistics.fmean(v), "algorithmic_bytes": cb[k],
                    "gbs": cb[k] / (statistics.fmean(v) * 1e-3) / 1e9,
                    "frac_of_peak": cb[k] / (statistics.fmean(v) * 1e-3) / 1e9 / PEAK_HBM_GBS,
                    "bound": "hbm" if k == "scatter_kv" else "latency"}
                for k, v in split.items()},
            "per_call_note": "events between the calls; prepare and slot mapping move under "
                             "1 MB here, so their time is launch and memory latency",
        },
        "context": context,
        "state_calls": state,
        "variant_calls": variants,
        "gather_kv": gather,
        "prefix_cache": prefix,
        "hip_graph_replay": {
            "three_calls_ms_per_step": graph_ms["three_calls"],
            "fused_ms_per_step": graph_ms["fused"],
            "note": "each batch's step captured once in a HIP graph, replays back to back",
        },
        "host_wall_with_upload": {
            "us_median": statistics.median(upload_wall),
            "us_p10": statistics.quantiles(upload_wall, n=10)[0],
            "us_p90": statistics.quantiles(upload_wall, n=10)[-1],
            "note": "schedule (n x 8 bytes) copied from pinned host memory, pkv_step, "
                    "synchronize; host clock, one step at a time from an idle GPU",
        },
        "cold_single_step": {
            "reps": COLD_REPS,
            "ms_median": statistics.median(cold),
            "ms_p10": statistics.quantiles(cold, n=10)[0],
            "ms_p90": statistics.quantiles(cold, n=10)[-1],
            "lone_tiny_kernel_ms_median": statistics.median(lone),
            "note": "1 GiB rewrite before each step (L2 and Infinity Cache flushed); HIP "
                    "events around the one step, so each rep also carries the event and "
                    "dispatch latency of a lone launch (lone_tiny_kernel: the same protocol "
                    "around a one-element kernel)",
        },
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic_from_profile(prof_key, args.workload),
            "algorithmic_bytes_per_launch": kbytes,
            "launch_ms": launch_ms,
            "flushed_step": {
                "reps": COLD_REPS,
                "ms_median": statistics.median(cold),
                "ms_p10": statistics.quantiles(cold, n=10)[0],
                "ms_p90": statistics.quantiles(cold, n=10)[-1],
                "frac_median": ab["total"] / (statistics.median(cold) * 1e-3) / 1e9
                / PEAK_HBM_GBS,
                "frac_p10_time": ab["total"] / (statistics.quantiles(cold, n=10)[0] * 1e-3)
                / 1e9 / PEAK_HBM_GBS,
                "frac_p90_time": ab["total"] / (statistics.quantiles(cold, n=10)[-1] * 1e-3)
                / 1e9 / PEAK_HBM_GBS,
                "lone_tiny_kernel_ms_median": statistics.median(lone),
                "note": "the whole step's algorithmic bytes over single steps timed after a "
                        "1 GiB cache flush, HIP events around each (median of the reps); "
                        "lone_tiny_kernel: the same protocol around a one-element kernel, "
                        "the event and dispatch latency each rep carries",
            },
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
