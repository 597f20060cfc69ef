"""Benchmark of one step of the paged-KV input path on one MI355X.

A step is the whole path on one synthetic batch: prepare_batch, then for every
KV-cache group compute_slot_mapping and scatter_kv (one layer), on one stream
with every input already resident in HBM.  Default workload: 16 requests x
2048 new tokens (32768 tokens) from an empty history, block size 32, a
131072-block pool, K/V of 8 heads x 128 in bf16.

Timing: W untimed warm-up steps, then exactly K timed steps.  Before each
timed step a 1 GiB buffer is rewritten (outside the timed interval) so the
step starts with L2 and the 256 MB Infinity Cache holding none of its data;
HIP events recorded on the launch stream around each call give the per-call
and per-step device times.  The whole K-step loop is bracketed by
torch.cuda.synchronize() on both sides.

Prints one JSON line (rank 0, N = 1 only: this build runs on one GPU).
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


def scatter_bytes_per_launch(batch, gi):
    """Algorithmic bytes of one scatter_kv launch: per token, read K and V rows,
    write both cache rows, read the slot (4 * row_bytes + 4)."""
    g = batch.groups[gi]
    return batch.T * (4 * g.row_bytes + 4)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel, workload, kernel_src):
    """HBM bytes per launch of the kernel from the committed rocprofv3 counter
    summary, when it was taken on the kernel's current source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_b) or m_src.group(1) != source_digest(kernel_src):
        return None
    return float(m_b.group(1))


def cpu_baseline(batch, budget_s):
    """The CPU oracle, as it stands, on the same step: prepare, slots and the
    scatter into lazily mapped host caches, repeated for about budget_s."""
    import numpy as np
    import oracle

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
    return dict(value=batch.T * reps / el, unit="tokens/s", cores=1, kind="oracle",
                sample=f"the full {batch.name} step (T={batch.T}) repeated {reps} times, "
                       f"{el:.1f} s on one host thread (plain C oracle, gcc -O2)",
                seconds=el, reps=reps)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_16x2048")
    ap.add_argument("--no-flush", action="store_true", help="back-to-back steps (warm caches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch a plain 256 MiB device copy (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    torch.cuda.set_device(0)
    batch = workloads.make(args.workload)
    groups = [GroupSpec(g.block_table, g.block_size, g.num_blocks, g.k, g.v) for g in batch.groups]
    step = DeviceStep(batch.sched_rows, batch.num_scheduled, batch.completed, batch.token_ids,
                      groups)
    stream = torch.cuda.current_stream()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    print(f"[bench] {batch.name}: n={batch.n} T={batch.T} groups={len(batch.groups)}",
          file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            flush.fill_(1)
            dst.copy_(src)
        torch.cuda.synchronize()

    ng = len(batch.groups)

    def timed(run_fn, marks):
        """W warm-up steps, then exactly K timed steps (cache flush before each,
        outside the events); returns per-step lists of event intervals."""
        for _ in range(args.warmup):
            if not args.no_flush:
                flush.fill_(1)
            run_fn(None)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)]
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(args.steps):
            if not args.no_flush:
                flush.fill_(1)
            run_fn(ev[i])
        torch.cuda.synchronize()
        return ev, time.perf_counter() - w0

    def calls(e):
        # prepare_batch | compute_slot_mapping per group | scatter_kv per group
        if e is not None:
            e[0].record(stream)
        step.prepare(stream)
        if e is not None:
            e[1].record(stream)
        for gi in range(ng):
            step.slots(gi, stream)
        if e is not None:
            e[2].record(stream)
        for gi in range(ng):
            step.scatter(gi, stream)
        if e is not None:
            e[3].record(stream)

    def fused(e):
        if e is not None:
            e[0].record(stream)
        step.run_fused(stream)
        if e is not None:
            e[1].record(stream)

    ev_c, wall_c = timed(calls, 4)
    ev_f, wall_f = timed(fused, 2)
    if step.status_bits() != 0:
        raise RuntimeError(f"device status bits set: {step.status_bits():#x}")

    calls_ms = [e[0].elapsed_time(e[3]) for e in ev_c]
    prep_ms = [e[0].elapsed_time(e[1]) for e in ev_c]
    slot_ms = [e[1].elapsed_time(e[2]) for e in ev_c]
    scat_ms = [e[2].elapsed_time(e[3]) for e in ev_c]
    fused_ms = [e[0].elapsed_time(e[1]) for e in ev_f]
    T = batch.T
    ab = algorithmic_bytes(batch)
    use_fused = statistics.fmean(fused_ms) <= statistics.fmean(calls_ms)
    step_ms = fused_ms if use_fused else calls_ms
    ms = statistics.fmean(step_ms)

    # Dominant kernel: the one launch of the fused step (all of the step's
    # bytes), or scatter_kv when the separate calls are faster.
    if use_fused:
        kernel, launch_ms, kbytes = "pkv_step (k_step)", ms, ab["total"]
        src = os.path.join(ROOT, "paged_kv_input_amd", "csrc", "step.hip")
        prof_key = "step"
    else:
        kernel = "scatter_kv (k_scatter)"
        launch_ms = statistics.fmean(scat_ms) / ng
        kbytes = statistics.fmean(scatter_bytes_per_launch(batch, gi) for gi in range(ng))
        src = os.path.join(ROOT, "paged_kv_input_amd", "csrc", "scatter.hip")
        prof_key = "scatter_kv"
    achieved = kbytes / (launch_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(prof_key, args.workload, src)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(batch, args.cpu_seconds)

    g0 = batch.groups[0]
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
            "kv_groups": ng, "layers": 1,
            "cache_state": "cold (1 GiB rewrite before each step)" if not args.no_flush else "warm",
        },
        "step": {
            "path": "pkv_step (one launch)" if use_fused else "three calls",
            "algorithmic_bytes": ab["total"],
            "hbm_gbs": ab["total"] / (ms * 1e-3) / 1e9,
            "frac_of_peak": ab["total"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "ms_median": statistics.median(step_ms),
            "ms_p10": sorted(step_ms)[len(step_ms) // 10],
            "ms_p90": sorted(step_ms)[(9 * len(step_ms)) // 10],
            "wall_ms_per_step_incl_flush": (wall_f if use_fused else wall_c) * 1e3 / args.steps,
        },
        "three_calls": {
            "ms_per_step": statistics.fmean(calls_ms),
            "tokens_per_s": T / (statistics.fmean(calls_ms) * 1e-3),
            "prepare_batch_ms": statistics.fmean(prep_ms),
            "compute_slot_mapping_ms": statistics.fmean(slot_ms),
            "scatter_kv_ms": statistics.fmean(scat_ms),
            "scatter_kv_gbs": statistics.fmean(scatter_bytes_per_launch(batch, gi)
                                               for gi in range(ng)) * ng
            / (statistics.fmean(scat_ms) * 1e-3) / 1e9,
        },
        "fused": {
            "ms_per_step": statistics.fmean(fused_ms),
            "tokens_per_s": T / (statistics.fmean(fused_ms) * 1e-3),
        },
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kbytes,
            "launch_ms": launch_ms,
        },
        "cpu_baseline": ({k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")}
                         if cpu else None),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
