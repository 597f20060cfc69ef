"""Shared helpers of the GPU parity tests: run the HIP path on a workloads.Batch
and compare every output with the CPU oracle on the same inputs."""
import sys

import numpy as np

import oracle

SENTINEL16 = -1          # int16 all-ones = 0xFFFF: a NaN in fp16 and bf16, never in the payload


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_step(batch, **kw):
    import torch  # noqa: F401  (loads the HIP runtime before the library)
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    groups = [GroupSpec(g.block_table, g.block_size, g.num_blocks, g.k, g.v) for g in batch.groups]
    return DeviceStep(batch.sched_rows, batch.num_scheduled, batch.completed, batch.token_ids,
                      groups, cache_fill=SENTINEL16, ibt_fill=oracle.IBT_UNWRITTEN, **kw)


def assert_equal(name, got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, (f"{name}: {bad.size} mismatches, first at flat index {bad[0]}: "
                           f"got {got.reshape(-1)[bad[0]]} want {want.reshape(-1)[bad[0]]}")


def compare_indices(step, prep, groups_o):
    for key in ("index_mapping", "query_start_loc", "seq_lens", "positions", "input_ids"):
        if getattr(step, key) is not None:
            assert_equal(key, step.host(key), prep[key])
    for gi, go in enumerate(groups_o):
        assert_equal(f"g{gi} slot_mapping", step.host("slot_mapping", gi), go["slot_mapping"])
        if step.groups[gi]["input_block_tables"] is not None:
            assert_equal(f"g{gi} input_block_tables", step.host("input_block_tables", gi),
                         go["input_block_tables"])


def compare_caches_full(step, groups_o):
    """Whole-cache comparison (small pools only)."""
    for gi, go in enumerate(groups_o):
        for key in ("k_cache", "v_cache"):
            got = step.host(key, gi).view(np.uint16)
            assert_equal(f"g{gi} {key}", got, go[key])


def compare_caches_at_slots(step, batch, groups_o):
    """Large pools: the oracle scatters into lazily mapped zero caches; compare the
    GPU rows at the oracle's written slots with the oracle's rows there, then
    check that the GPU cache holds exactly that many non-sentinel rows (so
    nothing was written anywhere else)."""
    import torch

    for gi, (g, go) in enumerate(zip(batch.groups, groups_o)):
        slots = go["slot_mapping"]
        written = np.unique(slots[slots >= 0])
        idx = torch.from_numpy(written.astype(np.int64)).to(step.device)
        for key in ("k_cache", "v_cache"):
            dev = step.groups[gi][key]
            rows = dev.index_select(0, idx).cpu().numpy().view(np.uint16)
            assert_equal(f"g{gi} {key} rows at written slots", rows, go[key][written])
            flat = dev.view(dev.shape[0], -1).view(torch.int64)
            nonsent = int((flat != -1).any(dim=1).sum().item())
            assert nonsent == written.size, f"g{gi} {key}: {nonsent} rows written, want {written.size}"


def oracle_chain(batch, lazy_caches=False):
    if not lazy_caches:
        return oracle.run_chain(batch)
    caches = []
    for g in batch.groups:
        caches.append((np.zeros((g.num_slots, g.num_heads, g.head_dim), np.uint16),
                       np.zeros((g.num_slots, g.num_heads, g.head_dim), np.uint16)))
    return oracle.run_chain(batch, caches=caches)
