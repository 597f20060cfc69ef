"""paged_kv_input_amd -- MI355X (gfx950) library for one inference step's flat
input tensors and the paged K/V write.

The work runs in hand-written HIP kernels behind a C ABI (``libpagedkv.so``,
declared in ``include/pagedkv.h``).  This package is a thin binding with the
same call names: ``prepare_batch``, ``compute_slot_mapping`` (one call per
KV-cache group), ``scatter_kv`` (one call per group and layer) and ``step``
(all of them for a step's first layer, in one launch), the read side
``gather_kv`` (each request's KV range through its visible pages), the
prefix-cache block hashes and index (``hash_blocks``, ``prefix_*``), the
sliding-window and speculative-lookahead variants (``window_free``,
``lookahead_slots``, ``blocks_needed``), the persistent
request-state updates ``add_requests``, ``append_blocks`` and
``advance_state`` and the host-side ``RowPool`` that hands out state rows.  It takes
torch tensors for device memory and uses torch's current HIP stream; every
step of the path runs in the library's kernels.  Importing an entry point loads
the library and raises if it is missing -- there is no CPU fallback.
"""
from __future__ import annotations

_API = ("prepare_batch", "compute_slot_mapping", "scatter_kv", "step", "gather_kv",
        "hash_blocks", "prefix_clear", "prefix_lookup", "prefix_insert", "prefix_evict",
        "window_free", "lookahead_slots", "blocks_needed",
        "NO_BLOCK",
        "prepared_gather_kv", "add_requests",
        "append_blocks", "advance_state", "prepared_prepare_batch",
        "prepared_compute_slot_mapping", "prepared_scatter_kv", "prepared_step",
        "prepared_add_requests", "prepared_append_blocks", "prepared_advance_state",
        "RowPool", "PagedKVError",
        "library_path", "abi_version", "error_string", "load_library", "ST_BITS", "MAX_BATCH",
        "STEP_MAX_BATCH", "STEP_MAX_GROUPS")

__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
