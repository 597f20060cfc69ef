"""ctypes binding of libpagedkv: argument marshalling only.

Each function takes torch tensors (device memory), checks dtypes and shapes on
the host, passes raw pointers and sizes to the C entry point of the same name
(``pkv_*`` in include/pagedkv.h) on torch's current HIP stream, and raises
``PagedKVError`` on a non-zero return code.  ``prepared_<name>`` does the checks
and marshalling once and returns a ``launch(stream=None)`` function for loops
that repeat a call on the same tensors.  Nothing here computes any part of the
path.  The library is loaded at import; a missing library is an ImportError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import _abi
from ._abi import (EALIGN, EHIP, EINVAL, ENOMEM, ENOROWS, EUNSUPPORTED, MAX_BATCH, NO_BLOCK, OK,
                   ST_BITS, STEP_BATCH_THEN_SCATTER, STEP_MAX_BATCH, STEP_MAX_GROUPS,
                   STEP_ONE_LAUNCH, STEP_RANKED_MIN_BATCH, STEP_RANKED_ONE_LAUNCH, STEP_SEPARATE,
                   Group, PagedKVError, load_library)

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.environ.get("PAGEDKV_LIB", os.path.join(_HERE, "libpagedkv.so"))

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

_lib = load_library(library_path)


def abi_version() -> int:
    return int(_lib.pkv_abi_version())


def error_string(code: int) -> str:
    return _abi.error_string(_lib, code)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _idx(name: str, t: Optional[torch.Tensor], shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor on the GPU")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _tensors(obj):
    if isinstance(obj, torch.Tensor):
        yield obj
    elif isinstance(obj, dict):
        for v in obj.values():
            yield from _tensors(v)
    elif isinstance(obj, (list, tuple)):
        for v in obj:
            yield from _tensors(v)


def _prepared(name: str, fn, args: tuple, keep: tuple):
    """A launcher for one checked, marshalled call: ``launch(stream=None)``.
    ``keep`` holds the tensors whose pointers are baked into ``args``; they
    must all live on one GPU, and the call runs on that GPU's current stream
    (or on ``stream``, which must belong to it)."""
    devices = {t.device.index for t in _tensors(keep)}
    if len(devices) > 1:
        raise ValueError(f"{name}: tensors on several GPUs {sorted(devices)}")
    dev = devices.pop() if devices else torch.cuda.current_device()

    def launch(stream=None, _keep=keep):
        s = torch.cuda.current_stream(dev) if stream is None else stream
        # the null stream runs on the current device, any other on its own
        on = torch.cuda.current_device() if s.cuda_stream == 0 else s.device.index
        if on != dev:
            raise ValueError(f"{name}: the tensors are on cuda:{dev}, the stream runs on "
                             f"cuda:{on}")
        rc = fn(*args, s.cuda_stream)
        if rc != OK:
            raise PagedKVError(name, rc, _lib)

    launch.__name__ = f"prepared_{name}"
    return launch


def prepare_batch(sched_rows, num_scheduled, completed, token_ids, num_tokens, *, stream=None,
                  **outputs) -> None:
    """Batch assembly and flattening (pkv_prepare_batch); see prepared_prepare_batch."""
    prepared_prepare_batch(sched_rows, num_scheduled, completed, token_ids, num_tokens,
                           **outputs)(stream)


def prepared_prepare_batch(sched_rows: torch.Tensor, num_scheduled: torch.Tensor,
                           completed: torch.Tensor, token_ids: Optional[torch.Tensor],
                           num_tokens: int, *, index_mapping: torch.Tensor,
                           query_start_loc: torch.Tensor, seq_lens: torch.Tensor,
                           positions: torch.Tensor, input_ids: Optional[torch.Tensor] = None,
                           status: Optional[torch.Tensor] = None):
    """Batch assembly and flattening into caller-owned output tensors.

    sched_rows, num_scheduled: int32 [n]; completed: int32 [R]; token_ids: int32
    [R, L] with unit stride along L (row stride may be larger); num_tokens = T is
    the host's sum of num_scheduled.  Outputs: index_mapping [n],
    query_start_loc [n+1], seq_lens [n], positions [T], input_ids [T] (optional).
    """
    n = sched_rows.shape[0]
    T = int(num_tokens)
    _idx("sched_rows", sched_rows, (n,))
    _idx("num_scheduled", num_scheduled, (n,))
    _idx("completed", completed)
    _idx("index_mapping", index_mapping, (n,))
    _idx("query_start_loc", query_start_loc, (n + 1,))
    _idx("seq_lens", seq_lens, (n,))
    _idx("positions", positions, (T,))
    _idx("input_ids", input_ids, (T,), optional=True)
    R = completed.shape[0]
    L, stride = 0, 0
    if token_ids is not None:
        if token_ids.dtype != torch.int32 or not token_ids.is_cuda or token_ids.dim() != 2 \
                or token_ids.stride(1) != 1 or token_ids.shape[0] != R:
            raise ValueError("token_ids must be an int32 [R, L] GPU tensor with unit column stride")
        L, stride = token_ids.shape[1], token_ids.stride(0)
    elif input_ids is not None:
        raise ValueError("input_ids needs token_ids")
    if status is not None and (status.dtype != torch.int32 or not status.is_cuda
                               or status.numel() < 1):
        raise ValueError("status must be an int32 GPU tensor (bit pattern of a uint32)")
    args = (n, T, _ptr(sched_rows), _ptr(num_scheduled), _ptr(completed), R, _ptr(token_ids),
            stride, L, _ptr(index_mapping), _ptr(query_start_loc), _ptr(seq_lens),
            _ptr(positions), _ptr(input_ids), _ptr(status))
    return _prepared("prepare_batch", _lib.pkv_prepare_batch, args,
                     (sched_rows, num_scheduled, completed, token_ids, index_mapping,
                      query_start_loc, seq_lens, positions, input_ids, status))


def compute_slot_mapping(index_mapping, query_start_loc, seq_lens, positions, block_table,
                         block_size, num_blocks, *, stream=None, **outputs) -> None:
    """Write slots and visible pages of ONE KV-cache group (pkv_compute_slot_mapping);
    see prepared_compute_slot_mapping."""
    prepared_compute_slot_mapping(index_mapping, query_start_loc, seq_lens, positions,
                                  block_table, block_size, num_blocks, **outputs)(stream)


def prepared_compute_slot_mapping(index_mapping: torch.Tensor, query_start_loc: torch.Tensor,
                                  seq_lens: Optional[torch.Tensor], positions: torch.Tensor,
                                  block_table: torch.Tensor, block_size: int, num_blocks: int,
                                  *, slot_mapping: torch.Tensor,
                                  input_block_tables: Optional[torch.Tensor] = None,
                                  status: Optional[torch.Tensor] = None,
                                  sliding_window: int = 0):
    """Write slots (and optionally visible pages) of ONE KV-cache group.

    block_table: int32 [R, MB] contiguous; slot_mapping: int32 [T];
    input_block_tables: int32 [n, MB] or None; sliding_window: 0 for full
    attention, else the group's window (visible pages before every window of
    the step may then be -1 holes).
    """
    n = index_mapping.shape[0]
    T = positions.shape[0]
    _idx("index_mapping", index_mapping, (n,))
    _idx("query_start_loc", query_start_loc, (n + 1,))
    _idx("positions", positions, (T,))
    _idx("block_table", block_table)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [R, MB]")
    R, MB = block_table.shape
    _idx("slot_mapping", slot_mapping, (T,))
    _idx("input_block_tables", input_block_tables, (n, MB), optional=True)
    if input_block_tables is not None:
        _idx("seq_lens", seq_lens, (n,))
    args = (n, T, _ptr(index_mapping), _ptr(query_start_loc), _ptr(seq_lens), _ptr(positions),
            _ptr(block_table), R, MB, int(block_size), int(num_blocks), int(sliding_window),
            _ptr(slot_mapping), _ptr(input_block_tables), _ptr(status))
    return _prepared("compute_slot_mapping", _lib.pkv_compute_slot_mapping, args,
                     (index_mapping, query_start_loc, seq_lens, positions, block_table,
                      slot_mapping, input_block_tables, status))


def scatter_kv(k, v, k_cache, v_cache, slot_mapping, *, status=None, stream=None) -> None:
    """Write K/V rows at their slots (pkv_scatter_kv); see prepared_scatter_kv."""
    prepared_scatter_kv(k, v, k_cache, v_cache, slot_mapping, status=status)(stream)


def prepared_scatter_kv(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, slot_mapping: torch.Tensor, *,
                        status: Optional[torch.Tensor] = None):
    """Write token t's K/V rows to slot slot_mapping[t] of ONE group's caches.

    k, v: [T, ...] GPU tensors whose per-token rows are contiguous (the token
    stride may be larger, e.g. a view into a fused QKV buffer); k_cache, v_cache:
    contiguous [num_slots, ...] with the same row size.  Any dtype: the payload
    is copied bit for bit.
    """
    T = slot_mapping.shape[0]
    _idx("slot_mapping", slot_mapping, (T,))
    row_bytes, strides = _kv_layout("", k, v, k_cache, v_cache, T)
    args = (T, row_bytes, _ptr(k), strides[0], _ptr(v), strides[1], _ptr(k_cache), _ptr(v_cache),
            k_cache.shape[0], _ptr(slot_mapping), _ptr(status))
    return _prepared("scatter_kv", _lib.pkv_scatter_kv, args,
                     (k, v, k_cache, v_cache, slot_mapping, status))


def gather_kv(seq_lens, input_block_tables, block_size, num_blocks, k_cache, v_cache, *,
              stream=None, **outputs) -> None:
    """Read each request's KV range through its visible pages (pkv_gather_kv);
    see prepared_gather_kv."""
    prepared_gather_kv(seq_lens, input_block_tables, block_size, num_blocks, k_cache, v_cache,
                       **outputs)(stream)


def prepared_gather_kv(seq_lens: torch.Tensor, input_block_tables: torch.Tensor,
                       block_size: int, num_blocks: int, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, *, k_out: torch.Tensor, v_out: torch.Tensor,
                       kv_start: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None,
                       query_start_loc: Optional[torch.Tensor] = None, sliding_window: int = 0):
    """Copy positions 0 .. seq_len-1 of every batch row, read through its
    visible pages, to rows kv_start[b] + p of k_out / v_out (ONE group, ONE layer).

    seq_lens: int32 [n]; input_block_tables: int32 [n, MB]; k_cache, v_cache:
    contiguous [num_slots, ...] with num_slots >= num_blocks * block_size;
    k_out, v_out: [out_tokens, ...] with rows of the cache's size (contiguous
    rows, the token stride may be larger); kv_start: int32 [n+1] or None.
    sliding_window > 0 reads only the positions some new token attends
    (query_start_loc [n+1] is then required).
    """
    n = seq_lens.shape[0]
    _idx("seq_lens", seq_lens, (n,))
    _idx("input_block_tables", input_block_tables)
    if input_block_tables.dim() != 2 or input_block_tables.shape[0] != n:
        raise ValueError("input_block_tables must be [n, MB]")
    MB = input_block_tables.shape[1]
    _idx("kv_start", kv_start, (n + 1,), optional=True)
    _idx("query_start_loc", query_start_loc, (n + 1,), optional=not sliding_window)
    out_tokens = k_out.shape[0]
    row_bytes, (ks, vs) = _kv_layout("", k_out, v_out, k_cache, v_cache, out_tokens)
    if k_cache.shape[0] < int(num_blocks) * int(block_size):
        raise ValueError("the caches hold fewer than num_blocks * block_size slots")
    args = (n, _ptr(seq_lens), _ptr(query_start_loc), int(sliding_window),
            _ptr(input_block_tables), MB, int(block_size), int(num_blocks),
            row_bytes, _ptr(k_cache), _ptr(v_cache), out_tokens, _ptr(k_out), ks, _ptr(v_out), vs,
            _ptr(kv_start), _ptr(_status(status)))
    return _prepared("gather_kv", _lib.pkv_gather_kv, args,
                     (seq_lens, input_block_tables, k_cache, v_cache, k_out, v_out, kv_start,
                      status, query_start_loc))


def _kv_layout(name_k, k, v, k_cache, v_cache, T):
    """row_bytes and per-token byte strides of K/V (rows contiguous)."""
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not c.is_cuda or not c.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if v_cache.shape != k_cache.shape or v_cache.element_size() != k_cache.element_size():
        raise ValueError("k_cache and v_cache must have the same shape and element size")
    row_bytes = (k_cache.numel() // max(k_cache.shape[0], 1)) * k_cache.element_size() \
        if k_cache.dim() > 1 else k_cache.element_size()
    strides = []
    for name, x in (("k", k), ("v", v)):
        if not x.is_cuda or x.shape[0] != T:
            raise ValueError(f"{name_k}{name} must be a GPU tensor with {T} rows")
        if T and (x[0].numel() * x.element_size() != row_bytes or not x[0].is_contiguous()):
            raise ValueError(f"{name_k}{name} rows must be contiguous and {row_bytes} bytes")
        strides.append(x.stride(0) * x.element_size() if T else row_bytes)
    return row_bytes, strides


def step(sched_rows: torch.Tensor, num_scheduled: torch.Tensor, completed: torch.Tensor,
         token_ids: Optional[torch.Tensor], num_tokens: int, groups, *,
         index_mapping: torch.Tensor, query_start_loc: torch.Tensor, seq_lens: torch.Tensor,
         positions: torch.Tensor, input_ids: Optional[torch.Tensor] = None,
         status: Optional[torch.Tensor] = None, stream=None) -> None:
    """A whole step in one call (pkv_step): prepare_batch, then per group
    compute_slot_mapping and scatter_kv, with identical results.

    groups: sequence of dicts with keys block_table, block_size, num_blocks,
    slot_mapping, input_block_tables (or None), k, v, k_cache, v_cache, and
    optionally sliding_window (default 0, full attention).
    """
    prepared_step(sched_rows, num_scheduled, completed, token_ids, num_tokens, groups,
                  index_mapping=index_mapping, query_start_loc=query_start_loc,
                  seq_lens=seq_lens, positions=positions, input_ids=input_ids,
                  status=status)(stream)


def prepared_step(sched_rows: torch.Tensor, num_scheduled: torch.Tensor, completed: torch.Tensor,
                  token_ids: Optional[torch.Tensor], num_tokens: int, groups, *,
                  index_mapping: torch.Tensor, query_start_loc: torch.Tensor,
                  seq_lens: torch.Tensor, positions: torch.Tensor,
                  input_ids: Optional[torch.Tensor] = None,
                  status: Optional[torch.Tensor] = None):
    """Check and marshal the arguments of ``step`` once; return a function
    ``launch(stream=None)`` that enqueues pkv_step with them.  ``launch.path``
    is the launch plan pkv_step takes for them (pkv_step_path: STEP_ONE_LAUNCH,
    STEP_RANKED_ONE_LAUNCH, STEP_BATCH_THEN_SCATTER or STEP_SEPARATE).  For loops that
    repeat a step on the same buffers (new contents, same tensors), this keeps
    the host's per-step cost to one foreign call.  The tensors must stay alive
    and unmoved while the returned function is used."""
    n = sched_rows.shape[0]
    T = int(num_tokens)
    _idx("sched_rows", sched_rows, (n,))
    _idx("num_scheduled", num_scheduled, (n,))
    _idx("completed", completed)
    _idx("index_mapping", index_mapping, (n,))
    _idx("query_start_loc", query_start_loc, (n + 1,))
    _idx("seq_lens", seq_lens, (n,))
    _idx("positions", positions, (T,))
    _idx("input_ids", input_ids, (T,), optional=True)
    R = completed.shape[0]
    L, stride = 0, 0
    if token_ids is not None:
        if token_ids.dtype != torch.int32 or not token_ids.is_cuda or token_ids.dim() != 2 \
                or token_ids.stride(1) != 1 or token_ids.shape[0] != R:
            raise ValueError("token_ids must be an int32 [R, L] GPU tensor with unit column stride")
        L, stride = token_ids.shape[1], token_ids.stride(0)
    elif input_ids is not None:
        raise ValueError("input_ids needs token_ids")
    arr = (Group * max(len(groups), 1))()
    for i, g in enumerate(groups):
        bt = _idx(f"groups[{i}].block_table", g["block_table"])
        if bt.dim() != 2 or bt.shape[0] != R:
            raise ValueError(f"groups[{i}].block_table must be [R, MB]")
        MB = bt.shape[1]
        _idx(f"groups[{i}].slot_mapping", g["slot_mapping"], (T,))
        _idx(f"groups[{i}].input_block_tables", g.get("input_block_tables"), (n, MB),
             optional=True)
        row_bytes, (ks, vs) = _kv_layout(f"groups[{i}].", g["k"], g["v"], g["k_cache"],
                                         g["v_cache"], T)
        arr[i] = Group(bt.data_ptr(), g["slot_mapping"].data_ptr(),
                       _ptr(g.get("input_block_tables")), g["k"].data_ptr(), g["v"].data_ptr(),
                       g["k_cache"].data_ptr(), g["v_cache"].data_ptr(), ks, vs,
                       g["k_cache"].shape[0], row_bytes, MB, int(g["block_size"]),
                       int(g["num_blocks"]), int(g.get("sliding_window", 0)))
    args = (n, T, _ptr(sched_rows), _ptr(num_scheduled), _ptr(completed), R, _ptr(token_ids),
            stride, L, _ptr(index_mapping), _ptr(query_start_loc), _ptr(seq_lens),
            _ptr(positions), _ptr(input_ids), len(groups), arr, _ptr(status))
    launch = _prepared("step", _lib.pkv_step, args,
                       (sched_rows, num_scheduled, completed, token_ids, index_mapping,
                        query_start_loc, seq_lens, positions, input_ids, status, list(groups),
                        arr))
    # the launch plan the library takes for these arguments (pkv_step_path)
    launch.path = _lib.pkv_step_path(n, T, len(groups), arr)
    if launch.path < 0:
        raise PagedKVError("step_path", launch.path, _lib)
    return launch


# -- persistent request state -------------------------------------------------
def _token_table(token_ids: torch.Tensor, R: int):
    if token_ids.dtype != torch.int32 or not token_ids.is_cuda or token_ids.dim() != 2 \
            or token_ids.stride(1) != 1 or token_ids.shape[0] != R:
        raise ValueError("token_ids must be an int32 [R, L] GPU tensor with unit column stride")
    return token_ids.shape[1], token_ids.stride(0)


def _block_table(block_table: torch.Tensor, R: int):
    _idx("block_table", block_table)
    if block_table.dim() != 2 or block_table.shape[0] != R:
        raise ValueError("block_table must be [R, MB]")
    return block_table.shape[1]


def _status(status):
    if status is not None and (status.dtype != torch.int32 or not status.is_cuda
                               or status.numel() < 1):
        raise ValueError("status must be an int32 GPU tensor (bit pattern of a uint32)")
    return status


def add_requests(rows, num_computed, prompt_start, prompt_tokens, block_start, blocks, *,
                 stream=None, **state) -> None:
    """add_request for m new requests (pkv_add_requests); see prepared_add_requests."""
    prepared_add_requests(rows, num_computed, prompt_start, prompt_tokens, block_start, blocks,
                          **state)(stream)


def prepared_add_requests(rows: torch.Tensor, num_computed: torch.Tensor,
                          prompt_start: torch.Tensor, prompt_tokens: torch.Tensor,
                          block_start: torch.Tensor, blocks: torch.Tensor, *,
                          completed: torch.Tensor, token_ids: torch.Tensor,
                          block_table: torch.Tensor, row_blocks: torch.Tensor,
                          status: Optional[torch.Tensor] = None):
    """Register m requests in the persistent state.

    rows, num_computed: int32 [m]; prompts and block ids as CSR lists:
    prompt_start [m+1] into prompt_tokens (flat int32), block_start [m+1] into
    blocks (flat int32).  State (updated in place): completed [R], token_ids
    [R, L], block_table [R, MB], row_blocks [R].
    """
    m = rows.shape[0]
    _idx("rows", rows, (m,))
    _idx("num_computed", num_computed, (m,))
    _idx("prompt_start", prompt_start, (m + 1,))
    _idx("prompt_tokens", prompt_tokens)
    _idx("block_start", block_start, (m + 1,))
    _idx("blocks", blocks)
    _idx("completed", completed)
    R = completed.shape[0]
    _idx("row_blocks", row_blocks, (R,))
    L, stride = _token_table(token_ids, R)
    MB = _block_table(block_table, R)
    args = (m, _ptr(rows), _ptr(num_computed), _ptr(prompt_start), _ptr(prompt_tokens),
            prompt_tokens.numel(), _ptr(block_start), _ptr(blocks), blocks.numel(), R,
            _ptr(completed), _ptr(token_ids), stride, L, _ptr(block_table), MB, _ptr(row_blocks),
            _ptr(_status(status)))
    return _prepared("add_requests", _lib.pkv_add_requests, args,
                     (rows, num_computed, prompt_start, prompt_tokens, block_start, blocks,
                      completed, token_ids, block_table, row_blocks, status))


def append_blocks(rows, block_start, blocks, *, stream=None, **state) -> None:
    """update_request: append new block ids (pkv_append_blocks); see prepared_append_blocks."""
    prepared_append_blocks(rows, block_start, blocks, **state)(stream)


def prepared_append_blocks(rows: torch.Tensor, block_start: torch.Tensor, blocks: torch.Tensor,
                           *, block_table: torch.Tensor, row_blocks: torch.Tensor,
                           status: Optional[torch.Tensor] = None):
    """Append each request's newly allocated block ids (CSR: block_start [m+1]
    into blocks) after the row_blocks[row] entries its block-table row holds."""
    m = rows.shape[0]
    _idx("rows", rows, (m,))
    _idx("block_start", block_start, (m + 1,))
    _idx("blocks", blocks)
    _idx("row_blocks", row_blocks)
    R = row_blocks.shape[0]
    MB = _block_table(block_table, R)
    args = (m, _ptr(rows), _ptr(block_start), _ptr(blocks), blocks.numel(), R, _ptr(block_table),
            MB, _ptr(row_blocks), _ptr(_status(status)))
    return _prepared("append_blocks", _lib.pkv_append_blocks, args,
                     (rows, block_start, blocks, block_table, row_blocks, status))


def advance_state(index_mapping, seq_lens, sampled=None, *, stream=None, **state) -> None:
    """After a step (pkv_advance_state); see prepared_advance_state."""
    prepared_advance_state(index_mapping, seq_lens, sampled, **state)(stream)


def prepared_advance_state(index_mapping: torch.Tensor, seq_lens: torch.Tensor,
                           sampled: Optional[torch.Tensor] = None, *, completed: torch.Tensor,
                           token_ids: Optional[torch.Tensor] = None,
                           status: Optional[torch.Tensor] = None):
    """completed[index_mapping[b]] = seq_lens[b]; sampled[b] >= 0 is appended
    to the row's token list at position seq_lens[b].  index_mapping, seq_lens,
    sampled: int32 [n] (the batch order of prepare_batch); token_ids [R, L] is
    needed with sampled."""
    n = index_mapping.shape[0]
    _idx("index_mapping", index_mapping, (n,))
    _idx("seq_lens", seq_lens, (n,))
    _idx("sampled", sampled, (n,), optional=True)
    _idx("completed", completed)
    R = completed.shape[0]
    L, stride = 0, 0
    if token_ids is not None:
        L, stride = _token_table(token_ids, R)
    elif sampled is not None:
        raise ValueError("sampled needs token_ids")
    args = (n, _ptr(index_mapping), _ptr(seq_lens), _ptr(sampled), R, _ptr(completed),
            _ptr(token_ids), stride, L, _ptr(_status(status)))
    return _prepared("advance_state", _lib.pkv_advance_state, args,
                     (index_mapping, seq_lens, sampled, completed, token_ids, status))


class RowPool(_abi.RowPool):
    """Host-side pool of request_state_index rows (pkv_row_pool_*): ``acquire(m)``
    hands out m free rows (the most recently released first), ``release(rows)``
    takes rows back.  Both raise PagedKVError and change nothing on failure."""

    def __init__(self, R: int):
        super().__init__(R, _lib)


# -- prefix-cache block hashes and the prefix index ---------------------------
def _i64t(name: str, t: Optional[torch.Tensor], shape=None, optional=False):
    """A contiguous int64 GPU tensor (64-bit hashes travel as int64 bit patterns)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype != torch.int64 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int64 tensor on the GPU")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _index(keys, vals):
    _i64t("keys", keys)
    _idx("vals", vals, tuple(keys.shape))
    if keys.dim() != 1 or (keys.numel() & (keys.numel() - 1)) != 0:
        raise ValueError("the index capacity must be a power of two (1-D keys)")
    return keys.numel()


def hash_blocks(tokens, starts, lengths, block_size, *, hashes, num_full=None, status=None,
                stream=None) -> None:
    """Chained hashes of every full block of m token lists (pkv_hash_blocks).

    tokens: flat int32 GPU tensor; list b is tokens[starts[b] : starts[b] +
    lengths[b]] (starts int64 [m], lengths int32 [m]); hashes: int64 [m, MB]
    (uint64 bit patterns); num_full: int32 [m] or None."""
    m = lengths.shape[0]
    _idx("tokens", tokens)
    _i64t("starts", starts, (m,))
    _idx("lengths", lengths, (m,))
    _i64t("hashes", hashes)
    if hashes.dim() != 2 or hashes.shape[0] != m:
        raise ValueError("hashes must be [m, MB]")
    _idx("num_full", num_full, (m,), optional=True)
    args = (m, _ptr(tokens), tokens.numel(), _ptr(starts), _ptr(lengths), int(block_size),
            hashes.shape[1], _ptr(hashes), _ptr(num_full), _ptr(_status(status)))
    _prepared("hash_blocks", _lib.pkv_hash_blocks, args,
              (tokens, starts, lengths, hashes, num_full, status))(stream)


def prefix_clear(keys, vals, *, stream=None) -> None:
    """Empty the prefix index (pkv_prefix_clear)."""
    cap = _index(keys, vals)
    args = (_ptr(keys), _ptr(vals), cap)
    _prepared("prefix_clear", _lib.pkv_prefix_clear, args, (keys, vals))(stream)


def prefix_lookup(hashes, lengths, block_size, keys, vals, *, num_computed, hit_blocks=None,
                  status=None, stream=None) -> None:
    """Longest cached run of leading full blocks per request (pkv_prefix_lookup)."""
    m = lengths.shape[0]
    _i64t("hashes", hashes)
    if hashes.dim() != 2 or hashes.shape[0] != m:
        raise ValueError("hashes must be [m, MB]")
    MB = hashes.shape[1]
    _idx("lengths", lengths, (m,))
    _idx("num_computed", num_computed, (m,))
    _idx("hit_blocks", hit_blocks, (m, MB), optional=True)
    cap = _index(keys, vals)
    args = (m, _ptr(hashes), MB, _ptr(lengths), int(block_size), _ptr(keys), _ptr(vals), cap,
            _ptr(hit_blocks), _ptr(num_computed), _ptr(_status(status)))
    _prepared("prefix_lookup", _lib.pkv_prefix_lookup, args,
              (hashes, lengths, keys, vals, hit_blocks, num_computed, status))(stream)


def prefix_insert(hashes, lo, hi, rows, block_table, keys, vals, *, status=None,
                  stream=None) -> None:
    """Register blocks [lo[b], hi[b]) of each request (pkv_prefix_insert)."""
    m = rows.shape[0]
    _i64t("hashes", hashes)
    if hashes.dim() != 2 or hashes.shape[0] != m:
        raise ValueError("hashes must be [m, MB]")
    MB = hashes.shape[1]
    for name, t in (("lo", lo), ("hi", hi), ("rows", rows)):
        _idx(name, t, (m,))
    _idx("block_table", block_table)
    if block_table.dim() != 2 or block_table.shape[1] != MB:
        raise ValueError("block_table must be [R, MB] with the hashes' MB")
    cap = _index(keys, vals)
    args = (m, _ptr(hashes), MB, _ptr(lo), _ptr(hi), _ptr(rows), _ptr(block_table),
            block_table.shape[0], _ptr(keys), _ptr(vals), cap, _ptr(_status(status)))
    _prepared("prefix_insert", _lib.pkv_prefix_insert, args,
              (hashes, lo, hi, rows, block_table, keys, vals, status))(stream)


def prefix_evict(hashes, blocks, keys, vals, *, stream=None) -> None:
    """Drop entries hashes[i] -> blocks[i] (pkv_prefix_evict)."""
    count = hashes.numel()
    _i64t("hashes", hashes)
    _idx("blocks", blocks)
    if blocks.numel() != count:
        raise ValueError("hashes and blocks must have the same length")
    cap = _index(keys, vals)
    args = (count, _ptr(hashes), _ptr(blocks), _ptr(keys), _ptr(vals), cap)
    _prepared("prefix_evict", _lib.pkv_prefix_evict, args, (hashes, blocks, keys, vals))(stream)


# -- allocation-side variants: sliding-window holes, speculative lookahead ------
def window_free(rows, completed, block_table, block_size, sliding_window, *, freed, num_freed,
                status=None, stream=None) -> None:
    """Release the blocks wholly before every window (pkv_window_free); see
    prepared_window_free."""
    prepared_window_free(rows, completed, block_table, block_size, sliding_window, freed=freed,
                         num_freed=num_freed, status=status)(stream)


def prepared_window_free(rows, completed, block_table, block_size, sliding_window, *, freed,
                         num_freed, status=None):
    """Release the blocks wholly before every window: block_table [R, MB] is
    updated in place (freed entries become -1), freed [m, MB] lists each row's
    released ids in block order, num_freed [m] counts them."""
    m = rows.shape[0]
    _idx("rows", rows, (m,))
    _idx("completed", completed)
    R = completed.shape[0]
    _idx("block_table", block_table)
    if block_table.dim() != 2 or block_table.shape[0] != R:
        raise ValueError("block_table must be [R, MB]")
    MB = block_table.shape[1]
    _idx("freed", freed, (m, MB))
    _idx("num_freed", num_freed, (m,))
    args = (m, _ptr(rows), _ptr(completed), _ptr(block_table), R, MB, int(block_size),
            int(sliding_window), _ptr(freed), _ptr(num_freed), _ptr(_status(status)))
    return _prepared("window_free", _lib.pkv_window_free, args,
                     (rows, completed, block_table, freed, num_freed, status))


def lookahead_slots(index_mapping, seq_lens, block_table, block_size, num_blocks, *, out,
                    status=None, stream=None) -> None:
    """Slots of the positions after each request's seq_len (pkv_lookahead_slots);
    see prepared_lookahead_slots."""
    prepared_lookahead_slots(index_mapping, seq_lens, block_table, block_size, num_blocks,
                             out=out, status=status)(stream)


def prepared_lookahead_slots(index_mapping, seq_lens, block_table, block_size, num_blocks, *, out,
                             status=None):
    """Slots of the k = out.shape[1] positions after each request's seq_len."""
    n = index_mapping.shape[0]
    _idx("index_mapping", index_mapping, (n,))
    _idx("seq_lens", seq_lens, (n,))
    _idx("block_table", block_table)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [R, MB]")
    R, MB = block_table.shape
    _idx("out", out)
    if out.dim() != 2 or out.shape[0] != n:
        raise ValueError("out must be [n, k]")
    args = (n, _ptr(index_mapping), _ptr(seq_lens), _ptr(block_table), R, MB, int(block_size),
            int(num_blocks), out.shape[1], _ptr(out), _ptr(_status(status)))
    return _prepared("lookahead_slots", _lib.pkv_lookahead_slots, args,
                     (index_mapping, seq_lens, block_table, out, status))


def blocks_needed(rows, num_new, k, block_size, completed, row_blocks, *, need, status=None,
                  stream=None) -> None:
    """New blocks each request needs (pkv_blocks_needed); see prepared_blocks_needed."""
    prepared_blocks_needed(rows, num_new, k, block_size, completed, row_blocks, need=need,
                           status=status)(stream)


def prepared_blocks_needed(rows, num_new, k, block_size, completed, row_blocks, *, need,
                           status=None):
    """New blocks each request needs for its new and k lookahead tokens."""
    n = rows.shape[0]
    _idx("rows", rows, (n,))
    _idx("num_new", num_new, (n,))
    _idx("completed", completed)
    R = completed.shape[0]
    _idx("row_blocks", row_blocks, (R,))
    _idx("need", need, (n,))
    args = (n, _ptr(rows), _ptr(num_new), int(k), int(block_size), _ptr(completed),
            _ptr(row_blocks), R, _ptr(need), _ptr(_status(status)))
    return _prepared("blocks_needed", _lib.pkv_blocks_needed, args,
                     (rows, num_new, completed, row_blocks, need, status))
