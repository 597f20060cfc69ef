"""One step of the path on the GPU: prepare_batch, then per KV-cache group
compute_slot_mapping and scatter_kv, into device buffers this object owns.

It only allocates and holds torch tensors and calls the library's three entry
points in order on one stream; every computation runs in the HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import api


@dataclass
class GroupSpec:
    """Host description of one KV-cache group for a step."""

    block_table: np.ndarray     # int32 [R, MB] (or a device tensor, used in place)
    block_size: int
    num_blocks: int
    k: np.ndarray               # [T, H, D] payload words (any dtype, copied as bits)
    v: np.ndarray
    sliding_window: int = 0     # 0: full attention


class DeviceStep:
    """Device-resident inputs, outputs and paged caches for one step."""

    def __init__(self, sched_rows, num_scheduled, completed, token_ids,
                 groups: Sequence[GroupSpec], *, device="cuda", cache_fill: Optional[int] = None,
                 ibt_fill: Optional[int] = None, with_input_ids: bool = True,
                 with_block_tables: bool = True, num_tokens: Optional[int] = None,
                 caches: Optional[Sequence] = None):
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())

        def up(a, dtype=None):
            if isinstance(a, torch.Tensor):      # already on the device (e.g. DeviceState's)
                if a.device != dev or (dtype is not None and a.dtype != dtype):
                    raise ValueError("device tensors must be on the step's device")
                return a
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype is not None:
                t = t.to(dtype)
            return t.to(dev)

        def as_i32(a):
            return up(a, torch.int32) if isinstance(a, torch.Tensor) else up(np.asarray(a, np.int32))

        self.device = dev
        self.sched_rows = as_i32(sched_rows)
        self.num_scheduled = as_i32(num_scheduled)
        self.completed = as_i32(completed)
        self.token_ids = as_i32(token_ids) if with_input_ids else None
        self.n = int(self.sched_rows.shape[0])
        if num_tokens is None:
            if isinstance(num_scheduled, torch.Tensor):
                raise ValueError("num_tokens is required when num_scheduled is a device tensor")
            num_tokens = int(np.maximum(np.asarray(num_scheduled, np.int64), 0).sum())
        self.T = int(num_tokens)
        i32 = dict(dtype=torch.int32, device=dev)
        self.index_mapping = torch.empty(self.n, **i32)
        self.query_start_loc = torch.empty(self.n + 1, **i32)
        self.seq_lens = torch.empty(self.n, **i32)
        self.positions = torch.empty(self.T, **i32)
        self.input_ids = torch.empty(self.T, **i32) if with_input_ids else None
        self.status = torch.zeros(1, **i32)
        self.groups: List[dict] = []
        self._fused = None
        self._prep = None
        for g in groups:
            bt = as_i32(g.block_table)
            k = up(np.ascontiguousarray(g.k).view(np.int16))
            v = up(np.ascontiguousarray(g.v).view(np.int16))
            row_shape = tuple(k.shape[1:])
            num_slots = int(g.num_blocks) * int(g.block_size)
            if caches is not None:       # shared with another step (same pool and layout)
                kc, vc = caches[len(self.groups)]
                assert kc.shape == (num_slots, *row_shape) and kc.dtype == k.dtype
            else:
                kc = torch.empty((num_slots, *row_shape), dtype=k.dtype, device=dev)
                vc = torch.empty((num_slots, *row_shape), dtype=k.dtype, device=dev)
            if cache_fill is not None:
                kc.fill_(cache_fill)
                vc.fill_(cache_fill)
            ibt = None
            if with_block_tables:
                ibt = torch.empty((self.n, bt.shape[1]), **i32)
                if ibt_fill is not None:
                    ibt.fill_(ibt_fill)
            self.groups.append(dict(block_table=bt, block_size=int(g.block_size),
                                    num_blocks=int(g.num_blocks),
                                    sliding_window=int(g.sliding_window), k=k, v=v, k_cache=kc,
                                    v_cache=vc, slot_mapping=torch.empty(self.T, **i32),
                                    input_block_tables=ibt))

    # -- the three calls (arguments checked and marshalled once, then reused) -----
    def prepare(self, stream=None):
        if self._prep is None:
            self._prep = api.prepared_prepare_batch(
                self.sched_rows, self.num_scheduled, self.completed, self.token_ids, self.T,
                index_mapping=self.index_mapping, query_start_loc=self.query_start_loc,
                seq_lens=self.seq_lens, positions=self.positions, input_ids=self.input_ids,
                status=self.status)
        self._prep(stream)

    def slots(self, gi: int, stream=None):
        g = self.groups[gi]
        if g.get("_slots") is None:
            g["_slots"] = api.prepared_compute_slot_mapping(
                self.index_mapping, self.query_start_loc, self.seq_lens, self.positions,
                g["block_table"], g["block_size"], g["num_blocks"],
                slot_mapping=g["slot_mapping"], input_block_tables=g["input_block_tables"],
                status=self.status, sliding_window=g["sliding_window"])
        g["_slots"](stream)

    def scatter(self, gi: int, stream=None):
        g = self.groups[gi]
        if g.get("_scatter") is None:
            g["_scatter"] = api.prepared_scatter_kv(g["k"], g["v"], g["k_cache"], g["v_cache"],
                                                    g["slot_mapping"], status=self.status)
        g["_scatter"](stream)

    def run(self, stream=None):
        """One whole step: prepare, then every group's slots and scatter."""
        self.prepare(stream)
        for gi in range(len(self.groups)):
            self.slots(gi, stream)
        for gi in range(len(self.groups)):
            self.scatter(gi, stream)

    def _prepared_fused(self):
        if self._fused is None:
            self._fused = api.prepared_step(
                self.sched_rows, self.num_scheduled, self.completed, self.token_ids, self.T,
                [dict(block_table=g["block_table"], block_size=g["block_size"],
                      num_blocks=g["num_blocks"], sliding_window=g["sliding_window"],
                      slot_mapping=g["slot_mapping"],
                      input_block_tables=g["input_block_tables"], k=g["k"], v=g["v"],
                      k_cache=g["k_cache"], v_cache=g["v_cache"]) for g in self.groups],
                index_mapping=self.index_mapping, query_start_loc=self.query_start_loc,
                seq_lens=self.seq_lens, positions=self.positions, input_ids=self.input_ids,
                status=self.status)
        return self._fused

    def run_fused(self, stream=None):
        """The same step through the single pkv_step entry point (arguments
        checked and marshalled on the first call, then reused)."""
        self._prepared_fused()(stream)

    def fused_path(self) -> int:
        """The launch plan pkv_step takes for this step (pkv_step_path:
        api.STEP_ONE_LAUNCH, STEP_RANKED_ONE_LAUNCH, STEP_BATCH_THEN_SCATTER or
        STEP_SEPARATE)."""
        return self._prepared_fused().path

    def status_bits(self) -> int:
        return int(self.status.item()) & 0xFFFFFFFF

    def host(self, name: str, gi: Optional[int] = None) -> np.ndarray:
        t = self.groups[gi][name] if gi is not None else getattr(self, name)
        return t.cpu().numpy()
