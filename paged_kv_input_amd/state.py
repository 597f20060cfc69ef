"""The persistent request state on the device: per state row the tokens
already processed, the request's token list, its block table and the number of
logical blocks allocated to it.

``DeviceState`` owns the four tensors and calls the library's state entry
points (add_requests, append_blocks, advance_state) on them; its tensors are
the ``completed``, ``token_ids`` and ``block_table`` inputs of a step.  Ragged
per-request lists are packed on the host into CSR (offsets plus one flat
array) and copied to the device: that packing is argument marshalling, every
state update runs in the library's kernels.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import api


def pack_csr(lists: Sequence[Sequence[int]]):
    """[list, ...] -> (start int32 [m+1], flat int32 [max(total, 1)]) on the host.
    The flat array holds at least one element so its pointer is never NULL;
    the library takes its true length from start[m]."""
    start = np.zeros(len(lists) + 1, np.int64)
    if len(lists):
        start[1:] = np.cumsum([len(x) for x in lists])
    if start[-1] > np.iinfo(np.int32).max:
        raise ValueError("CSR list too long for int32 offsets")
    flat = np.fromiter((v for x in lists for v in x), np.int32, count=int(start[-1]))
    return start.astype(np.int32), (flat if flat.size else np.zeros(1, np.int32)), int(start[-1])


class DeviceState:
    """completed [R], token_ids [R, L], block_table [R, MB], row_blocks [R]
    (int32, device) plus a status word."""

    def __init__(self, R: int, L: int, MB: int, *, device="cuda", token_fill: int = -1):
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.device = dev
        self.R, self.L, self.MB = int(R), int(L), int(MB)
        self.completed = torch.zeros(self.R, **i32)
        self.token_ids = torch.full((self.R, self.L), token_fill, **i32)
        self.block_table = torch.full((self.R, self.MB), -1, **i32)
        self.row_blocks = torch.zeros(self.R, **i32)
        self.status = torch.zeros(1, **i32)

    def _up(self, a):
        if isinstance(a, torch.Tensor):
            return a
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.device)

    def _csr(self, lists):
        """Lists, or an already packed (start, flat, total) triple (which may
        hold bad ranges: the kernels flag them)."""
        start, flat, total = lists if isinstance(lists, tuple) else pack_csr(lists)
        flat = self._up(flat)
        return self._up(start), flat[:total] if total < flat.numel() else flat

    def add_requests(self, rows, num_computed, prompts, blocks, stream=None):
        """add_request for each new request: prompts and blocks are one list
        per request (or CSR triples)."""
        ps, pt = self._csr(prompts)
        bs_, bl = self._csr(blocks)
        api.add_requests(self._up(rows), self._up(num_computed), ps, pt, bs_, bl,
                         completed=self.completed, token_ids=self.token_ids,
                         block_table=self.block_table, row_blocks=self.row_blocks,
                         status=self.status, stream=stream)

    def append_blocks(self, rows, blocks, stream=None):
        """update_request: append each request's newly allocated block ids."""
        bs_, bl = self._csr(blocks)
        api.append_blocks(self._up(rows), bs_, bl, block_table=self.block_table,
                          row_blocks=self.row_blocks, status=self.status, stream=stream)

    def advance(self, index_mapping, seq_lens, sampled: Optional[object] = None, stream=None):
        """After a step: completed = seq_len and sampled tokens appended, in
        the step's batch order (index_mapping, seq_lens as it produced them)."""
        api.advance_state(self._up(index_mapping), self._up(seq_lens),
                          None if sampled is None else self._up(sampled),
                          completed=self.completed, token_ids=self.token_ids,
                          status=self.status, stream=stream)

    def status_bits(self) -> int:
        return int(self.status.item()) & 0xFFFFFFFF

    def host(self) -> dict:
        return {"completed": self.completed.cpu().numpy(),
                "token_ids": self.token_ids.cpu().numpy(),
                "block_table": self.block_table.cpu().numpy(),
                "row_blocks": self.row_blocks.cpu().numpy()}
