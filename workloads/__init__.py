"""Seeded synthetic schedules for the paged-KV input path.

This module only *builds inputs*: a step's schedule (state rows and scheduled
token counts), the worker's persistent state (completed tokens, token table,
per-group block tables) and the new tokens' K/V payload. It computes none of
the outputs the path produces (batch order, prefix sums, positions, slots,
scatter). Both the CPU oracle's tests and the HIP library's tests and benchmark
draw their inputs from here, so the two sides see the same bits.

Shapes and distributions follow the workloads the pages imply:

* the worked example of "Deep Dive into vLLM's Scheduling Mechanism"
  (kongchang.com/en), sections "Design Logic Behind the Dual-Index System" and
  "Address Calculation Example": request B in state row 7 with 31 tokens done and
  blocks [37, 12], request A in row 6 with 16 done and blocks [81, 44], 1 and 8
  tokens scheduled, block size 16;
* decode-heavy, mixed chunked-prefill, long-prefill and two-KV-cache-group
  batches with random, non-contiguous physical block assignment (the page-table
  indirection of the same article's "Persistent Request Context Strategy").

Every config draws from ``numpy.random.default_rng(seed)``. K/V values are
N(0, 1) float32 rounded to the payload dtype (round-to-nearest-even) and kept as
raw 16-bit words, because the path copies them bit for bit.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "KVGroup",
    "Batch",
    "make",
    "CONFIGS",
    "pages_example",
    "prefix_reuse_example",
    "budget_tie_example",
    "random_tiny",
]

VOCAB = 128256  # token ids drawn uniformly from [0, VOCAB)


@dataclass
class KVGroup:
    """One KV-cache group: its own block size, pool, block table and payload."""

    block_size: int
    num_blocks: int
    max_blocks: int               # block-table width (logical blocks per request)
    block_table: np.ndarray       # int32 [R, max_blocks]; -1 = not allocated
    num_heads: int
    head_dim: int
    dtype: str                    # "fp16" | "bf16" (payload words are uint16)
    k: Optional[np.ndarray] = None  # uint16 [T, H, D]
    v: Optional[np.ndarray] = None  # uint16 [T, H, D]

    @property
    def num_slots(self) -> int:
        return self.num_blocks * self.block_size

    @property
    def row_bytes(self) -> int:
        return self.num_heads * self.head_dim * 2


@dataclass
class Batch:
    """One step's schedule plus the persistent worker state it refers to."""

    name: str
    seed: int
    sched_rows: np.ndarray        # int32 [n], schedule order (as the host lists it)
    num_scheduled: np.ndarray     # int32 [n]
    completed: np.ndarray         # int32 [R], tokens already processed, before this step
    token_ids: np.ndarray         # int32 [R, L]
    groups: List[KVGroup] = field(default_factory=list)

    @property
    def n(self) -> int:
        return int(self.sched_rows.shape[0])

    @property
    def T(self) -> int:
        return int(self.num_scheduled.astype(np.int64).sum()) if self.n else 0

    @property
    def R(self) -> int:
        return int(self.completed.shape[0])

    @property
    def L(self) -> int:
        return int(self.token_ids.shape[1])


# ---------------------------------------------------------------------------
# payload
# ---------------------------------------------------------------------------

def _payload(rng: np.random.Generator, T: int, H: int, D: int, dtype: str) -> np.ndarray:
    """N(0,1) float32 rounded to fp16/bf16 (round-to-nearest-even), as uint16 words."""
    x = rng.standard_normal((T, H, D), dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch  # CPU cast only: plumbing for the input bits

        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"unknown payload dtype {dtype!r}")


def _attach_payload(rng: np.random.Generator, b: Batch) -> None:
    for g in b.groups:
        g.k = _payload(rng, b.T, g.num_heads, g.head_dim, g.dtype)
        g.v = _payload(rng, b.T, g.num_heads, g.head_dim, g.dtype)


# ---------------------------------------------------------------------------
# block tables
# ---------------------------------------------------------------------------

def _block_table(rng: np.random.Generator, R: int, MB: int, NB: int, bs: int,
                 rows: np.ndarray, counts: np.ndarray, completed: np.ndarray) -> np.ndarray:
    """Random, non-contiguous physical block assignment for the scheduled rows.

    Pool rule: with ``perm`` a random permutation of the NB physical blocks,
    (1) the request's private blocks -- logical blocks from floor(done / bs)
        up to the one holding its last token, ceil((done + count) / bs) - 1,
        i.e. the partly filled block and every block this step writes into --
        are taken from ``perm`` without replacement, request by request, so no
        two new tokens share a slot;
    (2) full history blocks (logical block < floor(done / bs)) are taken from
        the rest of ``perm``, cycling over it when it runs out (shared full
        history blocks read as prefix reuse; they are never written).
    Entries past a row's allocation, and every entry of an unscheduled row, are -1.
    """
    bt = np.full((R, MB), -1, dtype=np.int32)
    perm = rng.permutation(NB).astype(np.int32)
    cur = 0
    for r, c in zip(rows.tolist(), counts.tolist()):
        done = int(completed[r])
        first, end = done // bs, -(-(done + max(c, 0)) // bs)
        need = end - first
        if need <= 0:
            continue
        if end > MB:
            raise ValueError("block table too narrow for the generated schedule")
        if cur + need > NB:
            raise ValueError("pool too small for unique write blocks")
        bt[r, first:end] = perm[cur:cur + need]
        cur += need
    rest = perm[cur:]
    j = 0
    for r in rows.tolist():
        full = int(completed[r]) // bs
        if full == 0:
            continue
        if rest.size == 0:
            raise ValueError("no pool left for history blocks")
        idx = (j + np.arange(full)) % rest.size
        bt[r, :full] = rest[idx]
        j += full
    return bt


def _token_table(rng: np.random.Generator, R: int, L: int) -> np.ndarray:
    return rng.integers(0, VOCAB, size=(R, L), dtype=np.int32)


# ---------------------------------------------------------------------------
# the pages' worked examples
# ---------------------------------------------------------------------------

def pages_example(seed: int = 0, with_payload: bool = True) -> Batch:
    """The worked example of the kongchang.com article (both language versions).

    Request B: state row 7, 31 tokens completed, physical blocks [37, 12], 1 token
    scheduled.  Request A: state row 6, 16 completed, blocks [81, 44], 8 tokens.
    Block size 16.  The schedule lists B first, as the article does.  The token
    table is the identity code token_ids[r][p] = r * L + p (the article prints no
    token ids), so every input id decodes back to its (row, position).
    """
    R, L, MB, NB, bs = 8, 32, 2, 128, 16
    completed = np.zeros(R, np.int32)
    completed[7], completed[6] = 31, 16
    bt = np.full((R, MB), -1, np.int32)
    bt[7] = [37, 12]
    bt[6] = [81, 44]
    token_ids = (np.arange(R, dtype=np.int32)[:, None] * L + np.arange(L, dtype=np.int32)[None, :])
    b = Batch("pages_example", seed, np.array([7, 6], np.int32), np.array([1, 8], np.int32),
              completed, token_ids.astype(np.int32),
              [KVGroup(bs, NB, MB, bt, 8, 128, "fp16")])
    if with_payload:
        _attach_payload(np.random.default_rng(seed), b)
    return b


def prefix_reuse_example(p1: int = 5, p2: int = 9, b3: int = 2, seed: int = 0) -> Batch:
    """The prefix-reuse example of "从源码读 vLLM Scheduler" (caffein.top), section
    "Prefix Cache：复用的是 KV，不是答案" and the allocate_slots() section.

    Block size 4; request B shares an 8-token system prompt that is already cached
    in blocks P1, P2 and brings 2 new tokens, which land in one newly allocated
    block B3, so B's logical block table reads [P1][P2][B3].  The page names the
    blocks symbolically; ``p1, p2, b3`` instantiate them with distinct ids.
    """
    R, L, MB, NB, bs = 4, 12, 3, 16, 4
    row = 1
    completed = np.zeros(R, np.int32)
    completed[row] = 8
    bt = np.full((R, MB), -1, np.int32)
    bt[row] = [p1, p2, b3]
    token_ids = (np.arange(R, dtype=np.int32)[:, None] * L + np.arange(L, dtype=np.int32)[None, :])
    b = Batch("prefix_reuse_example", seed, np.array([row], np.int32), np.array([2], np.int32),
              completed, token_ids.astype(np.int32), [KVGroup(bs, NB, MB, bt, 1, 8, "fp16")])
    _attach_payload(np.random.default_rng(seed), b)
    return b


def budget_tie_example(seed: int = 0) -> Batch:
    """The 8-token-budget example of the caffein.top article, section
    "schedule()：先保住正在运行的请求": A (10-token prompt, 8 done, running) gets
    2 tokens; B (2-token prompt, waiting) gets min(2, 6) = 2.  Both advance by the
    same count, so the batch order is decided by the tie-break alone.  The host
    lists A (state row 5) before B (state row 3).
    """
    R, L, MB, NB, bs = 8, 16, 4, 32, 4
    completed = np.zeros(R, np.int32)
    completed[5], completed[3] = 8, 0
    rows = np.array([5, 3], np.int32)
    counts = np.array([2, 2], np.int32)
    rng = np.random.default_rng(seed)
    bt = _block_table(rng, R, MB, NB, bs, rows, counts, completed)
    token_ids = (np.arange(R, dtype=np.int32)[:, None] * L + np.arange(L, dtype=np.int32)[None, :])
    b = Batch("budget_tie_example", seed, rows, counts, completed, token_ids.astype(np.int32),
              [KVGroup(bs, NB, MB, bt, 2, 8, "bf16")])
    _attach_payload(rng, b)
    return b


# ---------------------------------------------------------------------------
# seeded configurations
# ---------------------------------------------------------------------------

def _seeded_small(seed: int, decode_frac: float = 0.0, n: int = 16, R: int = 32,
                  max_count: int = 64, max_done: int = 512, bs: int = 16, NB: int = 4096,
                  H: int = 8, D: int = 128, dtype: str = "fp16", name: str = "seeded_16req") -> Batch:
    """16 requests in 32 state rows; counts uniform on {1..64} (a fraction forced to
    1 for ties), completed uniform 0..512, block size 16, 4096-block pool."""
    rng = np.random.default_rng(seed)
    rows = rng.choice(R, size=n, replace=False).astype(np.int32)
    counts = rng.integers(1, max_count + 1, size=n).astype(np.int32)
    if decode_frac > 0:
        counts[rng.random(n) < decode_frac] = 1
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, max_done + 1, size=n)
    L = max_done + max_count
    MB = -(-L // bs)
    bt = _block_table(rng, R, MB, NB, bs, rows, counts, completed)
    b = Batch(name, seed, rows, counts, completed, _token_table(rng, R, L),
              [KVGroup(bs, NB, MB, bt, H, D, dtype)])
    _attach_payload(rng, b)
    return b


def _decode_heavy(seed: int, n: int = 256, R: int = 1024, lo: int = 128, hi: int = 8192,
                  bs: int = 16, NB: int = 65536, H: int = 8, D: int = 128,
                  name: str = "decode_256x1") -> Batch:
    """n decode requests x 1 token in R state rows; context uniform lo..hi is read as
    the tokens already completed; 16-token blocks from a 65536-block pool."""
    rng = np.random.default_rng(seed)
    rows = rng.choice(R, size=n, replace=False).astype(np.int32)
    counts = np.ones(n, np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(lo, hi + 1, size=n)
    L = hi + 1
    MB = -(-L // bs)
    bt = _block_table(rng, R, MB, NB, bs, rows, counts, completed)
    b = Batch(name, seed, rows, counts, completed, _token_table(rng, R, L),
              [KVGroup(bs, NB, MB, bt, H, D, "bf16")])
    _attach_payload(rng, b)
    return b


def _free_list_rows(rng: np.random.Generator, R: int, n: int) -> np.ndarray:
    """State rows recycled through a free list with churn: allocate R/2 rows, free a
    random half of them (pushed back on top, LIFO), then allocate the batch."""
    free = list(range(R - 1, -1, -1))          # stack, top = end
    held = [free.pop() for _ in range(R // 2)]
    back = rng.permutation(len(held))[: len(held) // 2]
    for i in back.tolist():
        free.append(held[i])
    return np.array([free.pop() for _ in range(n)], np.int32)


def _mixed_chunked(seed: int, budget: int = 8192, decodes: int = 64, lo: int = 256,
                   hi: int = 2048, max_done: int = 4096, R: int = 256, bs: int = 16,
                   NB: int = 32768, H: int = 8, D: int = 128, name: str = "mixed_8192") -> Batch:
    """64 decode requests plus prefill chunks uniform lo..hi filling the rest of an
    8192-token budget (the last chunk clipped to what is left); completed uniform
    0..4096; rows from a churned free list."""
    rng = np.random.default_rng(seed)
    counts = [1] * decodes
    left = budget - decodes
    while left > 0:
        c = int(rng.integers(lo, hi + 1))
        c = min(c, left)
        counts.append(c)
        left -= c
    counts = np.array(counts, np.int32)
    order = rng.permutation(counts.size)
    counts = counts[order]
    n = counts.size
    rows = _free_list_rows(rng, R, n)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, max_done + 1, size=n)
    L = max_done + hi
    MB = -(-L // bs)
    bt = _block_table(rng, R, MB, NB, bs, rows, counts, completed)
    b = Batch(name, seed, rows, counts, completed, _token_table(rng, R, L),
              [KVGroup(bs, NB, MB, bt, H, D, "bf16")])
    _attach_payload(rng, b)
    return b


def _long_prefill(seed: int, n: int = 16, count: int = 2048, bs: int = 32, NB: int = 131072,
                  H: int = 8, D: int = 128, name: str = "prefill_16x2048") -> Batch:
    """n requests x ``count`` new tokens from completed = 0; block size 32;
    131072-block pool; 8 KV heads x 128 bf16 (a GQA layer of a 70B-class model)."""
    rng = np.random.default_rng(seed)
    R = 2 * n
    rows = rng.choice(R, size=n, replace=False).astype(np.int32)
    counts = np.full(n, count, np.int32)
    completed = np.zeros(R, np.int32)
    L = count
    MB = -(-L // bs)
    bt = _block_table(rng, R, MB, NB, bs, rows, counts, completed)
    b = Batch(name, seed, rows, counts, completed, _token_table(rng, R, L),
              [KVGroup(bs, NB, MB, bt, H, D, "bf16")])
    _attach_payload(rng, b)
    return b


def _two_groups(seed: int, n: int = 512, R: int = 1024, lo: int = 16, hi: int = 512,
                max_done: int = 16384, bss=(16, 64), NB: int = 65536, H: int = 4, D: int = 128,
                name: str = "two_groups_512req") -> Batch:
    """Two KV-cache groups (block sizes 16 and 64, separate 65536-block pools and
    permutations): 512 requests, half decodes and half prefill chunks uniform
    16..512 in a seeded shuffled order; completed uniform 0..16384; 4 KV heads x 128
    bf16 per group."""
    rng = np.random.default_rng(seed)
    half = n // 2
    counts = np.concatenate([np.ones(half, np.int64), rng.integers(lo, hi + 1, size=n - half)])
    counts = counts[rng.permutation(n)].astype(np.int32)
    rows = rng.choice(R, size=n, replace=False).astype(np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, max_done + 1, size=n)
    L = max_done + hi
    groups = []
    for bs in bss:
        MB = -(-L // bs)
        bt = _block_table(rng, R, MB, NB, bs, rows, counts, completed)
        groups.append(KVGroup(bs, NB, MB, bt, H, D, "bf16"))
    b = Batch(name, seed, rows, counts, completed, _token_table(rng, R, L), groups)
    _attach_payload(rng, b)
    return b


def random_tiny(seed: int, max_n: int = 8, max_T: int = 64, block_sizes=(1, 3, 4, 16),
                groups: int = 0, zero_counts: bool = False) -> Batch:
    """Tiny random batch for brute-force checks: n <= 8, T <= 64, block size drawn
    from {1, 3, 4, 16} (a non-power-of-two included), 1-2 groups, small payload."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, max_n + 1))
    R = int(rng.integers(n, 2 * n + 2))
    rows = rng.choice(R, size=n, replace=False).astype(np.int32)
    lo = 0 if zero_counts else 1
    counts = rng.integers(lo, 9, size=n).astype(np.int32)
    while counts.astype(np.int64).sum() > max_T:
        counts = np.maximum(counts // 2, lo).astype(np.int32)
    completed = np.zeros(R, np.int32)
    completed[rows] = rng.integers(0, 40, size=n)
    L = 40 + 9
    ng = groups if groups else int(rng.integers(1, 3))
    gs = []
    for _ in range(ng):
        bs = int(rng.choice(block_sizes))
        MB = -(-L // bs)
        need = 0
        for r, c in zip(rows.tolist(), counts.tolist()):
            d = int(completed[r])
            need += max(0, -(-(d + c) // bs) - d // bs)
        NB = need + int(rng.integers(1, 16))
        bt = _block_table(rng, R, MB, NB, bs, rows, counts, completed)
        gs.append(KVGroup(bs, NB, MB, bt, int(rng.choice([1, 2])), 8, "fp16"))
    b = Batch(f"tiny_{seed}", seed, rows, counts, completed, _token_table(rng, R, L), gs)
    _attach_payload(rng, b)
    return b


CONFIGS = {
    # configuration name -> (builder, seed)
    "pages_example": (lambda s: pages_example(s), 0),
    "seeded_16req": (lambda s: _seeded_small(s), 1),
    "seeded_16req_decode50": (lambda s: _seeded_small(s, decode_frac=0.5,
                                                      name="seeded_16req_decode50"), 11),
    "decode_256x1": (lambda s: _decode_heavy(s), 2),
    "mixed_8192": (lambda s: _mixed_chunked(s), 3),
    "prefill_16x2048": (lambda s: _long_prefill(s), 4),
    # One GPU's share when the KV heads are split over 8 GPUs: the same schedule,
    # block tables and pool, one head of 128 bf16 per token (256-byte rows).
    "prefill_16x2048_tp8": (lambda s: _long_prefill(s, H=1, name="prefill_16x2048_tp8"), 4),
    "two_groups_512req": (lambda s: _two_groups(s), 5),
    # A wide decode batch: 4096 requests x 1 token among 8192 state rows,
    # contexts U{128..2048}; past the one-launch step's batch limit.
    "decode_4096x1": (lambda s: _decode_heavy(s, n=4096, R=8192, hi=2048,
                                              name="decode_4096x1"), 6),
}

# Reduced versions: same structure, sizes the oracle finishes in well under a
# second, still spanning several tiles and a ragged tail.
REDUCED = {
    "decode_256x1": lambda s: _decode_heavy(s, n=200, R=512, hi=2048, NB=16384,
                                            name="decode_200x1_reduced"),
    "mixed_8192": lambda s: _mixed_chunked(s, budget=3001, decodes=37, lo=64, hi=700,
                                           name="mixed_3001_reduced"),
    "prefill_16x2048": lambda s: _long_prefill(s, n=5, count=777, NB=4096,
                                               name="prefill_5x777_reduced"),
    "two_groups_512req": lambda s: _two_groups(s, n=96, R=256, hi=200, max_done=3000,
                                               NB=8192, name="two_groups_96req_reduced"),
}


def make(name: str, seed: Optional[int] = None, reduced: bool = False) -> Batch:
    """Build the named configuration (full size unless ``reduced``)."""
    if reduced:
        if name not in REDUCED:
            return make(name, seed)
        return REDUCED[name](CONFIGS[name][1] if seed is None else seed)
    builder, default_seed = CONFIGS[name]
    return builder(default_seed if seed is None else seed)
