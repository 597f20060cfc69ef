"""The C ABI of libpagedkv as ctypes declarations: return codes, status bits,
limits, the pkv_group descriptor, the signatures of every entry point and the
host-only row pool.  No torch here, so that host-only builds of the library
(e.g. under the address sanitizer) load with the same declarations; the
torch-facing binding is ``api``.  Values restate include/pagedkv.h, and a test
compares them with it.
"""
from __future__ import annotations

import ctypes
import os

OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP, ENOROWS, ENOMEM = 0, -1, -2, -3, -4, -5, -6
ST_BITS = {
    "BAD_ROW": 0x01, "BAD_COUNT": 0x02, "TOKEN_SUM": 0x04, "POS_OOR": 0x08,
    "LB_OOR": 0x10, "BLOCK_OOR": 0x20, "SLOT_OOR": 0x40, "BAD_RANGE": 0x80,
    "TABLE_FULL": 0x100,
}
NO_BLOCK = 2**31 - 1        # prefix index: an entry without a block
MAX_BATCH = 4096

STEP_MAX_BATCH = 512
STEP_MAX_GROUPS = 4
STEP_RANKED_MIN_BATCH = 32
# pkv_step_path's values: the launch plan of pkv_step
STEP_ONE_LAUNCH, STEP_BATCH_THEN_SCATTER, STEP_SEPARATE, STEP_RANKED_ONE_LAUNCH = 0, 1, 2, 3

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class Group(ctypes.Structure):
    """pkv_group: one KV-cache group's inputs and outputs for pkv_step."""

    _fields_ = [
        ("block_table", _P), ("slot_mapping", _P), ("input_block_tables", _P),
        ("k", _P), ("v", _P), ("k_cache", _P), ("v_cache", _P),
        ("k_stride", _I64), ("v_stride", _I64), ("num_slots", _I64), ("row_bytes", _I64),
        ("MB", _I32), ("block_size", _I32), ("num_blocks", _I32), ("sliding_window", _I32),
    ]


def error_string(lib: ctypes.CDLL, code: int) -> str:
    return lib.pkv_error_string(code).decode()


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, code: int, lib: ctypes.CDLL = None):
        text = error_string(lib, code) if lib is not None else "error"
        super().__init__(f"{fn}: {text} (code {code})")
        self.code = code


def load_library(path: str) -> ctypes.CDLL:
    """Load libpagedkv (or a host-only build of its entry points) and declare
    its signatures.  A caller that also uses torch imports torch first, so the
    library binds to the HIP runtime torch already loaded."""
    if not os.path.exists(path):
        raise ImportError(
            f"libpagedkv not built at {path}: run `python __graft_entry__.py` or "
            "`python paged_kv_input_amd/build.py` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    lib.pkv_prepare_batch.restype = ctypes.c_int
    lib.pkv_prepare_batch.argtypes = [_I32, _I32, _P, _P, _P, _I32, _P, _I64, _I32,
                                      _P, _P, _P, _P, _P, _P, _P]
    lib.pkv_compute_slot_mapping.restype = ctypes.c_int
    lib.pkv_compute_slot_mapping.argtypes = [_I32, _I32, _P, _P, _P, _P, _P, _I32, _I32,
                                             _I32, _I32, _I32, _P, _P, _P, _P]
    lib.pkv_scatter_kv.restype = ctypes.c_int
    lib.pkv_scatter_kv.argtypes = [_I32, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _P, _P]
    lib.pkv_step.restype = ctypes.c_int
    lib.pkv_step.argtypes = [_I32, _I32, _P, _P, _P, _I32, _P, _I64, _I32, _P, _P, _P, _P, _P,
                             _I32, ctypes.POINTER(Group), _P, _P]
    lib.pkv_step_path.restype = ctypes.c_int
    lib.pkv_step_path.argtypes = [_I32, _I32, _I32, ctypes.POINTER(Group)]
    lib.pkv_gather_kv.restype = ctypes.c_int
    lib.pkv_gather_kv.argtypes = [_I32, _P, _P, _I32, _P, _I32, _I32, _I32, _I64, _P, _P, _I64,
                                  _P, _I64, _P, _I64, _P, _P, _P]
    lib.pkv_window_free.restype = ctypes.c_int
    lib.pkv_window_free.argtypes = [_I32, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P]
    lib.pkv_lookahead_slots.restype = ctypes.c_int
    lib.pkv_lookahead_slots.argtypes = [_I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P,
                                        _P]
    lib.pkv_blocks_needed.restype = ctypes.c_int
    lib.pkv_blocks_needed.argtypes = [_I32, _P, _P, _I32, _I32, _P, _P, _I32, _P, _P, _P]
    lib.pkv_hash_blocks.restype = ctypes.c_int
    lib.pkv_hash_blocks.argtypes = [_I32, _P, _I64, _P, _P, _I32, _I32, _P, _P, _P, _P]
    lib.pkv_prefix_clear.restype = ctypes.c_int
    lib.pkv_prefix_clear.argtypes = [_P, _P, _I64, _P]
    lib.pkv_prefix_lookup.restype = ctypes.c_int
    lib.pkv_prefix_lookup.argtypes = [_I32, _P, _I32, _P, _I32, _P, _P, _I64, _P, _P, _P, _P]
    lib.pkv_prefix_insert.restype = ctypes.c_int
    lib.pkv_prefix_insert.argtypes = [_I32, _P, _I32, _P, _P, _P, _P, _I32, _P, _P, _I64, _P,
                                      _P]
    lib.pkv_prefix_evict.restype = ctypes.c_int
    lib.pkv_prefix_evict.argtypes = [_I32, _P, _P, _P, _P, _I64, _P]
    lib.pkv_add_requests.restype = ctypes.c_int
    lib.pkv_add_requests.argtypes = [_I32, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _P, _P,
                                     _I64, _I32, _P, _I32, _P, _P, _P]
    lib.pkv_append_blocks.restype = ctypes.c_int
    lib.pkv_append_blocks.argtypes = [_I32, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _P]
    lib.pkv_advance_state.restype = ctypes.c_int
    lib.pkv_advance_state.argtypes = [_I32, _P, _P, _P, _I32, _P, _P, _I64, _I32, _P, _P]
    lib.pkv_row_pool_create.restype = ctypes.c_int
    lib.pkv_row_pool_create.argtypes = [_I32, ctypes.POINTER(_P)]
    lib.pkv_row_pool_destroy.restype = None
    lib.pkv_row_pool_destroy.argtypes = [_P]
    lib.pkv_row_pool_acquire.restype = ctypes.c_int
    lib.pkv_row_pool_acquire.argtypes = [_P, _I32, _P]
    lib.pkv_row_pool_release.restype = ctypes.c_int
    lib.pkv_row_pool_release.argtypes = [_P, _I32, _P]
    lib.pkv_row_pool_num_free.restype = _I32
    lib.pkv_row_pool_num_free.argtypes = [_P]
    lib.pkv_error_string.restype = ctypes.c_char_p
    lib.pkv_error_string.argtypes = [ctypes.c_int]
    lib.pkv_abi_version.restype = ctypes.c_int
    lib.pkv_abi_version.argtypes = []
    return lib



class RowPool:
    """Host-side pool of request_state_index rows (pkv_row_pool_*) of ``lib``:
    ``acquire(m)`` hands out m free rows (the most recently released first),
    ``release(rows)`` takes rows back.  Both raise PagedKVError and change
    nothing on failure."""

    def __init__(self, R: int, lib: ctypes.CDLL):
        self._lib = lib
        h = _P()
        rc = lib.pkv_row_pool_create(int(R), ctypes.byref(h))
        if rc != OK:
            raise PagedKVError("row_pool_create", rc, lib)
        self._h = h
        self.R = int(R)

    def acquire(self, m: int):
        out = (_I32 * max(int(m), 1))()
        rc = self._lib.pkv_row_pool_acquire(self._h, int(m), out)
        if rc != OK:
            raise PagedKVError("row_pool_acquire", rc, self._lib)
        return list(out[:int(m)])

    def release(self, rows) -> None:
        rows = [int(r) for r in rows]
        arr = (_I32 * max(len(rows), 1))(*rows)
        rc = self._lib.pkv_row_pool_release(self._h, len(rows), arr)
        if rc != OK:
            raise PagedKVError("row_pool_release", rc, self._lib)

    @property
    def num_free(self) -> int:
        return int(self._lib.pkv_row_pool_num_free(self._h))

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        lib = getattr(self, "_lib", None)
        if h is not None and lib is not None:
            lib.pkv_row_pool_destroy(h)
