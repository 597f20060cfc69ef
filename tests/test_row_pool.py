"""The library's host-side row pool against the oracle's (no GPU: the pool is
host code).  Same random acquire/release sequences, same rows handed out,
same return codes, same free count after every call.  The tests take the
library as a parameter, so that a host-only sanitized build runs them too
(tests/test_host_sanitized.py)."""
import numpy as np
import pytest

import oracle
from paged_kv_input_amd import _abi as api


@pytest.fixture(scope="module")
def lib():
    from paged_kv_input_amd.api import _lib

    return _lib


@pytest.mark.parametrize("seed", range(30))
def test_pool_matches_oracle(lib, seed):
    rng = np.random.default_rng(3100 + seed)
    R = int(rng.integers(0, 70))
    mine, ref = api.RowPool(R, lib), oracle.RowPool(R)
    out = []
    for _ in range(60):
        if rng.random() < 0.5:
            m = int(rng.integers(0, R // 3 + 3))
            rc, want = ref.acquire(m)
            if rc == 0:
                assert mine.acquire(m) == want
                out += want
            else:
                with pytest.raises(api.PagedKVError) as e:
                    mine.acquire(m)
                assert e.value.code == rc == api.ENOROWS
        else:
            k = int(rng.integers(0, 5))
            cand = out * 3 + list(range(R)) + [-1, R]
            rows = [int(x) for x in rng.choice(cand, k)] if k and cand else []
            rc = ref.release(rows)
            if rc == 0:
                mine.release(rows)
                out = [r for r in out if r not in rows]
            else:
                with pytest.raises(api.PagedKVError) as e:
                    mine.release(rows)
                assert e.value.code == rc == api.EINVAL
        assert mine.num_free == ref.free == R - len(out)


def test_pool_host_argument_errors(lib):
    import ctypes

    h = ctypes.c_void_p()
    assert lib.pkv_row_pool_create(-1, ctypes.byref(h)) == api.EINVAL
    assert lib.pkv_row_pool_create(4, None) == api.EINVAL
    assert lib.pkv_row_pool_acquire(None, 1, None) == api.EINVAL
    assert lib.pkv_row_pool_release(None, 0, None) == api.EINVAL
    assert lib.pkv_row_pool_num_free(None) == -1
    assert lib.pkv_row_pool_create(4, ctypes.byref(h)) == 0
    assert lib.pkv_row_pool_acquire(h, -1, None) == api.EINVAL
    assert lib.pkv_row_pool_acquire(h, 2, None) == api.EINVAL
    assert lib.pkv_row_pool_acquire(h, 0, None) == 0
    assert lib.pkv_row_pool_num_free(h) == 4
    lib.pkv_row_pool_destroy(h)
    lib.pkv_row_pool_destroy(None)


def test_pool_epoch_reuse(lib):
    """Many releases in a row: the duplicate check's per-call marks never
    mistake an old call's row for a duplicate."""
    pool = api.RowPool(3, lib)
    for _ in range(2000):
        rows = pool.acquire(3)
        pool.release(rows[::-1])
    # release pushes 2, 1, 0 in that order, so 0 is on top again
    assert pool.acquire(3) == [0, 1, 2]
    with pytest.raises(api.PagedKVError):
        pool.release([0, 0])
    pool.release([1])
    assert pool.acquire(1) == [1]
