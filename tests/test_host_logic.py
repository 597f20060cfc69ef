"""Host-side logic of the binding, on the CPU: CSR packing of ragged lists
and the argument checks that reject bad tensors before any GPU call."""
import numpy as np
import pytest
import torch


def test_pack_csr_matches_oracle_csr():
    from paged_kv_input_amd.state import pack_csr
    import oracle

    rng = np.random.default_rng(0)
    for _ in range(50):
        lists = [rng.integers(-5, 100, int(rng.integers(0, 7))).tolist()
                 for _ in range(int(rng.integers(0, 9)))]
        start, flat, total = pack_csr(lists)
        o_start, o_flat, o_total = oracle.csr(lists)
        assert total == o_total
        assert start.dtype == np.int32 and flat.dtype == np.int32
        assert np.array_equal(start, o_start)
        assert np.array_equal(flat[:total], o_flat[:total])
        assert flat.size >= 1                       # never a NULL pointer
        for i, x in enumerate(lists):
            assert flat[start[i]:start[i + 1]].tolist() == list(x)


def test_binding_rejects_bad_tensors_before_any_gpu_call():
    from paged_kv_input_amd import api

    cpu = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        api.prepared_add_requests(cpu, cpu, cpu, cpu, cpu, cpu, completed=cpu, token_ids=cpu,
                                  block_table=cpu, row_blocks=cpu)
    with pytest.raises(ValueError):
        api.hash_blocks(cpu, torch.zeros(4, dtype=torch.int64), cpu, 16,
                        hashes=torch.zeros((4, 2), dtype=torch.int64))
    with pytest.raises(ValueError):
        api.blocks_needed(cpu, cpu, 0, 16, cpu, cpu, need=cpu)
    with pytest.raises(ValueError):
        api.window_free(cpu, cpu, cpu.view(2, 2), 16, 8, freed=cpu.view(2, 2), num_freed=cpu)
    with pytest.raises(ValueError):
        api.prefix_clear(torch.zeros(12, dtype=torch.int64), torch.zeros(12, dtype=torch.int32))


def test_row_pool_is_host_only():
    """The row pool needs no GPU at all."""
    from paged_kv_input_amd import RowPool

    pool = RowPool(3)
    assert pool.acquire(2) == [0, 1]
    pool.release([0])
    assert pool.acquire(2) == [0, 2]
    assert pool.num_free == 0
