"""A decode iteration captured once in a HIP graph and replayed: append the
new blocks, the step (pkv_step), advance the state.  The entry points only
enqueue kernels (no allocation, no synchronization, no memset), so the
iteration can be captured; every replay, with the host's own copies and
synchronizations between replays, is checked against the oracle's loop."""
import numpy as np
import pytest

import oracle
from gpu_util import SENTINEL16, assert_equal, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_input_amd  # noqa: F401  (raises if the library is missing)
    yield
    torch.cuda.synchronize()


def test_decode_iteration_in_hip_graph():
    import torch
    from paged_kv_input_amd import api
    from paged_kv_input_amd.state import DeviceState
    from paged_kv_input_amd.step import DeviceStep, GroupSpec

    rng = np.random.default_rng(77)
    R, L, MB, bs, NB, H, D, n, steps = 64, 1024, 64, 16, 2048, 2, 64, 40, 24
    ds = DeviceState(R, L, MB)
    st = oracle.empty_state(R, L, MB)
    pool = rng.permutation(NB).tolist()
    rows = sorted(rng.choice(R, n, replace=False).tolist())
    plens = rng.integers(1, 300, n).tolist()
    prompts = [rng.integers(0, 1 << 20, p).tolist() for p in plens]
    # Registered as computed up to the last prompt token: decoding starts there.
    done = [p - 1 for p in plens]
    blocks = [[pool.pop() for _ in range(-(-p // bs))] for p in plens]
    ds.add_requests(rows, done, prompts, blocks)
    oracle.add_requests(st, rows, done, prompts, blocks)

    dev = ds.device
    i32 = dict(dtype=torch.int32, device=dev)
    rows_d = torch.tensor(rows, **i32)
    blk_start = torch.zeros(n + 1, **i32)          # static inputs, refilled before each replay
    blk_flat = torch.zeros(n, **i32)
    sampled = torch.zeros(n, **i32)
    k0 = np.zeros((n, H, D), np.int16)
    step = DeviceStep(rows, [1] * n, ds.completed, ds.token_ids,
                      [GroupSpec(ds.block_table, bs, NB, k0, k0)], num_tokens=n,
                      cache_fill=SENTINEL16, ibt_fill=oracle.IBT_UNWRITTEN)
    g = step.groups[0]
    append = api.prepared_append_blocks(rows_d, blk_start, blk_flat, block_table=ds.block_table,
                                        row_blocks=ds.row_blocks, status=ds.status)
    fused = api.prepared_step(
        step.sched_rows, step.num_scheduled, ds.completed, ds.token_ids, n,
        [dict(block_table=ds.block_table, block_size=bs, num_blocks=NB,
              slot_mapping=g["slot_mapping"], input_block_tables=g["input_block_tables"],
              k=g["k"], v=g["v"], k_cache=g["k_cache"], v_cache=g["v_cache"])],
        index_mapping=step.index_mapping, query_start_loc=step.query_start_loc,
        seq_lens=step.seq_lens, positions=step.positions, input_ids=step.input_ids,
        status=step.status)
    advance = api.prepared_advance_state(step.index_mapping, step.seq_lens, sampled,
                                         completed=ds.completed, token_ids=ds.token_ids,
                                         status=ds.status)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        append()
        fused()
        advance()
    kc_o = np.full((NB * bs, H, D), 0xFFFF, np.uint16)
    vc_o = kc_o.copy()
    for s in range(steps):
        # the host's work between replays: new blocks, payload, sampled tokens
        need = []
        for r in rows:
            want = -(-(int(st["completed"][r]) + 1) // bs)
            need.append([pool.pop() for _ in range(max(0, want - int(st["row_blocks"][r])))])
        start, flat, total = oracle.csr(need)
        flat_pad = np.zeros(n, np.int32)
        flat_pad[:total] = flat[:total]
        blk_start.copy_(torch.from_numpy(start))
        blk_flat.copy_(torch.from_numpy(flat_pad))
        k = rng.integers(-30000, 30000, (n, H, D)).astype(np.int16)
        v = rng.integers(-30000, 30000, (n, H, D)).astype(np.int16)
        g["k"].copy_(torch.from_numpy(k))
        g["v"].copy_(torch.from_numpy(v))
        smp = rng.integers(0, 1 << 20, n).astype(np.int32)
        sampled.copy_(torch.from_numpy(smp))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"[case] graph replay {s}")
        # the oracle's same iteration (blocks by request; total = padded length)
        oracle.append_blocks(st, rows, (start, flat_pad, n))
        prep = oracle.prepare_batch(rows, [1] * n, st["completed"], st["token_ids"])
        sm = oracle.compute_slot_mapping(prep["index_mapping"], prep["query_start_loc"],
                                         prep["seq_lens"], prep["positions"], st["block_table"],
                                         bs, NB)
        oracle.scatter_kv(k.view(np.uint16), v.view(np.uint16), kc_o, vc_o, sm["slot_mapping"])
        oracle.advance_state(st, prep["index_mapping"], prep["seq_lens"], smp)
        assert step.status_bits() == 0 and ds.status_bits() == 0
        for key in ("index_mapping", "seq_lens", "positions", "input_ids"):
            assert_equal(f"replay {s} {key}", step.host(key), prep[key])
        assert_equal(f"replay {s} slots", step.host("slot_mapping", 0), sm["slot_mapping"])
        got = ds.host()
        for key in ("completed", "token_ids", "block_table", "row_blocks"):
            assert_equal(f"replay {s} {key}", got[key], st[key])
    assert_equal("k_cache", g["k_cache"].cpu().numpy().view(np.uint16), kc_o)
    assert_equal("v_cache", g["v_cache"].cpu().numpy().view(np.uint16), vc_o)
