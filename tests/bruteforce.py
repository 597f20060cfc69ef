"""Brute-force restatement of the chain for tiny inputs, by other means than the
oracle: ranks by counting instead of a sort, boundaries by summing instead of a
running prefix, a token's request by walking the batch, and a token's slot by
enumerating the request's paged address space block by block (no division or
remainder).  Pure Python loops; only for n <= 8, T <= 64.

Source: "Deep Dive into vLLM's Scheduling Mechanism: The Complete CPU-to-GPU
Mapping Pipeline" (kongchang.com/en), sections "Batch Construction and Sequence
Flattening" through "Complete Input Preparation for the Attention Module".
"""


def batch_order(rows, counts):
    """batch_index of request i = number of requests whose (count, row) key is
    smaller, plus earlier requests with an identical key."""
    n = len(rows)
    rank = []
    for i in range(n):
        r = 0
        for j in range(n):
            kj, ki = (counts[j], rows[j]), (counts[i], rows[i])
            if kj < ki or (kj == ki and j < i):
                r += 1
        rank.append(r)
    order = [None] * n
    for i in range(n):
        order[rank[i]] = i
    return order


def chain(rows, counts, completed, token_ids, groups):
    """groups: list of (block_table rows as lists, block_size).  Returns dict."""
    rows, counts = [int(x) for x in rows], [int(x) for x in counts]
    order = batch_order(rows, counts)
    n = len(rows)
    index_mapping = [rows[i] for i in order]
    sorted_counts = [counts[i] for i in order]
    qsl = []
    for b in range(n + 1):
        s = 0
        for bb in range(b):
            s += sorted_counts[bb]
        qsl.append(s)
    T = qsl[n]
    seq_lens = [int(completed[index_mapping[b]]) + sorted_counts[b] for b in range(n)]
    positions, input_ids, owner = [], [], []
    for t in range(T):
        b, start = 0, 0
        while not (start <= t < start + sorted_counts[b]):
            start += sorted_counts[b]
            b += 1
        row = index_mapping[b]
        p = int(completed[row]) + (t - start)
        positions.append(p)
        input_ids.append(int(token_ids[row][p]))
        owner.append(b)
    out_groups = []
    for bt, bs in groups:
        slots = []
        for t in range(T):
            row = index_mapping[owner[t]]
            space = []                        # the request's logical KV address space
            for blk in bt[row]:
                for o in range(bs):
                    space.append(-1 if blk < 0 else int(blk) * bs + o)
            slots.append(space[positions[t]])
        ibt = []
        for b in range(n):
            vis = 0
            while vis * bs < seq_lens[b]:
                vis += 1
            ibt.append([int(x) for x in bt[index_mapping[b]][:vis]])
        out_groups.append({"slot_mapping": slots, "input_block_tables": ibt})
    return {"index_mapping": index_mapping, "query_start_loc": qsl, "seq_lens": seq_lens,
            "positions": positions, "input_ids": input_ids, "groups": out_groups}


def gather_slots(seq_lens, visible_pages, bs):
    """Slot read for every output row of the paged K/V read, by enumerating each
    request's address space page by page (no division or remainder): request
    b's rows follow the earlier requests' rows, and its position p sits at the
    p-th address of its space.  -1 where no page exists."""
    out = []
    for b, sl in enumerate(seq_lens):
        space = []
        for blk in visible_pages[b]:
            for o in range(bs):
                space.append(-1 if blk < 0 else int(blk) * bs + o)
        for p in range(max(int(sl), 0)):
            out.append(space[p] if p < len(space) else -1)
    return out
