"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one (a dropped term, a wrong sign or index, a transposed operand).

Each mutant is oracle.c with one textual substitution, compiled with gcc into a
temporary directory; the real oracle is never modified.  Mutants are chosen so
that they stay memory-safe (the pins then fail on values, not on a crash).
"""
import os

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "sort_descending": (
        "return a->tokens_this_step < b->tokens_this_step ? -1 : 1;",
        "return a->tokens_this_step < b->tokens_this_step ? 1 : -1;"),
    "tie_break_reversed": (
        "return a->request_state_index < b->request_state_index ? -1 : 1;",
        "return a->request_state_index < b->request_state_index ? 1 : -1;"),
    "no_tie_break": (
        "    if (a->request_state_index != b->request_state_index)\n"
        "        return a->request_state_index < b->request_state_index ? -1 : 1;\n",
        ""),
    "prefix_not_running": (
        "running += batch[b].tokens_this_step;",
        "running = batch[b].tokens_this_step;"),
    "position_off_by_one": (
        "int64_t position = (int64_t)completed[row] + j;",
        "int64_t position = (int64_t)completed[row] + j + 1;"),
    "position_drops_history": (
        "int64_t position = (int64_t)completed[row] + j;",
        "int64_t position = j;"),
    "seq_len_drops_history": (
        "int64_t len = (int64_t)completed[row] + batch[b].tokens_this_step;",
        "int64_t len = batch[b].tokens_this_step;"),
    "seq_len_drops_new": (
        "int64_t len = (int64_t)completed[row] + batch[b].tokens_this_step;",
        "int64_t len = (int64_t)completed[row];"),
    "input_ids_shifted": (
        "input_ids[flat_token_index] = token_ids[(int64_t)row * token_stride + position];",
        "input_ids[flat_token_index] = token_ids[(int64_t)row * token_stride + (position > 0 ? position - 1 : 0)];"),
    "slot_drops_scale": (
        "slot_mapping[flat_token_index] = physical_block_id * block_size + offset;",
        "slot_mapping[flat_token_index] = physical_block_id + offset;"),
    "slot_drops_offset": (
        "slot_mapping[flat_token_index] = physical_block_id * block_size + offset;",
        "slot_mapping[flat_token_index] = physical_block_id * block_size;"),
    "offset_fixed_16": (
        "int32_t offset = position % block_size;",
        "int32_t offset = position & 15;"),
    "block_table_transposed": (
        "block_table[(int64_t)request_state_index * MB + logic_block];",
        "block_table[((int64_t)logic_block * R + request_state_index) % ((int64_t)R * MB)];"),
    "logic_block_rounds_up": (
        "int32_t logic_block = position / block_size;",
        "int32_t logic_block = (position + block_size - 1) / block_size;\n"
        "            if (logic_block >= MB) logic_block = MB - 1;"),
    "visible_floor": (
        "int64_t visible = seq_len <= 0 ? 0 : ((int64_t)seq_len + block_size - 1) / block_size;",
        "int64_t visible = seq_len <= 0 ? 0 : (int64_t)seq_len / block_size;"),
    "scatter_k_from_v": (
        "memcpy(kdst + slot_id * row_bytes, ksrc + (int64_t)flat_token_index * k_stride,",
        "memcpy(kdst + slot_id * row_bytes, vsrc + (int64_t)flat_token_index * v_stride,"),
    "scatter_source_row_shift": (
        "memcpy(vdst + slot_id * row_bytes, vsrc + (int64_t)flat_token_index * v_stride,",
        "memcpy(vdst + slot_id * row_bytes, vsrc + (int64_t)(flat_token_index ? flat_token_index - 1 : 0) * v_stride,"),
    "scatter_ignores_stride": (
        "memcpy(kdst + slot_id * row_bytes, ksrc + (int64_t)flat_token_index * k_stride,",
        "memcpy(kdst + slot_id * row_bytes, ksrc + (int64_t)flat_token_index * row_bytes,"),
    "add_keeps_old_blocks": (
        "block_table[(int64_t)r * MB + j] = j < given ? blocks[block_start[i] + j] : -1;",
        "if (j < given) block_table[(int64_t)r * MB + j] = blocks[block_start[i] + j];"),
    "add_ignores_computed": (
        "        completed[r] = num_computed[i];\n",
        "        completed[r] = 0;\n"),
    "append_overwrites_last": (
        "            block_table[(int64_t)r * MB + have] = blocks[block_start[i] + j];",
        "            block_table[(int64_t)r * MB + (have > 0 ? have - 1 : 0)] = blocks[block_start[i] + j];"),
    "append_forgets_count": (
        "        row_blocks[r] = (int32_t)have;",
        "        (void)have;"),
    "advance_adds_instead_of_sets": (
        "        completed[r] = seq_lens[b];",
        "        completed[r] += seq_lens[b];"),
    "advance_token_one_early": (
        "            int32_t p = seq_lens[b];",
        "            int32_t p = seq_lens[b] - 1;"),
    "gather_drops_offset": (
        "int64_t slot_id = (int64_t)physical_block_id * block_size + offset;",
        "int64_t slot_id = (int64_t)physical_block_id * block_size;"),
    "gather_start_not_running": (
        "        start += seq_len - first;",
        "        start = seq_len - first;"),
    "gather_page_of_next_request": (
        "input_block_tables[(int64_t)batch_index * MB + logic_block];",
        "input_block_tables[((int64_t)batch_index * MB + logic_block + MB) % ((int64_t)n * MB)];"),
    "gather_v_from_k": (
        "memcpy(vo + out_row * v_out_stride, vc + slot_id * row_bytes, (size_t)row_bytes);",
        "memcpy(vo + out_row * v_out_stride, kc + slot_id * row_bytes, (size_t)row_bytes);"),
    "gather_one_row_short": (
        "        for (int64_t position = first; position < seq_len; ++position) {",
        "        for (int64_t position = first; position + 1 < seq_len; ++position) {"),
    "hash_chain_drops_parent": (
        "            s = s * 1099511628211ull + c;",
        "            s = c;"),
    "hash_tokens_big_endian": (
        "                    buf[4 * j + k] = (unsigned char)(t >> (8 * k));",
        "                    buf[4 * j + k] = (unsigned char)(t >> (8 * (3 - k)));"),
    "hash_fnv1_order": (
        "        h ^= bytes[i];\n        h *= 1099511628211ull;",
        "        h *= 1099511628211ull;\n        h ^= bytes[i];"),
    "hash_counts_partial_block": (
        "            full = len / block_size;",
        "            full = (len + block_size - 1) / block_size;\n            if (starts[b] + full * block_size > total) full = len / block_size;"),
    "lookup_cap_off_by_one": (
        "        int64_t cap = len > 0 ? (len - 1) / block_size : 0;",
        "        int64_t cap = len / block_size;"),
    "lookup_skips_misses": (
        "            if (at < 0 || vals[at] == ORC_NO_BLOCK)\n                break;",
        "            if (at < 0 || vals[at] == ORC_NO_BLOCK)\n                { ++hits; continue; }"),
    "insert_keeps_last": (
        "            if (block < vals[at])\n                vals[at] = block;",
        "            vals[at] = block;"),
    "evict_unconditional": (
        "        if (at >= 0 && vals[at] == blocks[i])",
        "        if (at >= 0)"),
    "window_first_off_by_one": (
        "    int64_t first = (int64_t)seq_len - count - window + 1;",
        "    int64_t first = (int64_t)seq_len - count - window;"),
    "window_hole_flagged": (
        "                int hole = i < first_block && blk == -1;                      /* R21 */",
        "                int hole = 0;"),
    "window_read_from_zero": (
        "            first = window_first((int32_t)seq_len, count > 0 ? count : 0, sliding_window);",
        "            first = 0 * window_first((int32_t)seq_len, count > 0 ? count : 0, sliding_window);"),
    "window_free_one_too_many": (
        "            int64_t blocks = first > 0 ? first / block_size : 0;",
        "            int64_t blocks = first > 0 ? (first + block_size - 1) / block_size : 0;"),
    "lookahead_from_last_token": (
        "            int64_t position = (int64_t)seq_lens[b] + j;",
        "            int64_t position = (int64_t)seq_lens[b] + j - 1;"),
    "blocks_needed_ignores_lookahead": (
        "            int64_t tokens = (int64_t)completed[r] + add + k;",
        "            int64_t tokens = (int64_t)completed[r] + add;"),
    "pool_fifo": (
        "        int32_t r = free_rows[*num_free - 1];",
        "        int32_t r = free_rows[R - *num_free];"),
    "pool_no_duplicate_check": (
        "            if (rows[j] == rows[i])\n                return ORC_EINVAL;",
        "            (void)rows[j];"),
    "pool_release_not_in_use": (
        "        if (rows[i] < 0 || rows[i] >= R || !in_use[rows[i]])",
        "        if (rows[i] < 0 || rows[i] >= R)"),
    "bad_row_not_flagged": (
        "            st |= ORC_ST_BAD_ROW;\n            seq_lens[b] = -1;",
        "            seq_lens[b] = -1;"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} must be unique"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(source.replace(old, new))
    so = oracle.build(str(path), str(tmp_path / "liboracle_mutant.so"), strict=False)
    lib = oracle.load(so)
    # One failing pin is enough; the slowest pin (full-size caches) runs last.
    slow = [pins.pin_library_routines]
    failed = []
    for pin in [p for p in pins.ALL_PINS if p not in slow] + slow:
        try:
            pin(lib)
        except Exception:  # a wrong value, or a shape the pins cannot even build
            failed.append(pin.__name__)
            break
    assert failed, f"mutant {name} survived every pin"
