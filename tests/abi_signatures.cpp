// abi_signatures.cpp -- compile-time check of every entry point's C signature
// in include/pagedkv.h (built with g++ -fsyntax-only by tests/test_abi.py; it
// is never run).  Where the boundary differs from the interface first planned
// for the path -- the scatter's row-bytes-and-strides form, the name of the
// return-code text call, `void*` streams, the sliding-window argument of the
// slot mapping -- the signature below is the one built, so a silent change to
// any of them fails to compile.
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "pagedkv.h"

#define PKV_SIG(fn, ...) \
    static_assert(std::is_same<decltype(fn), __VA_ARGS__>::value, "signature of " #fn)

// the path
PKV_SIG(pkv_prepare_batch,
        int(int32_t n, int32_t T, const int32_t* sched_rows, const int32_t* num_scheduled,
            const int32_t* completed, int32_t R, const int32_t* token_ids, int64_t token_stride,
            int32_t L, int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
            int32_t* positions, int32_t* input_ids, uint32_t* status, void* stream));
PKV_SIG(pkv_compute_slot_mapping,
        int(int32_t n, int32_t T, const int32_t* index_mapping, const int32_t* query_start_loc,
            const int32_t* seq_lens, const int32_t* positions, const int32_t* block_table,
            int32_t R, int32_t MB, int32_t block_size, int32_t num_blocks,
            int32_t sliding_window, int32_t* slot_mapping, int32_t* input_block_tables,
            uint32_t* status, void* stream));
PKV_SIG(pkv_scatter_kv,
        int(int32_t T, int64_t row_bytes, const void* k, int64_t k_stride, const void* v,
            int64_t v_stride, void* k_cache, void* v_cache, int64_t num_slots,
            const int32_t* slot_mapping, uint32_t* status, void* stream));
PKV_SIG(pkv_step,
        int(int32_t n, int32_t T, const int32_t* sched_rows, const int32_t* num_scheduled,
            const int32_t* completed, int32_t R, const int32_t* token_ids, int64_t token_stride,
            int32_t L, int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
            int32_t* positions, int32_t* input_ids, int32_t num_groups, const pkv_group* groups,
            uint32_t* status, void* stream));
PKV_SIG(pkv_step_path, int(int32_t n, int32_t T, int32_t num_groups, const pkv_group* groups));
PKV_SIG(pkv_error_string, const char*(int code));
PKV_SIG(pkv_abi_version, int(void));

// the read side
PKV_SIG(pkv_gather_kv,
        int(int32_t n, const int32_t* seq_lens, const int32_t* query_start_loc,
            int32_t sliding_window, const int32_t* input_block_tables, int32_t MB,
            int32_t block_size, int32_t num_blocks, int64_t row_bytes, const void* k_cache,
            const void* v_cache, int64_t out_tokens, void* k_out, int64_t k_out_stride,
            void* v_out, int64_t v_out_stride, int32_t* kv_start, uint32_t* status,
            void* stream));

// variants
PKV_SIG(pkv_window_free,
        int(int32_t m, const int32_t* rows, const int32_t* completed, int32_t* block_table,
            int32_t R, int32_t MB, int32_t block_size, int32_t sliding_window, int32_t* freed,
            int32_t* num_freed, uint32_t* status, void* stream));
PKV_SIG(pkv_lookahead_slots,
        int(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
            const int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
            int32_t num_blocks, int32_t k, int32_t* lookahead_slots, uint32_t* status,
            void* stream));
PKV_SIG(pkv_blocks_needed,
        int(int32_t n, const int32_t* rows, const int32_t* num_new, int32_t k,
            int32_t block_size, const int32_t* completed, const int32_t* row_blocks, int32_t R,
            int32_t* need, uint32_t* status, void* stream));

// prefix cache
PKV_SIG(pkv_hash_blocks,
        int(int32_t m, const int32_t* tokens, int64_t total, const int64_t* starts,
            const int32_t* lengths, int32_t block_size, int32_t MB, uint64_t* hashes,
            int32_t* num_full, uint32_t* status, void* stream));
PKV_SIG(pkv_prefix_clear, int(uint64_t* keys, int32_t* vals, int64_t capacity, void* stream));
PKV_SIG(pkv_prefix_lookup,
        int(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lengths,
            int32_t block_size, const uint64_t* keys, const int32_t* vals, int64_t capacity,
            int32_t* hit_blocks, int32_t* num_computed, uint32_t* status, void* stream));
PKV_SIG(pkv_prefix_insert,
        int(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lo, const int32_t* hi,
            const int32_t* rows, const int32_t* block_table, int32_t R, uint64_t* keys,
            int32_t* vals, int64_t capacity, uint32_t* status, void* stream));
PKV_SIG(pkv_prefix_evict,
        int(int32_t count, const uint64_t* hashes, const int32_t* blocks, uint64_t* keys,
            int32_t* vals, int64_t capacity, void* stream));

// persistent state
PKV_SIG(pkv_add_requests,
        int(int32_t m, const int32_t* rows, const int32_t* num_computed,
            const int32_t* prompt_start, const int32_t* prompt_tokens, int32_t num_prompt_tokens,
            const int32_t* block_start, const int32_t* blocks, int32_t num_blocks_given,
            int32_t R, int32_t* completed, int32_t* token_ids, int64_t token_stride, int32_t L,
            int32_t* block_table, int32_t MB, int32_t* row_blocks, uint32_t* status,
            void* stream));
PKV_SIG(pkv_append_blocks,
        int(int32_t m, const int32_t* rows, const int32_t* block_start, const int32_t* blocks,
            int32_t num_blocks_given, int32_t R, int32_t* block_table, int32_t MB,
            int32_t* row_blocks, uint32_t* status, void* stream));
PKV_SIG(pkv_advance_state,
        int(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
            const int32_t* sampled, int32_t R, int32_t* completed, int32_t* token_ids,
            int64_t token_stride, int32_t L, uint32_t* status, void* stream));
PKV_SIG(pkv_row_pool_create, int(int32_t R, pkv_row_pool** out));
PKV_SIG(pkv_row_pool_destroy, void(pkv_row_pool* pool));
PKV_SIG(pkv_row_pool_acquire, int(pkv_row_pool* pool, int32_t m, int32_t* rows));
PKV_SIG(pkv_row_pool_release, int(pkv_row_pool* pool, int32_t m, const int32_t* rows));
PKV_SIG(pkv_row_pool_num_free, int32_t(const pkv_row_pool* pool));

// the group descriptor of pkv_step: field order and size as the bindings lay it out
static_assert(sizeof(pkv_group) == 104, "pkv_group size");
static_assert(offsetof(pkv_group, k_stride) == 56, "pkv_group layout");
static_assert(offsetof(pkv_group, MB) == 88, "pkv_group layout");
static_assert(offsetof(pkv_group, sliding_window) == 100, "pkv_group layout");
