// launchers.h -- host-side launchers of libpagedkv's kernels, called by the C
// entry points in api.cpp.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// Launchers (host side).  Arguments are already validated; each returns a
// hipError_t from the launch.

// Batch assembly and flattening; with 1 <= num_groups <= PKV_STEP_MAX_GROUPS
// also every group's slots and visible pages (those of launch_slots), and
// with with_scatter also every group's K/V write (that of launch_scatter), in
// the same launch.  num_groups = 0: the batch alone.
hipError_t launch_prepare(int32_t n, int32_t T, const int32_t* sched_rows,
                          const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                          const int32_t* token_ids, int64_t token_stride, int32_t L,
                          int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                          int32_t* positions, int32_t* input_ids, int32_t num_groups,
                          const pkv_group* groups, bool with_scatter, uint32_t* status,
                          hipStream_t stream);

hipError_t launch_slots(int32_t n, int32_t T, const int32_t* index_mapping,
                        const int32_t* query_start_loc, const int32_t* seq_lens,
                        const int32_t* positions, const int32_t* block_table, int32_t R,
                        int32_t MB, int32_t block_size, int32_t num_blocks,
                        int32_t sliding_window, int32_t* slot_mapping,
                        int32_t* input_block_tables, uint32_t* status, hipStream_t stream);

hipError_t launch_step(int32_t n, int32_t T, const int32_t* sched_rows,
                       const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                       const int32_t* token_ids, int64_t token_stride, int32_t L,
                       int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                       int32_t* positions, int32_t* input_ids, int32_t num_groups,
                       const pkv_group* groups, uint32_t* status, hipStream_t stream);

hipError_t launch_gather(int32_t n, const int32_t* seq_lens, const int32_t* query_start_loc,
                         int32_t sliding_window, const int32_t* input_block_tables, int32_t MB,
                         int32_t block_size, int32_t num_blocks, int64_t row_bytes,
                         const void* k_cache, const void* v_cache, int32_t out_tokens,
                         void* k_out, int64_t k_out_stride, void* v_out, int64_t v_out_stride,
                         int32_t* kv_start, uint32_t* status, hipStream_t stream);

hipError_t launch_add_requests(int32_t m, const int32_t* rows, const int32_t* num_computed,
                               const int32_t* prompt_start, const int32_t* prompt_tokens,
                               int32_t num_prompt_tokens, const int32_t* block_start,
                               const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                               int32_t* completed, int32_t* token_ids, int64_t token_stride,
                               int32_t L, int32_t* block_table, int32_t MB, int32_t* row_blocks,
                               uint32_t* status, hipStream_t stream);

hipError_t launch_append_blocks(int32_t m, const int32_t* rows, const int32_t* block_start,
                                const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                                int32_t* block_table, int32_t MB, int32_t* row_blocks,
                                uint32_t* status, hipStream_t stream);

hipError_t launch_advance_state(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                                const int32_t* sampled, int32_t R, int32_t* completed,
                                int32_t* token_ids, int64_t token_stride, int32_t L,
                                uint32_t* status, hipStream_t stream);

hipError_t launch_scatter(int32_t T, int64_t row_bytes, const void* k, int64_t k_stride,
                          const void* v, int64_t v_stride, void* k_cache, void* v_cache,
                          int64_t num_slots, const int32_t* slot_mapping, uint32_t* status,
                          hipStream_t stream);

hipError_t launch_window_free(int32_t m, const int32_t* rows, const int32_t* completed,
                              int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                              int32_t sliding_window, int32_t* freed, int32_t* num_freed,
                              uint32_t* status, hipStream_t stream);

hipError_t launch_lookahead_slots(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                                  const int32_t* block_table, int32_t R, int32_t MB,
                                  int32_t block_size, int32_t num_blocks, int32_t k,
                                  int32_t* lookahead_slots, uint32_t* status, hipStream_t stream);

hipError_t launch_blocks_needed(int32_t n, const int32_t* rows, const int32_t* num_new, int32_t k,
                                int32_t block_size, const int32_t* completed,
                                const int32_t* row_blocks, int32_t R, int32_t* need,
                                uint32_t* status, hipStream_t stream);

hipError_t launch_hash_blocks(int32_t m, const int32_t* tokens, int64_t total,
                              const int64_t* starts, const int32_t* lengths, int32_t block_size,
                              int32_t MB, uint64_t* hashes, int32_t* num_full, uint32_t* status,
                              hipStream_t stream);

hipError_t launch_prefix_lookup(int32_t m, const uint64_t* hashes, int32_t MB,
                                const int32_t* lengths, int32_t block_size, const uint64_t* keys,
                                const int32_t* vals, int64_t capacity, int32_t* hit_blocks,
                                int32_t* num_computed, uint32_t* status, hipStream_t stream);

hipError_t launch_prefix_insert(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lo,
                                const int32_t* hi, const int32_t* rows,
                                const int32_t* block_table, int32_t R, uint64_t* keys,
                                int32_t* vals, int64_t capacity, uint32_t* status,
                                hipStream_t stream);

hipError_t launch_prefix_evict(int32_t count, const uint64_t* hashes, const int32_t* blocks,
                               uint64_t* keys, int32_t* vals, int64_t capacity,
                               hipStream_t stream);

hipError_t launch_prefix_clear(uint64_t* keys, int32_t* vals, int64_t capacity,
                               hipStream_t stream);

}  // namespace pkv
