// api.cpp -- the extern "C" entry points of libpagedkv: argument checks on the
// host, then stream-ordered launches.  The contract of each entry point
// (layouts, outputs, error behaviour) is stated in include/pagedkv.h.  Host
// code only: it reaches the GPU through the launchers of launchers.h alone.
#include <stdint.h>

#include "geometry.h"
#include "launchers.h"

namespace {

constexpr int64_t kMaxGridThreads = (int64_t)1 << 32;   // work-items per grid dimension

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_EHIP; }

int check_prepare(int32_t n, int32_t T, const int32_t* sched_rows, const int32_t* num_scheduled,
                  const int32_t* completed, int32_t R, const int32_t* token_ids,
                  int64_t token_stride, int32_t L, const int32_t* index_mapping,
                  const int32_t* query_start_loc, const int32_t* seq_lens,
                  const int32_t* positions, const int32_t* input_ids)
{
    if (n < 0 || T < 0 || R < 0 || L < 0)
        return PKV_EINVAL;
    if (query_start_loc == nullptr)
        return PKV_EINVAL;
    if (n > 0 && (sched_rows == nullptr || num_scheduled == nullptr || index_mapping == nullptr ||
                  seq_lens == nullptr || (R > 0 && completed == nullptr)))
        return PKV_EINVAL;
    if (T > 0 && positions == nullptr)
        return PKV_EINVAL;
    if (input_ids != nullptr && T > 0 &&
        ((R > 0 && L > 0 && token_ids == nullptr) || token_stride < L))
        return PKV_EINVAL;
    if (n > PKV_MAX_BATCH)
        return PKV_EUNSUPPORTED;
    return PKV_OK;
}

int check_slots(int32_t n, int32_t T, const int32_t* index_mapping,
                const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* positions,
                const int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                int32_t num_blocks, int32_t sliding_window, const int32_t* slot_mapping,
                const int32_t* input_block_tables)
{
    if (n < 0 || T < 0 || R < 0 || MB < 0 || num_blocks < 0 || block_size <= 0 ||
        sliding_window < 0)
        return PKV_EINVAL;
    if ((int64_t)num_blocks * block_size > (int64_t)INT32_MAX + 1)
        return PKV_EINVAL;
    if (query_start_loc == nullptr || (n > 0 && index_mapping == nullptr))
        return PKV_EINVAL;
    if (T > 0 && (positions == nullptr || slot_mapping == nullptr))
        return PKV_EINVAL;
    if ((n > 0 || T > 0) && R > 0 && MB > 0 && block_table == nullptr)
        return PKV_EINVAL;
    if (input_block_tables != nullptr && n > 0 && seq_lens == nullptr)
        return PKV_EINVAL;
    if (n > PKV_MAX_BATCH)
        return PKV_EUNSUPPORTED;
    return PKV_OK;
}

int check_scatter(int32_t T, int64_t row_bytes, const void* k, int64_t k_stride, const void* v,
                  int64_t v_stride, const void* k_cache, const void* v_cache, int64_t num_slots,
                  const int32_t* slot_mapping)
{
    if (T < 0 || row_bytes <= 0 || num_slots < 0 || k_stride < row_bytes || v_stride < row_bytes)
        return PKV_EINVAL;
    if (T > 0 && (k == nullptr || v == nullptr || slot_mapping == nullptr ||
                  (num_slots > 0 && (k_cache == nullptr || v_cache == nullptr))))
        return PKV_EINVAL;
    if ((row_bytes & 15) != 0 || (k_stride & 15) != 0 || (v_stride & 15) != 0 || !aligned16(k) ||
        !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_EALIGN;
    // One lane per 16-byte chunk, a quarter of the chunks per lane at most.
    if ((int64_t)T * (row_bytes / 16) / 4 >= kMaxGridThreads)
        return PKV_EUNSUPPORTED;
    return PKV_OK;
}

// The launch plan of pkv_step (pkv_step_path's value), measured on MI355X
// (back-to-back steps, 8 x 128 bf16 rows, block size 16):
//   - Batches of at least PKV_STEP_RANKED_MIN_BATCH requests with few tokens
//     each (T <= 8 n, or T <= 16 n past 256 requests), 1-4 groups: one launch
//     in which each workgroup ranks its own requests and writes their
//     outputs, tokens, slots, pages and K/V rows -- no workgroup orders the
//     whole batch.  256 decodes 10.1 -> 7.8 us, 64 decodes 9.9 -> 7.4, 32
//     requests x 8 tokens 8.5 -> 7.9, 512 x 8 17.1 -> 11.7, 512 x 16 22.0 ->
//     17.2, 4096 decodes 19.7 -> 18.1; smaller batches stay faster in the
//     tile launch (2 requests x 4 tokens 6.2 against 7.2, 16 x 16 7.9 against
//     8.3), and so do longer requests (128 x 16 10.1 against 10.6, 256 x 32
//     16.5 against 17.0).
//   - Otherwise one launch of the tile kernel (k_step) whenever the batch fits
//     the in-LDS ordering of every workgroup, the group count fits the kernel
//     arguments, the grid fits one dimension and each group's tile rows can
//     be addressed by 32-bit chunk offsets.
//   - Otherwise, up to PKV_STEP_MAX_GROUPS groups: the batch with every
//     group's slots and pages, then the scatters; more groups: the separate
//     kernels.
int step_path(int32_t n, int32_t T, int32_t num_groups, const pkv_group* groups)
{
    const bool groups_fit = num_groups >= 1 && num_groups <= PKV_STEP_MAX_GROUPS;
    const int64_t per = n > PKV_STEP_MAX_BATCH / 2 ? 16 : 8;   // tokens per request, on average
    if (groups_fit && n >= PKV_STEP_RANKED_MIN_BATCH && (int64_t)T <= per * (int64_t)n)
        return PKV_STEP_RANKED_ONE_LAUNCH;
    bool fused = n <= PKV_STEP_MAX_BATCH && groups_fit &&
                 pkv::step_grid_blocks(n, T, num_groups, groups) * pkv::kStepThreads <
                     kMaxGridThreads;
    for (int i = 0; fused && i < num_groups; ++i)
        fused = pkv::step_offsets_fit(groups[i]);
    if (fused)
        return PKV_STEP_ONE_LAUNCH;
    return num_groups <= PKV_STEP_MAX_GROUPS ? PKV_STEP_BATCH_THEN_SCATTER : PKV_STEP_SEPARATE;
}

}  // namespace

extern "C" {

int pkv_prepare_batch(int32_t n, int32_t T, const int32_t* sched_rows,
                      const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                      const int32_t* token_ids, int64_t token_stride, int32_t L,
                      int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                      int32_t* positions, int32_t* input_ids, uint32_t* status, void* stream)
{
    const int rc = check_prepare(n, T, sched_rows, num_scheduled, completed, R, token_ids,
                                 token_stride, L, index_mapping, query_start_loc, seq_lens,
                                 positions, input_ids);
    if (rc != PKV_OK)
        return rc;
    return from_hip(pkv::launch_prepare(n, T, sched_rows, num_scheduled, completed, R, token_ids,
                                        token_stride, L, index_mapping, query_start_loc, seq_lens,
                                        positions, input_ids, 0, nullptr, false, status,
                                        static_cast<hipStream_t>(stream)));
}

int pkv_compute_slot_mapping(int32_t n, int32_t T, const int32_t* index_mapping,
                             const int32_t* query_start_loc, const int32_t* seq_lens,
                             const int32_t* positions, const int32_t* block_table, int32_t R,
                             int32_t MB, int32_t block_size, int32_t num_blocks,
                             int32_t sliding_window, int32_t* slot_mapping,
                             int32_t* input_block_tables, uint32_t* status, void* stream)
{
    const int rc = check_slots(n, T, index_mapping, query_start_loc, seq_lens, positions,
                               block_table, R, MB, block_size, num_blocks, sliding_window,
                               slot_mapping, input_block_tables);
    if (rc != PKV_OK)
        return rc;
    return from_hip(pkv::launch_slots(n, T, index_mapping, query_start_loc, seq_lens, positions,
                                      block_table, R, MB, block_size, num_blocks, sliding_window,
                                      slot_mapping, input_block_tables, status,
                                      static_cast<hipStream_t>(stream)));
}

int pkv_scatter_kv(int32_t T, int64_t row_bytes, const void* k, int64_t k_stride, const void* v,
                   int64_t v_stride, void* k_cache, void* v_cache, int64_t num_slots,
                   const int32_t* slot_mapping, uint32_t* status, void* stream)
{
    const int rc = check_scatter(T, row_bytes, k, k_stride, v, v_stride, k_cache, v_cache,
                                 num_slots, slot_mapping);
    if (rc != PKV_OK)
        return rc;
    return from_hip(pkv::launch_scatter(T, row_bytes, k, k_stride, v, v_stride, k_cache, v_cache,
                                        num_slots, slot_mapping, status,
                                        static_cast<hipStream_t>(stream)));
}

int pkv_step(int32_t n, int32_t T, const int32_t* sched_rows, const int32_t* num_scheduled,
             const int32_t* completed, int32_t R, const int32_t* token_ids, int64_t token_stride,
             int32_t L, int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
             int32_t* positions, int32_t* input_ids, int32_t num_groups, const pkv_group* groups,
             uint32_t* status, void* stream)
{
    if (num_groups < 0 || (num_groups > 0 && groups == nullptr))
        return PKV_EINVAL;
    int rc = check_prepare(n, T, sched_rows, num_scheduled, completed, R, token_ids, token_stride,
                           L, index_mapping, query_start_loc, seq_lens, positions, input_ids);
    if (rc != PKV_OK)
        return rc;
    for (int i = 0; i < num_groups; ++i) {
        const pkv_group& g = groups[i];
        rc = check_slots(n, T, index_mapping, query_start_loc, seq_lens, positions, g.block_table,
                         R, g.MB, g.block_size, g.num_blocks, g.sliding_window, g.slot_mapping,
                         g.input_block_tables);
        if (rc != PKV_OK)
            return rc;
        rc = check_scatter(T, g.row_bytes, g.k, g.k_stride, g.v, g.v_stride, g.k_cache,
                           g.v_cache, g.num_slots, g.slot_mapping);
        if (rc != PKV_OK)
            return rc;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int path = step_path(n, T, num_groups, groups);
    if (path == PKV_STEP_ONE_LAUNCH)
        return from_hip(pkv::launch_step(n, T, sched_rows, num_scheduled, completed, R, token_ids,
                                         token_stride, L, index_mapping, query_start_loc,
                                         seq_lens, positions, input_ids, num_groups, groups,
                                         status, s));
    if (path == PKV_STEP_RANKED_ONE_LAUNCH)
        return from_hip(pkv::launch_prepare(n, T, sched_rows, num_scheduled, completed, R,
                                            token_ids, token_stride, L, index_mapping,
                                            query_start_loc, seq_lens, positions, input_ids,
                                            num_groups, groups, true, status, s));
    // Past the one-launch limits: the batch and, for up to PKV_STEP_MAX_GROUPS
    // groups, their slots and pages in one launch; then one scatter per group.
    const bool with_slots = path == PKV_STEP_BATCH_THEN_SCATTER;
    hipError_t e = pkv::launch_prepare(n, T, sched_rows, num_scheduled, completed, R, token_ids,
                                       token_stride, L, index_mapping, query_start_loc, seq_lens,
                                       positions, input_ids, with_slots ? num_groups : 0,
                                       groups, false, status, s);
    for (int i = 0; !with_slots && e == hipSuccess && i < num_groups; ++i) {
        const pkv_group& g = groups[i];
        e = pkv::launch_slots(n, T, index_mapping, query_start_loc, seq_lens, positions,
                              g.block_table, R, g.MB, g.block_size, g.num_blocks,
                              g.sliding_window, g.slot_mapping, g.input_block_tables, status, s);
    }
    for (int i = 0; e == hipSuccess && i < num_groups; ++i) {
        const pkv_group& g = groups[i];
        e = pkv::launch_scatter(T, g.row_bytes, g.k, g.k_stride, g.v, g.v_stride, g.k_cache,
                                g.v_cache, g.num_slots, g.slot_mapping, status, s);
    }
    return from_hip(e);
}

int pkv_step_path(int32_t n, int32_t T, int32_t num_groups, const pkv_group* groups)
{
    if (n < 0 || T < 0 || num_groups < 0 || (num_groups > 0 && groups == nullptr))
        return PKV_EINVAL;
    return step_path(n, T, num_groups, groups);
}

int pkv_gather_kv(int32_t n, const int32_t* seq_lens, const int32_t* query_start_loc,
                  int32_t sliding_window, const int32_t* input_block_tables,
                  int32_t MB, int32_t block_size, int32_t num_blocks, int64_t row_bytes,
                  const void* k_cache, const void* v_cache, int64_t out_tokens, void* k_out,
                  int64_t k_out_stride, void* v_out, int64_t v_out_stride, int32_t* kv_start,
                  uint32_t* status, void* stream)
{
    if (n < 0 || MB < 0 || block_size <= 0 || num_blocks < 0 || row_bytes <= 0 ||
        out_tokens < 0 || k_out_stride < row_bytes || v_out_stride < row_bytes ||
        sliding_window < 0)
        return PKV_EINVAL;
    if ((int64_t)num_blocks * block_size > (int64_t)INT32_MAX + 1)
        return PKV_EINVAL;
    if (n > 0 && (seq_lens == nullptr || (MB > 0 && input_block_tables == nullptr) ||
                  (sliding_window > 0 && query_start_loc == nullptr)))
        return PKV_EINVAL;
    if (out_tokens > 0 && (k_out == nullptr || v_out == nullptr))
        return PKV_EINVAL;
    if (num_blocks > 0 && (k_cache == nullptr || v_cache == nullptr))
        return PKV_EINVAL;
    if ((row_bytes & 15) != 0 || (k_out_stride & 15) != 0 || (v_out_stride & 15) != 0 ||
        !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out))
        return PKV_EALIGN;
    if (n > PKV_MAX_BATCH || out_tokens > INT32_MAX || row_bytes / 16 >= (int64_t)1 << 23)
        return PKV_EUNSUPPORTED;
    return from_hip(pkv::launch_gather(n, seq_lens, query_start_loc, sliding_window,
                                       input_block_tables, MB, block_size, num_blocks,
                                       row_bytes, k_cache, v_cache, (int32_t)out_tokens, k_out,
                                       k_out_stride, v_out, v_out_stride, kv_start, status,
                                       static_cast<hipStream_t>(stream)));
}

int pkv_window_free(int32_t m, const int32_t* rows, const int32_t* completed,
                    int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                    int32_t sliding_window, int32_t* freed, int32_t* num_freed,
                    uint32_t* status, void* stream)
{
    if (m < 0 || R < 0 || MB < 0 || block_size <= 0 || sliding_window < 0)
        return PKV_EINVAL;
    if (m > 0 && (rows == nullptr || num_freed == nullptr || (R > 0 && completed == nullptr) ||
                  (MB > 0 && (freed == nullptr || (R > 0 && block_table == nullptr)))))
        return PKV_EINVAL;
    return from_hip(pkv::launch_window_free(m, rows, completed, block_table, R, MB, block_size,
                                            sliding_window, freed, num_freed, status,
                                            static_cast<hipStream_t>(stream)));
}

int pkv_lookahead_slots(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                        const int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                        int32_t num_blocks, int32_t k, int32_t* lookahead_slots,
                        uint32_t* status, void* stream)
{
    if (n < 0 || R < 0 || MB < 0 || block_size <= 0 || num_blocks < 0 || k < 0)
        return PKV_EINVAL;
    if ((int64_t)num_blocks * block_size > (int64_t)INT32_MAX + 1)
        return PKV_EINVAL;
    if (n > 0 && k > 0 &&
        (index_mapping == nullptr || seq_lens == nullptr || lookahead_slots == nullptr ||
         (R > 0 && MB > 0 && block_table == nullptr)))
        return PKV_EINVAL;
    return from_hip(pkv::launch_lookahead_slots(n, index_mapping, seq_lens, block_table, R, MB,
                                                block_size, num_blocks, k, lookahead_slots, status,
                                                static_cast<hipStream_t>(stream)));
}

int pkv_blocks_needed(int32_t n, const int32_t* rows, const int32_t* num_new, int32_t k,
                      int32_t block_size, const int32_t* completed, const int32_t* row_blocks,
                      int32_t R, int32_t* need, uint32_t* status, void* stream)
{
    if (n < 0 || k < 0 || block_size <= 0 || R < 0)
        return PKV_EINVAL;
    if (n > 0 && (rows == nullptr || num_new == nullptr || need == nullptr ||
                  (R > 0 && (completed == nullptr || row_blocks == nullptr))))
        return PKV_EINVAL;
    return from_hip(pkv::launch_blocks_needed(n, rows, num_new, k, block_size, completed,
                                              row_blocks, R, need, status,
                                              static_cast<hipStream_t>(stream)));
}

int pkv_hash_blocks(int32_t m, const int32_t* tokens, int64_t total, const int64_t* starts,
                    const int32_t* lengths, int32_t block_size, int32_t MB, uint64_t* hashes,
                    int32_t* num_full, uint32_t* status, void* stream)
{
    if (m < 0 || total < 0 || block_size <= 0 || MB < 0)
        return PKV_EINVAL;
    if (m > 0 && (starts == nullptr || lengths == nullptr || (MB > 0 && hashes == nullptr) ||
                  (total > 0 && tokens == nullptr)))
        return PKV_EINVAL;
    return from_hip(pkv::launch_hash_blocks(m, tokens, total, starts, lengths, block_size, MB,
                                            hashes, num_full, status,
                                            static_cast<hipStream_t>(stream)));
}

namespace {
bool bad_capacity(int64_t capacity) { return capacity < 0 || (capacity & (capacity - 1)) != 0; }
}  // namespace

int pkv_prefix_clear(uint64_t* keys, int32_t* vals, int64_t capacity, void* stream)
{
    if (bad_capacity(capacity) || (capacity > 0 && (keys == nullptr || vals == nullptr)))
        return PKV_EINVAL;
    return from_hip(
        pkv::launch_prefix_clear(keys, vals, capacity, static_cast<hipStream_t>(stream)));
}

int pkv_prefix_lookup(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lengths,
                      int32_t block_size, const uint64_t* keys, const int32_t* vals,
                      int64_t capacity, int32_t* hit_blocks, int32_t* num_computed,
                      uint32_t* status, void* stream)
{
    if (m < 0 || MB < 0 || block_size <= 0 || bad_capacity(capacity))
        return PKV_EINVAL;
    if (m > 0 && (lengths == nullptr || num_computed == nullptr ||
                  (MB > 0 && hashes == nullptr) ||
                  (capacity > 0 && (keys == nullptr || vals == nullptr))))
        return PKV_EINVAL;
    return from_hip(pkv::launch_prefix_lookup(m, hashes, MB, lengths, block_size, keys, vals,
                                              capacity, hit_blocks, num_computed, status,
                                              static_cast<hipStream_t>(stream)));
}

int pkv_prefix_insert(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lo,
                      const int32_t* hi, const int32_t* rows, const int32_t* block_table,
                      int32_t R, uint64_t* keys, int32_t* vals, int64_t capacity,
                      uint32_t* status, void* stream)
{
    if (m < 0 || MB < 0 || R < 0 || bad_capacity(capacity))
        return PKV_EINVAL;
    if (m > 0 && (lo == nullptr || hi == nullptr || rows == nullptr ||
                  (MB > 0 && (hashes == nullptr || (R > 0 && block_table == nullptr))) ||
                  (capacity > 0 && (keys == nullptr || vals == nullptr))))
        return PKV_EINVAL;
    return from_hip(pkv::launch_prefix_insert(m, hashes, MB, lo, hi, rows, block_table, R, keys,
                                              vals, capacity, status,
                                              static_cast<hipStream_t>(stream)));
}

int pkv_prefix_evict(int32_t count, const uint64_t* hashes, const int32_t* blocks,
                     uint64_t* keys, int32_t* vals, int64_t capacity, void* stream)
{
    if (count < 0 || bad_capacity(capacity))
        return PKV_EINVAL;
    if (count > 0 && (hashes == nullptr || blocks == nullptr ||
                      (capacity > 0 && (keys == nullptr || vals == nullptr))))
        return PKV_EINVAL;
    return from_hip(pkv::launch_prefix_evict(count, hashes, blocks, keys, vals, capacity,
                                             static_cast<hipStream_t>(stream)));
}

int pkv_add_requests(int32_t m, const int32_t* rows, const int32_t* num_computed,
                     const int32_t* prompt_start, const int32_t* prompt_tokens,
                     int32_t num_prompt_tokens, const int32_t* block_start, const int32_t* blocks,
                     int32_t num_blocks_given, int32_t R, int32_t* completed, int32_t* token_ids,
                     int64_t token_stride, int32_t L, int32_t* block_table, int32_t MB,
                     int32_t* row_blocks, uint32_t* status, void* stream)
{
    if (m < 0 || R < 0 || L < 0 || MB < 0 || token_stride < L || num_prompt_tokens < 0 ||
        num_blocks_given < 0)
        return PKV_EINVAL;
    if (m > 0 && (rows == nullptr || num_computed == nullptr || prompt_start == nullptr ||
                  block_start == nullptr || (num_prompt_tokens > 0 && prompt_tokens == nullptr) ||
                  (num_blocks_given > 0 && blocks == nullptr) ||
                  (R > 0 && (completed == nullptr || row_blocks == nullptr ||
                             (L > 0 && token_ids == nullptr) ||
                             (MB > 0 && block_table == nullptr)))))
        return PKV_EINVAL;
    return from_hip(pkv::launch_add_requests(m, rows, num_computed, prompt_start, prompt_tokens,
                                             num_prompt_tokens, block_start, blocks,
                                             num_blocks_given, R, completed, token_ids,
                                             token_stride, L, block_table, MB, row_blocks, status,
                                             static_cast<hipStream_t>(stream)));
}

int pkv_append_blocks(int32_t m, const int32_t* rows, const int32_t* block_start,
                      const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                      int32_t* block_table, int32_t MB, int32_t* row_blocks, uint32_t* status,
                      void* stream)
{
    if (m < 0 || R < 0 || MB < 0 || num_blocks_given < 0)
        return PKV_EINVAL;
    if (m > 0 && (rows == nullptr || block_start == nullptr ||
                  (num_blocks_given > 0 && blocks == nullptr) ||
                  (R > 0 && (row_blocks == nullptr || (MB > 0 && block_table == nullptr)))))
        return PKV_EINVAL;
    return from_hip(pkv::launch_append_blocks(m, rows, block_start, blocks, num_blocks_given, R,
                                              block_table, MB, row_blocks, status,
                                              static_cast<hipStream_t>(stream)));
}

int pkv_advance_state(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                      const int32_t* sampled, int32_t R, int32_t* completed, int32_t* token_ids,
                      int64_t token_stride, int32_t L, uint32_t* status, void* stream)
{
    if (n < 0 || R < 0 || L < 0 || token_stride < L)
        return PKV_EINVAL;
    if (n > 0 && (index_mapping == nullptr || seq_lens == nullptr ||
                  (R > 0 && completed == nullptr) ||
                  (sampled != nullptr && R > 0 && L > 0 && token_ids == nullptr)))
        return PKV_EINVAL;
    return from_hip(pkv::launch_advance_state(n, index_mapping, seq_lens, sampled, R, completed,
                                              token_ids, token_stride, L, status,
                                              static_cast<hipStream_t>(stream)));
}

const char* pkv_error_string(int code)
{
    switch (code) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EALIGN: return "K/V rows, strides and pointers must be 16-byte aligned";
    case PKV_EUNSUPPORTED: return "beyond a documented limit of the library";
    case PKV_EHIP: return "HIP launch failed";
    case PKV_ENOROWS: return "row pool: fewer free rows than asked for";
    case PKV_ENOMEM: return "row pool: out of host memory";
    default: return "unknown pagedkv error code";
    }
}

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

}  // extern "C"
