/*
 * pagedkv.h -- C ABI of libpagedkv, the MI355X (gfx950) library that turns one
 * inference step's schedule into flat GPU inputs and writes the new tokens' K/V
 * into a paged KV cache.
 *
 * The operations are those of "Deep Dive into vLLM's Scheduling Mechanism: The
 * Complete CPU-to-GPU Mapping Pipeline" (kongchang.com/en; Chinese original
 * "vLLM调度机制深度解析：CPU到GPU的完整映射流程", kongchang.com):
 *   pkv_prepare_batch        -- "Batch Construction and Sequence Flattening",
 *                               "Contiguous Token Sequence Processing", seq_lens
 *                               of "Complete Input Preparation for the Attention
 *                               Module";
 *   pkv_compute_slot_mapping -- "Multi-Layer Coordinate Conversion Pipeline" and
 *                               "Address Calculation Example", one call per
 *                               KV-cache group, plus the group's visible pages
 *                               (input_block_tables);
 *   pkv_scatter_kv           -- the write of each new token's K/V at its slot,
 *                               one call per KV-cache group and layer;
 *   pkv_step                 -- all three for a step's first layer, one launch;
 *   pkv_gather_kv            -- the read side: each request's KV range through
 *                               its visible pages ("Complete Input Preparation
 *                               for the Attention Module");
 *   pkv_hash_blocks, pkv_prefix_* -- prefix-cache block hashes and the hash
 *                               index of reusable blocks ("从源码读 vLLM
 *                               Scheduler", caffein.top: "Prefix Cache",
 *                               "allocate_slots()");
 *   pkv_add_requests, pkv_append_blocks, pkv_advance_state, pkv_row_pool_*
 *                            -- the persistent request state the path reads
 *                               ("Persistent Request Context Strategy", "Design
 *                               Logic Behind the Dual-Index System");
 *   pkv_window_free, pkv_lookahead_slots, pkv_blocks_needed, and the
 *   sliding_window arguments -- sliding-window groups and speculative
 *                               lookahead ("Scheduler.schedule()" and
 *                               "allocate_slots()" of the caffein.top article).
 *
 * Conventions shared by every call
 *   - Pointers named as device pointers must point to device memory (HBM) that
 *     the caller owns, sized as stated; the library never allocates, frees or
 *     keeps them.  Scalars are passed by value.
 *   - All index arrays are int32, contiguous, row-major.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it: it never synchronizes, never allocates and keeps no
 *     global state, so calls are reentrant.  Outputs are ready once the stream
 *     reaches the point after the call.
 *   - The return value reports errors found on the host from the arguments
 *     alone; then nothing is enqueued and no output is touched.
 *   - Errors in the *data* (found by the kernels) are OR-ed into `*status`, a
 *     device uint32 the caller zeroes (it may be NULL: checks still run, nothing
 *     is reported).  The affected outputs get the documented -1 values; no
 *     kernel ever reads or writes outside the buffers described here.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 3

/* Return codes. */
#define PKV_OK            0
#define PKV_EINVAL       (-1)  /* NULL where data is needed, negative size, block_size <= 0, ... */
#define PKV_EALIGN       (-2)  /* K/V row, stride or pointer not a multiple of 16 bytes          */
#define PKV_EUNSUPPORTED (-3)  /* beyond a documented limit (e.g. n > PKV_MAX_BATCH)             */
#define PKV_EHIP         (-4)  /* the HIP runtime refused the launch                              */
#define PKV_ENOROWS      (-5)  /* row pool: fewer free rows than asked for                       */
#define PKV_ENOMEM       (-6)  /* row pool: host memory could not be allocated                   */

/* Device status bits, OR-ed into *status. */
#define PKV_ST_BAD_ROW    0x01u /* request_state_index outside [0, R)                 */
#define PKV_ST_BAD_COUNT  0x02u /* negative scheduled-token count (read as 0)          */
#define PKV_ST_TOKEN_SUM  0x04u /* sum of scheduled counts != T                        */
#define PKV_ST_POS_OOR    0x08u /* position < 0, or >= token-table width L (input_ids)  */
#define PKV_ST_LB_OOR     0x10u /* logical block >= block-table width MB               */
#define PKV_ST_BLOCK_OOR  0x20u /* physical block id < 0 or >= num_blocks              */
#define PKV_ST_SLOT_OOR   0x40u /* slot id >= num_slots of the cache                   */
#define PKV_ST_BAD_RANGE  0x80u /* CSR offsets decreasing or outside their array       */
#define PKV_ST_TABLE_FULL 0x100u /* prefix index: no free slot for a new hash           */

/* Largest batch (scheduled requests per step) one call accepts: every
 * workgroup that orders the batch holds all of its keys in LDS. */
#define PKV_MAX_BATCH 4096

/*
 * pkv_prepare_batch -- batch assembly and flattening.
 *
 * Inputs (device):
 *   sched_rows[n]     request_state_index of each scheduled request, in any order
 *   num_scheduled[n]  tokens each request runs this step (0 allowed: an empty run)
 *   completed[R]      tokens each state row has already processed, *before* this
 *                     step (the request_state's completed_tokens)
 *   token_ids[R * token_stride]  persistent token table: token_ids[row *
 *                     token_stride + p] is the id of the row's token at position
 *                     p, valid for p < L (token_stride >= L)
 * Outputs (device):
 *   index_mapping[n]      batch_index -> request_state_index.  The batch is sorted
 *                         by tokens this step, ascending; equal counts by
 *                         request_state_index, ascending.  The result depends
 *                         only on the set of (row, count) pairs, not their order.
 *   query_start_loc[n+1]  prefix sum of the counts in batch order: request b owns
 *                         flat tokens [query_start_loc[b], query_start_loc[b+1]).
 *                         query_start_loc[0] = 0; sums saturate at INT32_MAX.
 *   seq_lens[n]           completed + count (history plus new tokens).
 *   positions[T]          completed[row] + j for the j-th token of its request.
 *   input_ids[T]          token_ids[row][position].  May be NULL (then token_ids
 *                         is not read).
 * Data errors: a row outside [0, R) flags BAD_ROW, keeps its place in the order,
 *   gets seq_len -1 and its tokens position -1 / input id -1; a negative count
 *   flags BAD_COUNT and reads as 0; sum of counts != T flags TOKEN_SUM (tokens
 *   past the last request get position -1 / input id -1, tokens beyond T are
 *   dropped); a negative position, or one >= L when input_ids is produced,
 *   flags POS_OOR and gets input id -1.
 *   Positions and seq_lens hold the low 32 bits of completed + offset.
 * Host errors: EINVAL for n < 0, T < 0, R < 0, L < 0, token_stride < L when
 *   input_ids is given, or a NULL pointer an enabled output needs;
 *   EUNSUPPORTED for n > PKV_MAX_BATCH.
 */
int pkv_prepare_batch(int32_t n, int32_t T,
                      const int32_t* sched_rows, const int32_t* num_scheduled,
                      const int32_t* completed, int32_t R,
                      const int32_t* token_ids, int64_t token_stride, int32_t L,
                      int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                      int32_t* positions, int32_t* input_ids,
                      uint32_t* status, void* stream);

/*
 * pkv_compute_slot_mapping -- physical write slots and visible pages for ONE
 * KV-cache group (each group has its own block table, block size and pool).
 *
 * Inputs (device), as produced by pkv_prepare_batch:
 *   index_mapping[n], query_start_loc[n+1] (non-decreasing, [0] = 0),
 *   seq_lens[n] (read only when input_block_tables is not NULL), positions[T]
 *   block_table[R * MB]  block_table[row * MB + i] = physical block of the row's
 *                        i-th logical block
 *   block_size, num_blocks  this group's block size and pool size;
 *                        num_blocks * block_size must fit in int32
 * Outputs (device):
 *   slot_mapping[T]      for token t of request b with row = index_mapping[b]:
 *                        slot = block_table[row][pos / block_size] * block_size
 *                               + pos % block_size,   pos = positions[t].
 *   input_block_tables[n * MB]  (may be NULL) row b = the first
 *                        ceil(seq_lens[b] / block_size) entries of the request's
 *                        block-table row; entries past them are not written.
 *   sliding_window       0 for full attention; W > 0 for a sliding-window
 *                        group (the token at position p attends p-W+1 .. p).
 *                        Batch row b (count c = query_start_loc[b+1] -
 *                        query_start_loc[b], seq_len s) then needs positions
 *                        from max(0, s - c - W + 1) on; its visible pages
 *                        before that position's block may be -1 holes left by
 *                        pkv_window_free ("allocate_slots()" of the caffein.top
 *                        page: blocks a sliding-window group no longer needs
 *                        are freed).
 * Data errors give slot -1: row outside [0, R) (BAD_ROW), position < 0
 *   (POS_OOR), logical block >= MB (LB_OOR), block id outside [0, num_blocks)
 *   (BLOCK_OOR).  Tokens outside [query_start_loc[0], query_start_loc[n]) get
 *   slot -1 unflagged.  In input_block_tables, visible entries are copied as they
 *   are (an out-of-pool one flags BLOCK_OOR, except a -1 hole before the
 *   window), a visible count above MB flags LB_OOR and is cut to MB, a bad
 *   row's output row is not written.
 * Host errors: EINVAL for n < 0, T < 0, R < 0, MB < 0, num_blocks < 0,
 *   block_size <= 0, sliding_window < 0, num_blocks * block_size > 2^31, or a
 *   NULL pointer an enabled output needs; EUNSUPPORTED for n > PKV_MAX_BATCH.
 */
int pkv_compute_slot_mapping(int32_t n, int32_t T,
                             const int32_t* index_mapping, const int32_t* query_start_loc,
                             const int32_t* seq_lens, const int32_t* positions,
                             const int32_t* block_table, int32_t R, int32_t MB,
                             int32_t block_size, int32_t num_blocks, int32_t sliding_window,
                             int32_t* slot_mapping, int32_t* input_block_tables,
                             uint32_t* status, void* stream);

/*
 * pkv_scatter_kv -- write each new token's K and V rows into ONE group's paged
 * caches for ONE layer.
 *
 *   k, v         device; token t's row of row_bytes bytes (H x D x element size)
 *                starts at k + t * k_stride (bytes), likewise v
 *   k_cache, v_cache  device, each [num_slots][row_bytes], slot-major: slot s
 *                starts at byte s * row_bytes
 *   slot_mapping[T]   device, from pkv_compute_slot_mapping
 * The payload is copied bit for bit (never converted).  A slot < 0 is skipped
 * silently (padding); a slot >= num_slots flags SLOT_OOR and is skipped.  Slots
 * must be unique among tokens with slot >= 0 (two tokens on one slot race).
 * Host errors: EINVAL for T < 0, row_bytes <= 0, num_slots < 0, a stride below
 *   row_bytes, or a NULL pointer with T > 0; EALIGN unless row_bytes, both
 *   strides and all four data pointers are multiples of 16 bytes.
 */
int pkv_scatter_kv(int32_t T, int64_t row_bytes,
                   const void* k, int64_t k_stride, const void* v, int64_t v_stride,
                   void* k_cache, void* v_cache, int64_t num_slots,
                   const int32_t* slot_mapping, uint32_t* status, void* stream);

/*
 * pkv_step -- a whole step in ONE call: pkv_prepare_batch, then for every
 * KV-cache group pkv_compute_slot_mapping and pkv_scatter_kv (the first layer's
 * K/V).  The outputs, status bits and return codes are exactly those of that
 * sequence of calls; later layers reuse each group's slot_mapping with
 * pkv_scatter_kv.  How many launches it enqueues (pkv_step_path below) depends
 * on the sizes only; the results never do.  With 1 <= num_groups <=
 * PKV_STEP_MAX_GROUPS everything runs in a single kernel launch: for batches
 * of at least PKV_STEP_RANKED_MIN_BATCH requests with few tokens each (T <= 8
 * n, or T <= 16 n past PKV_STEP_MAX_BATCH / 2 requests) one in which each
 * workgroup ranks its own requests and writes everything of theirs; else, for
 * n <= PKV_STEP_MAX_BATCH, one in which each workgroup orders the whole batch
 * and writes a tile of flat tokens -- unless the K/V strides are so large
 * that one tile's rows span more than 2^32 16-byte chunks.  Larger batches
 * with at most PKV_STEP_MAX_GROUPS groups take two kinds of launch: the batch
 * with every group's slots and visible pages, then one scatter per group;
 * more groups enqueue the separate kernels of the sequence.
 *
 * The schedule and per-request outputs are as for pkv_prepare_batch (R and the
 * token table are shared by all groups).  groups is a HOST array of num_groups
 * descriptors whose pointers are device pointers:
 *   block_table[R * MB], block_size, num_blocks     as for pkv_compute_slot_mapping
 *   slot_mapping[T] (out), input_block_tables[n * MB] (out, may be NULL)
 *   k, k_stride, v, v_stride, k_cache, v_cache, num_slots, row_bytes
 *                                                   as for pkv_scatter_kv
 *   sliding_window                                  as for pkv_compute_slot_mapping
 * Host errors: those of the three calls for the same arguments; EINVAL also for
 *   num_groups < 0 or groups == NULL with num_groups > 0.
 */
#define PKV_STEP_MAX_BATCH 512
#define PKV_STEP_MAX_GROUPS 4
#define PKV_STEP_RANKED_MIN_BATCH 32

typedef struct pkv_group {
    const int32_t* block_table;
    int32_t* slot_mapping;
    int32_t* input_block_tables;
    const void* k;
    const void* v;
    void* k_cache;
    void* v_cache;
    int64_t k_stride;
    int64_t v_stride;
    int64_t num_slots;
    int64_t row_bytes;
    int32_t MB;
    int32_t block_size;
    int32_t num_blocks;
    int32_t sliding_window;     /* 0: full attention */
} pkv_group;

int pkv_step(int32_t n, int32_t T,
             const int32_t* sched_rows, const int32_t* num_scheduled,
             const int32_t* completed, int32_t R,
             const int32_t* token_ids, int64_t token_stride, int32_t L,
             int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
             int32_t* positions, int32_t* input_ids,
             int32_t num_groups, const pkv_group* groups,
             uint32_t* status, void* stream);

/*
 * pkv_step_path -- the launch plan pkv_step takes for these arguments, without
 * enqueueing anything (host code only; it reads n, T, num_groups and, from
 * each descriptor, row_bytes, k_stride, v_stride and whether
 * input_block_tables is NULL, never the memory behind the pointers):
 *   PKV_STEP_ONE_LAUNCH          one launch; each workgroup orders the whole
 *                                batch and writes a tile of flat tokens;
 *   PKV_STEP_BATCH_THEN_SCATTER  the batch with every group's slots and pages
 *                                in one launch, then one scatter per group;
 *   PKV_STEP_SEPARATE            the kernels of pkv_prepare_batch, then of
 *                                pkv_compute_slot_mapping and pkv_scatter_kv
 *                                per group;
 *   PKV_STEP_RANKED_ONE_LAUNCH   one launch; each workgroup ranks its own
 *                                requests and writes their outputs, tokens,
 *                                slots, pages and K/V rows.
 * The plan changes only how the work is launched ("Contiguous Token Sequence
 * Processing" of the kongchang.com article: the batch is flattened so that a
 * step runs as few launches as possible); the results are the same.  EINVAL
 * for n < 0, T < 0, num_groups < 0 or groups == NULL with num_groups > 0.
 */
#define PKV_STEP_ONE_LAUNCH 0
#define PKV_STEP_BATCH_THEN_SCATTER 1
#define PKV_STEP_SEPARATE 2
#define PKV_STEP_RANKED_ONE_LAUNCH 3
int pkv_step_path(int32_t n, int32_t T, int32_t num_groups, const pkv_group* groups);

/*
 * pkv_gather_kv -- read every request's KV range through its visible pages
 * into one contiguous varlen array, for ONE group and ONE layer.  Attention
 * reads positions 0 .. seq_len-1 of each request (history plus new tokens)
 * through input_block_tables by indirect addressing ("Complete Input
 * Preparation for the Attention Module"); this call runs that address chain
 * ("Multi-Layer Coordinate Conversion Pipeline") and copies the rows out.  It
 * is the exact inverse of pkv_scatter_kv.
 *
 * Inputs (device):
 *   seq_lens[n]             as produced by pkv_prepare_batch
 *   query_start_loc[n+1], sliding_window
 *                           sliding_window 0: every position 0 .. seq_len-1 is
 *                           read (query_start_loc may be NULL).  W > 0: only
 *                           the positions some new token attends, from
 *                           first = max(0, seq_len - count - W + 1) on (count
 *                           from query_start_loc, as for
 *                           pkv_compute_slot_mapping), to rows kv_start[b] +
 *                           p - first; kv_start then sums seq_len - first.
 *   input_block_tables[n * MB]  visible pages, as produced by
 *                           pkv_compute_slot_mapping (entries past
 *                           ceil(seq_len / block_size) are never read)
 *   k_cache, v_cache        [num_blocks * block_size][row_bytes] each
 * Outputs (device):
 *   kv_start[n+1]           (may be NULL) running sum of the seq_lens,
 *                           kv_start[0] = 0, saturated at INT32_MAX
 *   k_out, v_out            row kv_start[b] + p = the K / V row of position p
 *                           of batch row b, i.e. of slot
 *                           input_block_tables[b][p / block_size] * block_size
 *                           + p % block_size; out_tokens rows, byte strides
 *                           k_out_stride / v_out_stride (rows contiguous)
 * Data errors (the row is not written; it keeps its contents): seq_len < 0
 *   counts as 0 (BAD_COUNT); a logical block >= MB (LB_OOR); a page outside
 *   [0, num_blocks) (BLOCK_OOR); rows at or past out_tokens (TOKEN_SUM).
 * Host errors: EINVAL for negative sizes, block_size <= 0, row_bytes <= 0,
 *   sliding_window < 0, strides < row_bytes, num_blocks * block_size > 2^31,
 *   or a NULL pointer that data is needed from; EALIGN unless row_bytes, the strides and every
 *   K/V pointer are multiples of 16 bytes; EUNSUPPORTED for n > PKV_MAX_BATCH,
 *   out_tokens > INT32_MAX or rows of 2^23 or more 16-byte chunks.
 */
int pkv_gather_kv(int32_t n, const int32_t* seq_lens, const int32_t* query_start_loc,
                  int32_t sliding_window, const int32_t* input_block_tables,
                  int32_t MB, int32_t block_size, int32_t num_blocks, int64_t row_bytes,
                  const void* k_cache, const void* v_cache, int64_t out_tokens, void* k_out,
                  int64_t k_out_stride, void* v_out, int64_t v_out_stride, int32_t* kv_start,
                  uint32_t* status, void* stream);

/*
 * Allocation-side variants ("从源码读 vLLM Scheduler：一轮调度如何分配请求与 KV
 * Cache", caffein.top, "Scheduler.schedule()" and "allocate_slots()": a
 * request advances towards num_tokens_with_spec, so speculative draft tokens
 * are scheduled like any others; the slots needed count computed, prefix-hit,
 * new and speculative lookahead tokens; a sliding-window group first frees the
 * blocks its attention no longer needs, and only the missing blocks are new).
 *
 * pkv_window_free: before a step, for each row rows[b], the blocks wholly
 *   before position completed[row] - W + 1 (logical blocks i < max(0,
 *   completed - W + 1) / block_size) are released: each entry >= 0 is listed
 *   in freed[b*MB ..] in block order, num_freed[b] counts them, and the entry
 *   becomes -1 (a hole).  W = 0 frees nothing.  Rows must be distinct.  Data
 *   errors: a bad row frees nothing (BAD_ROW).
 * pkv_lookahead_slots: lookahead_slots[b*k + j] = the slot of position
 *   seq_lens[b] + j of batch row b (j < k), where the next step's draft
 *   tokens go; same chain, flags and -1 as pkv_compute_slot_mapping.
 * pkv_blocks_needed: need[b] = max(0, ceil((completed[row] + num_new[b] + k) /
 *   block_size) - row_blocks[row]) for row = rows[b]: the new blocks the
 *   request must get for this step's tokens and k lookahead tokens.  Data
 *   errors: a bad row gives 0 (BAD_ROW); num_new < 0 counts as 0 (BAD_COUNT).
 * Host errors: EINVAL for negative sizes, block_size <= 0, sliding_window <
 *   0, k < 0, num_blocks * block_size > 2^31, or a NULL pointer that data is
 *   needed from.
 */
int pkv_window_free(int32_t m, const int32_t* rows, const int32_t* completed,
                    int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                    int32_t sliding_window, int32_t* freed, int32_t* num_freed,
                    uint32_t* status, void* stream);
int pkv_lookahead_slots(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                        const int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                        int32_t num_blocks, int32_t k, int32_t* lookahead_slots,
                        uint32_t* status, void* stream);
int pkv_blocks_needed(int32_t n, const int32_t* rows, const int32_t* num_new, int32_t k,
                      int32_t block_size, const int32_t* completed, const int32_t* row_blocks,
                      int32_t R, int32_t* need, uint32_t* status, void* stream);

/*
 * Prefix-cache block hashes ("从源码读 vLLM Scheduler：一轮调度如何分配请求与
 * KV Cache", caffein.top, "Prefix Cache": a request's full token blocks are
 * hashed with their prefix context and looked up in the block pool's hash
 * index; hit blocks are reused, and blocks whose contents are settled are
 * registered, "allocate_slots()").  The pages fix what the hash covers, not the
 * function; here, for full block i of a token list (tokens i*bs .. i*bs+bs-1,
 * int32 as 4 little-endian bytes):
 *   c_i = FNV-1a 64 of the block's bytes     (Fowler/Noll/Vo: basis
 *         14695981039346656037, per byte h ^= byte, h *= 1099511628211)
 *   s_i = s_{i-1} * 1099511628211 + c_i (mod 2^64), s_{-1} = 0
 *   h_i = FNV-1a 64 of s_i's 8 little-endian bytes; 0 becomes 1
 * so h_i depends on block i and every block before it.
 *
 * pkv_hash_blocks: token list b is tokens[starts[b] .. starts[b]+lengths[b])
 *   of a flat device array of `total` int32 (a CSR array, or the persistent
 *   token table with starts[b] = row * token_stride).  hashes[b*MB + i] = h_i
 *   for its floor(lengths[b] / block_size) full blocks (at most MB); entries
 *   past them are not written.  num_full[b] (may be NULL) = that count.
 *   Data errors: length < 0 counts as 0 (BAD_COUNT); a list outside
 *   [0, total) hashes nothing (BAD_RANGE); blocks past MB are not hashed
 *   (LB_OOR).  Host errors: EINVAL for m < 0, total < 0, block_size <= 0,
 *   MB < 0 or a NULL pointer that data is needed from.
 *
 * The index: keys[capacity] (uint64, 0 = unused) and vals[capacity] (int32
 * block id, INT32_MAX = none), device memory the caller owns; capacity is a
 * power of two.  An entry maps a hash to the smallest block registered for
 * it.  pkv_prefix_clear empties it.
 *
 * pkv_prefix_lookup: for request b (lengths[b] tokens, hashes from
 *   pkv_hash_blocks) the hit is the run of leading full blocks whose hashes
 *   have a block, at most floor((lengths[b]-1) / block_size) blocks (the last
 *   token is always computed again, for its logits).  num_computed[b] = hit
 *   blocks * block_size; hit_blocks[b*MB + i] (may be NULL) = the block of hit
 *   i, entries past the hit not written.  Data errors: length < 0 counts as 0
 *   (BAD_COUNT).
 * pkv_prefix_insert: registers hashes[b*MB + i] -> block_table[rows[b]*MB + i]
 *   for i in [lo[b], hi[b]).  Data errors: a bad row (BAD_ROW) or a range
 *   outside [0, MB] (BAD_RANGE) registers nothing; a block < 0 or INT32_MAX is
 *   skipped (BLOCK_OOR); a new hash finding no free slot is not registered
 *   (TABLE_FULL); a hash of 0 is ignored.  Order-independent: concurrent
 *   registrations of one hash keep the smallest block.
 * pkv_prefix_evict: entry hashes[i] loses its block if that is blocks[i] (the
 *   block was freed for other contents); an entry naming another block stays.
 *   Evicted hashes keep their slot until the next clear.
 * Host errors of the index calls: EINVAL for negative sizes, a capacity that
 *   is not a power of two (0 is allowed: nothing is ever found or stored), or
 *   a NULL pointer that data is needed from.
 */
int pkv_hash_blocks(int32_t m, const int32_t* tokens, int64_t total, const int64_t* starts,
                    const int32_t* lengths, int32_t block_size, int32_t MB, uint64_t* hashes,
                    int32_t* num_full, uint32_t* status, void* stream);
int pkv_prefix_clear(uint64_t* keys, int32_t* vals, int64_t capacity, void* stream);
int pkv_prefix_lookup(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lengths,
                      int32_t block_size, const uint64_t* keys, const int32_t* vals,
                      int64_t capacity, int32_t* hit_blocks, int32_t* num_computed,
                      uint32_t* status, void* stream);
int pkv_prefix_insert(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lo,
                      const int32_t* hi, const int32_t* rows, const int32_t* block_table,
                      int32_t R, uint64_t* keys, int32_t* vals, int64_t capacity,
                      uint32_t* status, void* stream);
int pkv_prefix_evict(int32_t count, const uint64_t* hashes, const int32_t* blocks,
                     uint64_t* keys, int32_t* vals, int64_t capacity, void* stream);

/*
 * Persistent request state ("Persistent Request Context Strategy" and "Design
 * Logic Behind the Dual-Index System" of the article above).  Per state row
 * (request_state_index) the caller keeps, in device memory:
 *   completed[R]            tokens already processed
 *   token_ids[R * token_stride]  the request's token list, positions < L
 *   block_table[R * MB]     logical block -> physical block, -1 = none
 *   row_blocks[R]           logical blocks allocated to the row (entries
 *                           0 .. row_blocks-1 of its block-table row)
 * Choosing and recycling rows is the caller's (scheduler-side) bookkeeping.
 * Ragged per-request lists come as CSR: list i is flat[start[i] .. start[i+1]),
 * start has m+1 entries and the flat array `total` entries.  Rows must be
 * distinct within one call.  Data errors (flagged in *status, never an
 * out-of-bounds access): a row outside [0, R) is skipped (BAD_ROW); a range
 * with start[i] < 0, start[i+1] < start[i] or start[i+1] > total skips its
 * request (BAD_RANGE); tokens at positions >= L are dropped (POS_OOR); block
 * ids past MB are dropped (LB_OOR).
 */

/* add_request: row rows[i] gets completed = num_computed[i], its prompt
 * tokens at positions 0.. (entries past the prompt are left as they are), its
 * blocks at logical blocks 0.. with the rest of the row set to -1, and
 * row_blocks = the number of blocks given.  Each KV-cache group has its own
 * block_table and row_blocks: register the requests in a further group by
 * calling again with that group's table and empty prompt lists (completed is
 * set to the same values again, the token table is left alone).  Host errors:
 * EINVAL for negative sizes, token_stride < L, or a NULL pointer with m > 0. */
int pkv_add_requests(int32_t m, const int32_t* rows, const int32_t* num_computed,
                     const int32_t* prompt_start, const int32_t* prompt_tokens,
                     int32_t num_prompt_tokens, const int32_t* block_start,
                     const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                     int32_t* completed, int32_t* token_ids, int64_t token_stride, int32_t L,
                     int32_t* block_table, int32_t MB, int32_t* row_blocks,
                     uint32_t* status, void* stream);

/* update_request: the new block ids of request i are appended to row
 * rows[i]'s block table after its row_blocks existing entries, and row_blocks
 * grows by as many.  Host errors: EINVAL for negative sizes or a NULL pointer
 * with m > 0. */
int pkv_append_blocks(int32_t m, const int32_t* rows, const int32_t* block_start,
                      const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                      int32_t* block_table, int32_t MB, int32_t* row_blocks,
                      uint32_t* status, void* stream);

/* After a step (index_mapping and seq_lens as produced by pkv_prepare_batch):
 * completed[index_mapping[b]] = seq_lens[b], and when sampled is not NULL and
 * sampled[b] >= 0 that token is written at position seq_lens[b] of the row's
 * token list (sampled[b] < 0: no new token, e.g. a prompt chunk that is not
 * the last).  Host errors: EINVAL for negative sizes, token_stride < L, or a
 * NULL pointer with n > 0. */
int pkv_advance_state(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                      const int32_t* sampled, int32_t R, int32_t* completed,
                      int32_t* token_ids, int64_t token_stride, int32_t L,
                      uint32_t* status, void* stream);

/*
 * Row pool (host side): request_state_index rows handed to new requests and
 * taken back from completed ones, so rows are reused instead of allocated
 * ("Design Logic Behind the Dual-Index System" of the article above).  The
 * host decides the row because the schedule names requests by it.  Free rows
 * form a stack: rows 0, 1, 2, ... come out first and the row released last is
 * handed out next.  `rows` are host arrays.  A pool is not thread-safe; it is
 * created and destroyed by the caller (the only calls here that allocate,
 * host memory only).
 *   create:  R rows, all free.  EINVAL (R < 0, out NULL), ENOMEM.
 *   acquire: m rows into rows[0..m).  ENOROWS (fewer than m free): none
 *            handed out.  EINVAL (pool NULL, m < 0, rows NULL with m > 0).
 *   release: rows[0..m) back to the pool, pushed in order.  EINVAL when a row
 *            is outside [0, R), not handed out, or listed twice: none released.
 *   num_free: free rows, -1 for a NULL pool.
 */
typedef struct pkv_row_pool pkv_row_pool;
int pkv_row_pool_create(int32_t R, pkv_row_pool** out);
void pkv_row_pool_destroy(pkv_row_pool* pool);
int pkv_row_pool_acquire(pkv_row_pool* pool, int32_t m, int32_t* rows);
int pkv_row_pool_release(pkv_row_pool* pool, int32_t m, const int32_t* rows);
int32_t pkv_row_pool_num_free(const pkv_row_pool* pool);

/* Static text for a return code (never NULL). */
const char* pkv_error_string(int code);

/* PKV_ABI_VERSION of the built library. */
int pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
