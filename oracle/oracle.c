/*
 * oracle.c -- plain CPU oracle of the schedule -> flat GPU inputs -> paged K/V
 * write chain.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference for the HIP
 * library in paged_kv_input_amd/.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product never does.  It shares no
 * source, header, helper or constant table with the HIP library: the numeric
 * values of return codes and status bits below restate the public contract and
 * are compared, not shared.
 *
 * It is written to be checked by eye against the pages, not to be fast: one
 * thread, plain loops, a library sort.  Sources, cited by title and section:
 *
 *   [KC]  "Deep Dive into vLLM's Scheduling Mechanism: The Complete CPU-to-GPU
 *         Mapping Pipeline" (kongchang.com/en) and its Chinese original
 *         "vLLM调度机制深度解析：CPU到GPU的完整映射流程" (kongchang.com).
 *   [CF]  "从源码读 vLLM Scheduler：一轮调度如何分配请求与 KV Cache" (caffein.top).
 *
 * Notation follows [KC] "Summary of the Four Index Space Mappings":
 * request_state_index (row of the worker's persistent state), batch_index (row
 * of this step's compact batch), flat_token_index (position in the flattened
 * token sequence) and position (the token's ordinal inside its own request).
 *
 * Pins (all in tests/, run on the CPU): every function here is pinned.
 *   orc_prepare_batch        -- [KC] worked example values (golden file), the
 *                               [CF] prefix example, brute-force loops on tiny
 *                               batches, NumPy lexsort/cumsum/repeat, closed-form
 *                               token table, invariants.
 *   orc_compute_slot_mapping -- the printed slot 207 and its derived neighbours,
 *                               a paged address space enumerated block by block
 *                               (no division), the contiguous-table closed form,
 *                               block size 1, invariants.
 *   orc_scatter_kv           -- NumPy fancy-index assignment, gather round trip,
 *                               sentinel count.
 *   orc_add_requests,        -- the [KC] worked example's state rebuilt from
 *   orc_append_blocks,          nothing, the [CF] prefix example's [P1][P2][B3]
 *   orc_advance_state           table (reuse, then one appended block), brute-
 *                               force state loops, a multi-step decode loop.
 *   orc_gather_kv            -- the [KC] example read back (slot 207 holds B's
 *                               new token), the inverse of the scatter,
 *                               addresses enumerated block by block, the
 *                               contiguous-table closed form, block size 1.
 *   orc_hash_blocks          -- FNV-1a's published test vectors, the chain's
 *                               closed form (a sum of powers), the [CF] shared
 *                               system prompt (equal hashes for equal prefixes).
 *   orc_prefix_*             -- the [CF] example (B hits P1, P2: 8 tokens),
 *                               the hit cap, a Python dict model of the index.
 *   orc_pool_*               -- a Python list used as a stack, run on random
 *                               acquire/release sequences; invariants (no row
 *                               out twice, free + in use = R).
 * Readings of points the pages leave open are listed at each step (R1..R9).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Return codes (host-detectable argument errors). */
#define ORC_OK       0
#define ORC_EINVAL  (-1)
#define ORC_ENOROWS (-5)  /* row pool: fewer free rows than asked for */

/* Status bits (data errors found while computing; OR-ed into *status). */
#define ORC_ST_BAD_ROW    0x01u  /* request_state_index outside [0, R)            */
#define ORC_ST_BAD_COUNT  0x02u  /* negative scheduled-token count                */
#define ORC_ST_TOKEN_SUM  0x04u  /* sum of scheduled counts != T                  */
#define ORC_ST_POS_OOR    0x08u  /* position < 0, or >= token-table width         */
#define ORC_ST_LB_OOR     0x10u  /* logic_block >= block-table width              */
#define ORC_ST_BLOCK_OOR  0x20u  /* physical_block_id < 0 or >= pool size         */
#define ORC_ST_SLOT_OOR   0x40u  /* slot_id >= cache slots                        */
#define ORC_ST_BAD_RANGE  0x80u  /* CSR offsets decreasing or outside the array   */
#define ORC_ST_TABLE_FULL 0x100u /* prefix index: no free slot for a new key      */

/* One scheduled request while the batch is being assembled. */
typedef struct {
    int32_t tokens_this_step;     /* num_scheduled (negative counts read as 0) */
    int32_t request_state_index;  /* the request's row in the persistent state */
} sched_req;

/*
 * [KC] "Extracting the Execution Batch from Global State": the batch is ordered
 * by the number of tokens each request executes this step.
 * R1 (direction): ascending -- the only order that gives the printed
 *     query_start_loc [0, 1, 9] (the 1-token request B before the 8-token A).
 * R2 (ties): smaller request_state_index first, so the batch depends only on
 *     which requests are scheduled, not on the order the host listed them.
 */
static int by_tokens_then_row(const void* pa, const void* pb)
{
    const sched_req* a = (const sched_req*)pa;
    const sched_req* b = (const sched_req*)pb;
    if (a->tokens_this_step != b->tokens_this_step)
        return a->tokens_this_step < b->tokens_this_step ? -1 : 1;
    if (a->request_state_index != b->request_state_index)
        return a->request_state_index < b->request_state_index ? -1 : 1;
    return 0;
}

/*
 * Batch assembly and flattening ([KC] "Batch Construction and Sequence
 * Flattening" and "Contiguous Token Sequence Processing"; seq_lens from
 * "Complete Input Preparation for the Attention Module").
 *
 *   sched_rows[n], num_scheduled[n]  this step's schedule, in host order
 *   completed[R]                     tokens each state row has already processed
 *   token_ids[R * token_stride]      the persistent token table, row-major
 *   outputs: index_mapping[n], query_start_loc[n+1], seq_lens[n],
 *            positions[T], input_ids[T] (input_ids may be NULL: not produced)
 *
 * R3: a position starts at completed_tokens, the value *before* this step
 *     (31 done -> position 31; 16 done -> positions 16..23 in the example).
 * R4: input_ids[t] = token_ids[row][position]: the request's token list read at
 *     the token's own position, kept as a persistent per-row table.
 * R5: seq_lens[b] = completed + tokens this step (history plus new).
 * R6 (data errors, never out-of-bounds accesses): a row outside [0, R) leaves
 *     its request in the batch order with seq_len -1 and its tokens at position
 *     -1 / input id -1; a negative count is read as 0; prefix sums saturate at
 *     INT32_MAX; tokens past the last request (sum < T) get position -1 and
 *     input id -1; tokens beyond T (sum > T) are dropped; a negative position,
 *     or one >= L when input_ids are produced, is flagged and gets input id -1.
 *     Positions and seq_lens keep the low 32 bits of the 64-bit sum.
 */
int orc_prepare_batch(int32_t n, int32_t T,
                      const int32_t* sched_rows, const int32_t* num_scheduled,
                      const int32_t* completed, int32_t R,
                      const int32_t* token_ids, int64_t token_stride, int32_t L,
                      int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                      int32_t* positions, int32_t* input_ids, uint32_t* status)
{
    if (n < 0 || T < 0 || R < 0 || L < 0)
        return ORC_EINVAL;
    if (query_start_loc == NULL)
        return ORC_EINVAL;
    if (n > 0 && (sched_rows == NULL || num_scheduled == NULL || index_mapping == NULL ||
                  seq_lens == NULL || (R > 0 && completed == NULL)))
        return ORC_EINVAL;
    if (T > 0 && positions == NULL)
        return ORC_EINVAL;
    if (input_ids != NULL && T > 0 && ((R > 0 && L > 0 && token_ids == NULL) || token_stride < L))
        return ORC_EINVAL;

    uint32_t st = 0;

    /* Step 1 -- extract the relevant requests from global state. */
    sched_req* batch = (sched_req*)malloc(sizeof(sched_req) * (size_t)(n > 0 ? n : 1));
    if (batch == NULL)
        return ORC_EINVAL;
    for (int32_t i = 0; i < n; ++i) {
        int32_t count = num_scheduled[i];
        if (count < 0) {
            st |= ORC_ST_BAD_COUNT;
            count = 0;
        }
        batch[i].tokens_this_step = count;
        batch[i].request_state_index = sched_rows[i];
    }

    /* Step 2 -- sort by the number of tokens to execute this step (R1, R2). */
    qsort(batch, (size_t)n, sizeof(sched_req), by_tokens_then_row);

    /* Step 3 -- assemble the batch: index_mapping[batch_index] = request_state_index. */
    for (int32_t b = 0; b < n; ++b)
        index_mapping[b] = batch[b].request_state_index;

    /* Flattening keeps the request boundaries as a prefix sum (CSR row pointers). */
    int64_t running = 0;
    query_start_loc[0] = 0;
    for (int32_t b = 0; b < n; ++b) {
        running += batch[b].tokens_this_step;
        query_start_loc[b + 1] = running > INT32_MAX ? INT32_MAX : (int32_t)running;
    }
    if (running != T)
        st |= ORC_ST_TOKEN_SUM;

    /* seq_lens: history plus this step's tokens, per batch row (R5). */
    for (int32_t b = 0; b < n; ++b) {
        int32_t row = batch[b].request_state_index;
        if (row < 0 || row >= R) {
            st |= ORC_ST_BAD_ROW;
            seq_lens[b] = -1;
            continue;
        }
        int64_t len = (int64_t)completed[row] + batch[b].tokens_this_step;
        seq_lens[b] = (int32_t)(uint32_t)(uint64_t)len;
    }

    /* Every flat token starts unassigned (R6). */
    for (int32_t t = 0; t < T; ++t) {
        positions[t] = -1;
        if (input_ids != NULL)
            input_ids[t] = -1;
    }

    /* position and input_ids, request by request, token by token. */
    for (int32_t b = 0; b < n; ++b) {
        int32_t row = batch[b].request_state_index;
        int64_t start = query_start_loc[b];
        for (int64_t j = 0; j < batch[b].tokens_this_step; ++j) {
            int64_t flat_token_index = start + j;
            if (flat_token_index >= T)
                break;                                   /* more tokens than T (R6) */
            if (row < 0 || row >= R)
                continue;                                /* flagged above */
            int64_t position = (int64_t)completed[row] + j;   /* R3 */
            positions[flat_token_index] = (int32_t)(uint32_t)(uint64_t)position;
            if (position < 0 || (input_ids != NULL && position >= L)) {
                st |= ORC_ST_POS_OOR;
                continue;
            }
            if (input_ids != NULL)
                input_ids[flat_token_index] = token_ids[(int64_t)row * token_stride + position];
        }
    }

    free(batch);
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * The physical-address chain of [KC] "Multi-Layer Coordinate Conversion
 * Pipeline", for one KV-cache group (each group keeps a block table of its own
 * and so gets a slot mapping of its own):
 *
 *   batch_index      -> request_state_index          (index_mapping)
 *   flat_token_index -> position                     (one to one)
 *   position         -> logic_block, offset          (division and remainder)
 *   request_state_index, logic_block -> physical_block_id   (block_table)
 *   physical_block_id, offset -> slot_id             (physical_block_id * block_size + offset)
 *
 * and the visible pages per request, input_block_tables, from "Complete Input
 * Preparation for the Attention Module".
 *
 *   block_table[R * MB], row-major; input_block_tables[n * MB] (may be NULL).
 *
 * R7: a token belongs to batch row b when query_start_loc[b] <= t <
 *     query_start_loc[b+1]; tokens before query_start_loc[0] or from
 *     query_start_loc[n] on belong to no request and get slot -1, unflagged.
 * R8: "visible" pages are the first ceil(seq_len / block_size) entries of the
 *     request's table (the blocks holding history and new tokens); entries past
 *     them are not written.  Visible entries are copied verbatim; one outside
 *     [0, num_blocks) is flagged BLOCK_OOR.  A visible count above MB is flagged
 *     LB_OOR and cut to MB.  seq_len <= 0 shows no page.
 * R6 (continued): a bad row, a negative position, a logic_block >= MB or a
 *     physical block outside [0, num_blocks) is flagged and gives slot -1.
 * R21 (sliding-window groups, [CF] "allocate_slots()": blocks a sliding-window
 *     group no longer needs are freed first): with window W > 0 the token at
 *     position p attends positions p-W+1 .. p, so batch row b (count c =
 *     query_start_loc[b+1] - query_start_loc[b], seq_len s) needs positions
 *     from first = max(0, s - c - W + 1) on.  Visible pages before
 *     first / block_size lie outside every window of the step: they are
 *     copied as they are and a -1 there (a freed block, a hole) is not
 *     flagged.  W = 0 is full attention.
 */
static int64_t window_first(int32_t seq_len, int64_t count, int32_t window)
{
    if (window <= 0)
        return 0;
    int64_t first = (int64_t)seq_len - count - window + 1;
    return first > 0 ? first : 0;
}

int orc_compute_slot_mapping(int32_t n, int32_t T,
                             const int32_t* index_mapping, const int32_t* query_start_loc,
                             const int32_t* seq_lens, const int32_t* positions,
                             const int32_t* block_table, int32_t R, int32_t MB,
                             int32_t block_size, int32_t num_blocks, int32_t sliding_window,
                             int32_t* slot_mapping, int32_t* input_block_tables,
                             uint32_t* status)
{
    if (n < 0 || T < 0 || R < 0 || MB < 0 || num_blocks < 0 || block_size <= 0 ||
        sliding_window < 0)
        return ORC_EINVAL;
    if ((int64_t)num_blocks * block_size > (int64_t)INT32_MAX + 1)
        return ORC_EINVAL;                       /* slot ids must fit in int32 */
    if (query_start_loc == NULL || (n > 0 && index_mapping == NULL))
        return ORC_EINVAL;
    if (T > 0 && (positions == NULL || slot_mapping == NULL))
        return ORC_EINVAL;
    if ((n > 0 || T > 0) && R > 0 && MB > 0 && block_table == NULL)
        return ORC_EINVAL;
    if (input_block_tables != NULL && n > 0 && seq_lens == NULL)
        return ORC_EINVAL;

    uint32_t st = 0;

    for (int32_t t = 0; t < T; ++t)
        slot_mapping[t] = -1;                                   /* R7 */

    for (int32_t batch_index = 0; batch_index < n; ++batch_index) {
        int32_t request_state_index = index_mapping[batch_index];
        int64_t begin = query_start_loc[batch_index];
        int64_t end = query_start_loc[batch_index + 1];
        if (begin < 0)
            begin = 0;
        if (end > T)
            end = T;
        for (int64_t flat_token_index = begin; flat_token_index < end; ++flat_token_index) {
            if (request_state_index < 0 || request_state_index >= R) {
                st |= ORC_ST_BAD_ROW;
                continue;
            }
            int32_t position = positions[flat_token_index];
            if (position < 0) {
                st |= ORC_ST_POS_OOR;
                continue;
            }
            int32_t logic_block = position / block_size;
            int32_t offset = position % block_size;
            if (logic_block >= MB) {
                st |= ORC_ST_LB_OOR;
                continue;
            }
            int32_t physical_block_id =
                block_table[(int64_t)request_state_index * MB + logic_block];
            if (physical_block_id < 0 || physical_block_id >= num_blocks) {
                st |= ORC_ST_BLOCK_OOR;
                continue;
            }
            slot_mapping[flat_token_index] = physical_block_id * block_size + offset;
        }
    }

    if (input_block_tables != NULL) {
        for (int32_t batch_index = 0; batch_index < n; ++batch_index) {
            int32_t request_state_index = index_mapping[batch_index];
            if (request_state_index < 0 || request_state_index >= R) {
                st |= ORC_ST_BAD_ROW;
                continue;
            }
            int32_t seq_len = seq_lens[batch_index];
            int64_t visible = seq_len <= 0 ? 0 : ((int64_t)seq_len + block_size - 1) / block_size;
            if (visible > MB) {
                st |= ORC_ST_LB_OOR;
                visible = MB;
            }
            int64_t count = (int64_t)query_start_loc[batch_index + 1] - query_start_loc[batch_index];
            int64_t first_block =
                window_first(seq_len, count > 0 ? count : 0, sliding_window) / block_size;
            for (int64_t i = 0; i < visible; ++i) {
                int32_t blk = block_table[(int64_t)request_state_index * MB + i];
                int hole = i < first_block && blk == -1;                      /* R21 */
                if ((blk < 0 || blk >= num_blocks) && !hole)
                    st |= ORC_ST_BLOCK_OOR;
                input_block_tables[(int64_t)batch_index * MB + i] = blk;
            }
        }
    }

    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * Write each new token's K and V into the paged cache at its slot ([KC]
 * "Multi-Layer Coordinate Conversion Pipeline": slot_mapping is the write
 * destination of this step's new K/V; "Address Calculation Example": a slot id
 * counts cache units, one token's K and V over all heads, not bytes).
 *
 * R9 (layout): separate K and V caches, each [num_slots, row_bytes] with the
 *     H x D row of a slot contiguous, so slot * row_bytes is the byte offset.
 *     Token t's K row starts at k + t * k_stride bytes (likewise V), so K/V may be
 *     strided views.  The payload is copied as bytes, never as numbers.
 * R6 (continued): slot < 0 marks a token with nothing to write and is skipped
 *     silently; slot >= num_slots is flagged SLOT_OOR and skipped.  Tokens are
 *     written in flat order (duplicate slots break the caller's contract).
 */
int orc_scatter_kv(int32_t T, int64_t row_bytes,
                   const void* k, int64_t k_stride, const void* v, int64_t v_stride,
                   void* k_cache, void* v_cache, int64_t num_slots,
                   const int32_t* slot_mapping, uint32_t* status)
{
    if (T < 0 || row_bytes <= 0 || num_slots < 0 || k_stride < row_bytes || v_stride < row_bytes)
        return ORC_EINVAL;
    if (T > 0 && (k == NULL || v == NULL || slot_mapping == NULL ||
                  (num_slots > 0 && (k_cache == NULL || v_cache == NULL))))
        return ORC_EINVAL;

    uint32_t st = 0;
    const unsigned char* ksrc = (const unsigned char*)k;
    const unsigned char* vsrc = (const unsigned char*)v;
    unsigned char* kdst = (unsigned char*)k_cache;
    unsigned char* vdst = (unsigned char*)v_cache;

    for (int32_t flat_token_index = 0; flat_token_index < T; ++flat_token_index) {
        int64_t slot_id = slot_mapping[flat_token_index];
        if (slot_id < 0)
            continue;
        if (slot_id >= num_slots) {
            st |= ORC_ST_SLOT_OOR;
            continue;
        }
        memcpy(kdst + slot_id * row_bytes, ksrc + (int64_t)flat_token_index * k_stride,
               (size_t)row_bytes);
        memcpy(vdst + slot_id * row_bytes, vsrc + (int64_t)flat_token_index * v_stride,
               (size_t)row_bytes);
    }

    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * Paged K/V read ([KC] "Complete Input Preparation for the Attention Module":
 * seq_lens gives each request's KV range, history plus new tokens, and
 * input_block_tables its visible pages, read by indirect addressing).  For
 * every batch row b and position p < seq_lens[b] the address chain of
 * "Multi-Layer Coordinate Conversion Pipeline" is run again -- logic_block =
 * p / block_size, offset = p % block_size, physical_block_id from the visible
 * pages, slot_id = physical_block_id * block_size + offset -- and the K and V
 * rows at that slot are read.
 * R14 (output): the pages' attention reads the pages in place; here the rows
 *     are copied into one contiguous varlen array, request after request in
 *     batch order: row kv_start[b] + p, where kv_start is the running sum of
 *     the seq_lens (kv_start[0] = 0, n+1 entries, int64 sum kept in int32,
 *     saturating at INT32_MAX).  This is the layout of a non-paged varlen
 *     attention input and the exact inverse of the scatter.
 * R22 (sliding-window groups, W > 0): only the positions some new token of
 *     the step attends are read, first .. seq_len-1 with first as in R21, to
 *     rows kv_start[b] + (p - first); kv_start sums seq_len - first.
 * R15 (data errors): a negative seq_len counts as 0 (BAD_COUNT); a position
 *     whose logical block is >= MB is not read (LB_OOR); a visible page
 *     outside [0, num_blocks) is not read (BLOCK_OOR); rows at or past
 *     out_tokens are not written (TOKEN_SUM).  Rows not read keep their
 *     previous contents.  The cache holds num_blocks * block_size slots.
 */
int orc_gather_kv(int32_t n, const int32_t* seq_lens, const int32_t* query_start_loc,
                  int32_t sliding_window, const int32_t* input_block_tables,
                  int32_t MB, int32_t block_size, int32_t num_blocks, int64_t row_bytes,
                  const void* k_cache, const void* v_cache, int64_t out_tokens, void* k_out,
                  int64_t k_out_stride, void* v_out, int64_t v_out_stride, int32_t* kv_start,
                  uint32_t* status)
{
    if (n < 0 || MB < 0 || block_size <= 0 || num_blocks < 0 || row_bytes <= 0 ||
        out_tokens < 0 || k_out_stride < row_bytes || v_out_stride < row_bytes ||
        sliding_window < 0)
        return ORC_EINVAL;
    if (n > 0 && (seq_lens == NULL || (MB > 0 && input_block_tables == NULL) ||
                  (sliding_window > 0 && query_start_loc == NULL)))
        return ORC_EINVAL;
    if (out_tokens > 0 && (k_out == NULL || v_out == NULL))
        return ORC_EINVAL;
    if (num_blocks > 0 && (k_cache == NULL || v_cache == NULL))
        return ORC_EINVAL;

    uint32_t st = 0;
    const unsigned char* kc = (const unsigned char*)k_cache;
    const unsigned char* vc = (const unsigned char*)v_cache;
    unsigned char* ko = (unsigned char*)k_out;
    unsigned char* vo = (unsigned char*)v_out;
    int64_t start = 0;
    for (int32_t batch_index = 0; batch_index < n; ++batch_index) {
        if (kv_start != NULL)
            kv_start[batch_index] = start > INT32_MAX ? INT32_MAX : (int32_t)start;
        int64_t seq_len = seq_lens[batch_index];
        if (seq_len < 0) {
            st |= ORC_ST_BAD_COUNT;
            seq_len = 0;
        }
        int64_t first = 0;                                     /* R22 */
        if (sliding_window > 0) {
            int64_t count = (int64_t)query_start_loc[batch_index + 1] - query_start_loc[batch_index];
            first = window_first((int32_t)seq_len, count > 0 ? count : 0, sliding_window);
        }
        for (int64_t position = first; position < seq_len; ++position) {
            int64_t out_row = start + (position - first);
            if (out_row >= out_tokens) {
                st |= ORC_ST_TOKEN_SUM;
                break;
            }
            int64_t logic_block = position / block_size;
            int64_t offset = position % block_size;
            if (logic_block >= MB) {
                st |= ORC_ST_LB_OOR;
                continue;
            }
            int32_t physical_block_id =
                input_block_tables[(int64_t)batch_index * MB + logic_block];
            if (physical_block_id < 0 || physical_block_id >= num_blocks) {
                st |= ORC_ST_BLOCK_OOR;
                continue;
            }
            int64_t slot_id = (int64_t)physical_block_id * block_size + offset;
            memcpy(ko + out_row * k_out_stride, kc + slot_id * row_bytes, (size_t)row_bytes);
            memcpy(vo + out_row * v_out_stride, vc + slot_id * row_bytes, (size_t)row_bytes);
        }
        start += seq_len - first;
    }
    if (kv_start != NULL)
        kv_start[n] = start > INT32_MAX ? INT32_MAX : (int32_t)start;
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * Persistent request state ([KC] "Persistent Request Context Strategy" and
 * "Design Logic Behind the Dual-Index System"): per request_state_index, the
 * tokens already processed (completed), the request's token list (token_ids
 * row) and its block table row.  R10: the state also keeps row_blocks[r], the
 * number of logical blocks allocated to row r, so that new block ids can be
 * appended after the existing ones.  Which row a request gets comes from the
 * row pool at the end of this file.
 */

/*
 * add_request for m new requests: row rows[i] gets completed = num_computed[i]
 * (tokens already covered, e.g. by reused prefix blocks), its prompt tokens
 * prompt_tokens[prompt_start[i] .. prompt_start[i+1]) at positions 0.., and its
 * block table blocks[block_start[i] .. block_start[i+1]) at logical blocks 0..,
 * the rest of the row set to -1 (a recycled row keeps nothing of its previous
 * request); row_blocks = the number of blocks given.
 * R11 (data errors): a row outside [0, R) is flagged BAD_ROW and skipped; a
 * request whose token or block range is not inside its flat array
 * (start < 0, end < start, end > the array's length) is flagged BAD_RANGE and
 * skipped; prompt tokens at positions >= L are flagged POS_OOR and dropped;
 * block ids past MB are flagged LB_OOR and dropped (row_blocks is cut to MB);
 * token-table entries past the prompt are left as they are.
 */
static int bad_range(const int32_t* start, int32_t i, int32_t total)
{
    return start[i] < 0 || start[i + 1] < start[i] || start[i + 1] > total;
}

int orc_add_requests(int32_t m, const int32_t* rows, const int32_t* num_computed,
                     const int32_t* prompt_start, const int32_t* prompt_tokens,
                     int32_t num_prompt_tokens, const int32_t* block_start,
                     const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                     int32_t* completed, int32_t* token_ids, int64_t token_stride, int32_t L,
                     int32_t* block_table, int32_t MB, int32_t* row_blocks, uint32_t* status)
{
    if (m < 0 || R < 0 || L < 0 || MB < 0 || token_stride < L || num_prompt_tokens < 0 ||
        num_blocks_given < 0)
        return ORC_EINVAL;
    if (m > 0 && (rows == NULL || num_computed == NULL || prompt_start == NULL ||
                  block_start == NULL))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t i = 0; i < m; ++i) {
        int32_t r = rows[i];
        if (r < 0 || r >= R) {
            st |= ORC_ST_BAD_ROW;
            continue;
        }
        if (bad_range(prompt_start, i, num_prompt_tokens) ||
            bad_range(block_start, i, num_blocks_given)) {
            st |= ORC_ST_BAD_RANGE;
            continue;
        }
        completed[r] = num_computed[i];
        for (int64_t j = 0; j < (int64_t)prompt_start[i + 1] - prompt_start[i]; ++j) {
            if (j >= L) {
                st |= ORC_ST_POS_OOR;
                break;
            }
            token_ids[(int64_t)r * token_stride + j] = prompt_tokens[prompt_start[i] + j];
        }
        int64_t given = (int64_t)block_start[i + 1] - block_start[i];
        if (given > MB) {
            st |= ORC_ST_LB_OOR;
            given = MB;
        }
        for (int64_t j = 0; j < MB; ++j)
            block_table[(int64_t)r * MB + j] = j < given ? blocks[block_start[i] + j] : -1;
        row_blocks[r] = (int32_t)given;
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * update_request for m requests already registered: the newly allocated block
 * ids blocks[block_start[i] .. block_start[i+1]) are appended to row rows[i]'s
 * block table after its row_blocks[r] existing entries; row_blocks grows by as
 * many.  R11: a bad row is flagged and skipped, a bad block range likewise
 * (BAD_RANGE); entries that would land at or past MB (or a row_blocks outside
 * [0, MB]) are flagged LB_OOR and dropped.  Rows must be distinct in one call.
 */
int orc_append_blocks(int32_t m, const int32_t* rows, const int32_t* block_start,
                      const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                      int32_t* block_table, int32_t MB, int32_t* row_blocks, uint32_t* status)
{
    if (m < 0 || R < 0 || MB < 0 || num_blocks_given < 0)
        return ORC_EINVAL;
    if (m > 0 && (rows == NULL || block_start == NULL))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t i = 0; i < m; ++i) {
        int32_t r = rows[i];
        if (r < 0 || r >= R) {
            st |= ORC_ST_BAD_ROW;
            continue;
        }
        if (bad_range(block_start, i, num_blocks_given)) {
            st |= ORC_ST_BAD_RANGE;
            continue;
        }
        int64_t have = row_blocks[r];
        for (int64_t j = 0; j < (int64_t)block_start[i + 1] - block_start[i]; ++j) {
            if (have >= MB || have < 0) {
                st |= ORC_ST_LB_OOR;
                break;
            }
            block_table[(int64_t)r * MB + have] = blocks[block_start[i] + j];
            ++have;
        }
        row_blocks[r] = (int32_t)have;
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * After a step: each scheduled request's tokens are now computed, so
 * completed[row] becomes its seq_len (history plus this step's tokens; [CF]
 * "为什么还有 num_in_flight_tokens": the computed count advances by the tokens
 * scheduled), and a request that produced a new token (sampled[b] >= 0; NULL:
 * none did) gets it appended to its token list at position seq_len, the next
 * position to compute.  R11: a bad row is flagged and skipped; a token at a
 * position outside [0, L) is flagged POS_OOR and dropped; sampled[b] < 0 means
 * no token (a prefill chunk that is not the prompt's last).
 */
int orc_advance_state(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                      const int32_t* sampled, int32_t R, int32_t* completed, int32_t* token_ids,
                      int64_t token_stride, int32_t L, uint32_t* status)
{
    if (n < 0 || R < 0 || L < 0 || token_stride < L)
        return ORC_EINVAL;
    if (n > 0 && (index_mapping == NULL || seq_lens == NULL))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t b = 0; b < n; ++b) {
        int32_t r = index_mapping[b];
        if (r < 0 || r >= R) {
            st |= ORC_ST_BAD_ROW;
            continue;
        }
        completed[r] = seq_lens[b];
        if (sampled != NULL && sampled[b] >= 0) {
            int32_t p = seq_lens[b];
            if (p < 0 || p >= L) {
                st |= ORC_ST_POS_OOR;
                continue;
            }
            token_ids[(int64_t)r * token_stride + p] = sampled[b];
        }
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * Row pool ([KC] "Design Logic Behind the Dual-Index System": a new request is
 * handed a request_state_index and a completed request gives its index back to
 * be handed out again, so rows are pooled instead of allocated and freed).
 * State, caller-owned: free_rows[R] (a stack, valid below *num_free) and
 * in_use[R] (1 while a row is handed out).
 * R12: the stack starts with every row, arranged so that rows 0, 1, 2, ... come
 *      out first; acquire pops from the top, release pushes the rows in the
 *      order given, so the row released last is handed out next.
 * R13: asking for more rows than are free hands out none (ORC_ENOROWS);
 *      releasing a row outside [0, R), one not handed out, or one listed twice
 *      in the call releases none (ORC_EINVAL).
 */
int orc_pool_reset(int32_t R, int32_t* free_rows, int32_t* num_free, uint8_t* in_use)
{
    if (R < 0 || num_free == NULL || (R > 0 && (free_rows == NULL || in_use == NULL)))
        return ORC_EINVAL;
    for (int32_t i = 0; i < R; ++i) {
        free_rows[i] = R - 1 - i;        /* row 0 on top */
        in_use[i] = 0;
    }
    *num_free = R;
    return ORC_OK;
}

int orc_pool_acquire(int32_t R, int32_t* free_rows, int32_t* num_free, uint8_t* in_use,
                     int32_t m, int32_t* out)
{
    if (R < 0 || m < 0 || num_free == NULL || (m > 0 && out == NULL))
        return ORC_EINVAL;
    if (m > *num_free)
        return ORC_ENOROWS;
    for (int32_t i = 0; i < m; ++i) {
        int32_t r = free_rows[*num_free - 1];
        *num_free -= 1;
        in_use[r] = 1;
        out[i] = r;
    }
    return ORC_OK;
}

int orc_pool_release(int32_t R, int32_t* free_rows, int32_t* num_free, uint8_t* in_use,
                     int32_t m, const int32_t* rows)
{
    if (R < 0 || m < 0 || num_free == NULL || (m > 0 && rows == NULL))
        return ORC_EINVAL;
    for (int32_t i = 0; i < m; ++i) {
        if (rows[i] < 0 || rows[i] >= R || !in_use[rows[i]])
            return ORC_EINVAL;
        for (int32_t j = 0; j < i; ++j)
            if (rows[j] == rows[i])
                return ORC_EINVAL;
    }
    for (int32_t i = 0; i < m; ++i) {
        in_use[rows[i]] = 0;
        free_rows[*num_free] = rows[i];
        *num_free += 1;
    }
    return ORC_OK;
}

/*
 * Prefix-cache block hashes ([CF] "Prefix Cache：复用的是 KV，不是答案"): a
 * request's full token blocks are hashed together with their prefix context
 * -- the hash is an index key over token blocks, not over K/V -- and looked up
 * in the block pool's hash index; hit blocks are reused as they are.
 *
 * R16 (the hash; the pages fix only what it covers): FNV-1a, 64-bit, as
 *     published by Fowler, Noll and Vo: h = 14695981039346656037; for each
 *     byte, h ^= byte, then h *= 1099511628211 (mod 2^64).  For full block i
 *     (tokens i*bs .. i*bs+bs-1, each int32 as 4 little-endian bytes):
 *       c_i = FNV-1a(the block's 4*bs bytes)             content
 *       s_i = s_{i-1} * 1099511628211 + c_i (mod 2^64)   prefix context,
 *             s_{-1} = 0
 *       h_i = FNV-1a(the 8 little-endian bytes of s_i), 0 replaced by 1
 *     so h_i depends on block i and every block before it.  Only full blocks
 *     (floor(num_tokens / bs) of them, at most MB) are hashed.
 * Token lists are ragged views into one flat array: list b is
 * tokens[starts[b] .. starts[b] + lengths[b]) (a CSR array, or rows of the
 * persistent token table with starts[b] = row * token_stride).
 * R17 (data errors): a negative length is read as 0 (BAD_COUNT); a view
 *     outside [0, total) hashes nothing (BAD_RANGE); blocks past MB are not
 *     hashed (LB_OOR).
 */
uint64_t orc_fnv1a64(const unsigned char* bytes, size_t len)
{
    uint64_t h = 14695981039346656037ull;
    for (size_t i = 0; i < len; ++i) {
        h ^= bytes[i];
        h *= 1099511628211ull;
    }
    return h;
}

static void le64(uint64_t x, unsigned char out[8])
{
    for (int i = 0; i < 8; ++i)
        out[i] = (unsigned char)(x >> (8 * i));
}

int orc_hash_blocks(int32_t m, const int32_t* tokens, int64_t total, const int64_t* starts,
                    const int32_t* lengths, int32_t block_size, int32_t MB, uint64_t* hashes,
                    int32_t* num_full, uint32_t* status)
{
    if (m < 0 || total < 0 || block_size <= 0 || MB < 0)
        return ORC_EINVAL;
    if (m > 0 && (starts == NULL || lengths == NULL || (MB > 0 && hashes == NULL) ||
                  (total > 0 && tokens == NULL)))
        return ORC_EINVAL;
    uint32_t st = 0;
    unsigned char* buf = (unsigned char*)malloc((size_t)block_size * 4);
    if (buf == NULL)
        return ORC_EINVAL;
    for (int32_t b = 0; b < m; ++b) {
        int64_t len = lengths[b];
        if (len < 0) {
            st |= ORC_ST_BAD_COUNT;
            len = 0;
        }
        int64_t full = 0;
        if (starts[b] < 0 || starts[b] + len > total) {
            st |= ORC_ST_BAD_RANGE;
        } else {
            full = len / block_size;
            if (full > MB) {
                st |= ORC_ST_LB_OOR;
                full = MB;
            }
        }
        uint64_t s = 0;
        for (int64_t i = 0; i < full; ++i) {
            for (int32_t j = 0; j < block_size; ++j) {
                uint32_t t = (uint32_t)tokens[starts[b] + i * block_size + j];
                for (int k = 0; k < 4; ++k)
                    buf[4 * j + k] = (unsigned char)(t >> (8 * k));
            }
            uint64_t c = orc_fnv1a64(buf, (size_t)block_size * 4);
            s = s * 1099511628211ull + c;
            unsigned char sb[8];
            le64(s, sb);
            uint64_t h = orc_fnv1a64(sb, 8);
            hashes[(int64_t)b * MB + i] = h == 0 ? 1 : h;
        }
        if (num_full != NULL)
            num_full[b] = (int32_t)full;
    }
    free(buf);
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * The prefix index: hash -> physical block id.  R18: an entry holds the
 * smallest block id registered for its hash (a deterministic choice among
 * blocks with the same content and prefix); evicting (hash, block) empties the
 * entry only if it still names that block.  The index has room for `capacity`
 * distinct hashes; a hash that stays known after eviction still takes its
 * room.  Here it is a plain list searched from the front (key 0 = unused);
 * a new hash that finds no room is flagged TABLE_FULL and not added.
 */
#define ORC_NO_BLOCK INT32_MAX

static int64_t find_key(const uint64_t* keys, int64_t capacity, uint64_t key)
{
    for (int64_t i = 0; i < capacity; ++i)
        if (keys[i] == key)
            return i;
    return -1;
}

/*
 * Lookup ([CF]: B's blocks are hashed and looked up; the hits P1, P2 are
 * reused and only the rest is computed).  R19: the hit is the run of leading
 * full blocks whose hashes are in the index with a block, at most
 * floor((num_tokens - 1) / bs) blocks ([CF]: a hit never covers the last
 * token, which is computed again for its logits).  Outputs: num_computed[b] =
 * hit blocks * bs; hit_blocks[b*MB + i] = the block of hit i (entries past the
 * hit are not written).
 */
int orc_prefix_lookup(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lengths,
                      int32_t block_size, const uint64_t* keys, const int32_t* vals,
                      int64_t capacity, int32_t* hit_blocks, int32_t* num_computed,
                      uint32_t* status)
{
    if (m < 0 || MB < 0 || block_size <= 0 || capacity < 0)
        return ORC_EINVAL;
    if (m > 0 && (lengths == NULL || num_computed == NULL || (MB > 0 && hashes == NULL)))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t b = 0; b < m; ++b) {
        int64_t len = lengths[b];
        if (len < 0) {
            st |= ORC_ST_BAD_COUNT;
            len = 0;
        }
        int64_t cap = len > 0 ? (len - 1) / block_size : 0;
        if (cap > MB)
            cap = MB;
        int64_t hits = 0;
        while (hits < cap) {
            int64_t at = find_key(keys, capacity, hashes[(int64_t)b * MB + hits]);
            if (at < 0 || vals[at] == ORC_NO_BLOCK)
                break;
            if (hit_blocks != NULL)
                hit_blocks[(int64_t)b * MB + hits] = vals[at];
            ++hits;
        }
        num_computed[b] = (int32_t)(hits * block_size);
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * Registration of full blocks ([CF]: after allocation the blocks whose
 * contents are settled are written into the prefix cache).  For request b,
 * blocks i in [lo[b], hi[b]) register hashes[b*MB + i] -> block_table[rows[b]
 * * MB + i].  R20 (data errors): a bad row (BAD_ROW) or a range outside
 * [0, MB] or reversed (BAD_RANGE) registers nothing; a block id < 0 or
 * == INT32_MAX is skipped (BLOCK_OOR); a hash of 0 is ignored.
 */
int orc_prefix_insert(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lo,
                      const int32_t* hi, const int32_t* rows, const int32_t* block_table,
                      int32_t R, uint64_t* keys, int32_t* vals, int64_t capacity,
                      uint32_t* status)
{
    if (m < 0 || MB < 0 || R < 0 || capacity < 0)
        return ORC_EINVAL;
    if (m > 0 && (lo == NULL || hi == NULL || rows == NULL))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t b = 0; b < m; ++b) {
        int32_t r = rows[b];
        if (r < 0 || r >= R) {
            st |= ORC_ST_BAD_ROW;
            continue;
        }
        if (lo[b] < 0 || hi[b] < lo[b] || hi[b] > MB) {
            st |= ORC_ST_BAD_RANGE;
            continue;
        }
        for (int32_t i = lo[b]; i < hi[b]; ++i) {
            int32_t block = block_table[(int64_t)r * MB + i];
            if (block < 0 || block == ORC_NO_BLOCK) {
                st |= ORC_ST_BLOCK_OOR;
                continue;
            }
            uint64_t key = hashes[(int64_t)b * MB + i];
            if (key == 0)
                continue;                 /* never produced by the hash; marks unused entries */
            int64_t at = find_key(keys, capacity, key);
            if (at < 0) {
                at = find_key(keys, capacity, 0);        /* the first unused entry */
                if (at < 0) {
                    st |= ORC_ST_TABLE_FULL;
                    continue;
                }
                keys[at] = key;
                vals[at] = ORC_NO_BLOCK;
            }
            if (block < vals[at])
                vals[at] = block;
        }
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/* Eviction (R18): entry (hashes[i] -> blocks[i]) loses its block when the
 * block is freed for other contents; an entry naming another block stays. */
int orc_prefix_evict(int32_t count, const uint64_t* hashes, const int32_t* blocks,
                     uint64_t* keys, int32_t* vals, int64_t capacity)
{
    if (count < 0 || capacity < 0 || (count > 0 && (hashes == NULL || blocks == NULL)))
        return ORC_EINVAL;
    for (int32_t i = 0; i < count; ++i) {
        int64_t at = find_key(keys, capacity, hashes[i]);
        if (at >= 0 && vals[at] == blocks[i])
            vals[at] = ORC_NO_BLOCK;
    }
    return ORC_OK;
}

/*
 * Freeing the blocks a sliding-window group no longer needs ([CF]
 * "allocate_slots()": before new blocks are counted, the old blocks that
 * sliding-window attention no longer needs are released).  R23: before a step
 * the request's next token is at position completed[row], which attends
 * completed-W+1 .. completed; later positions attend further right.  So every
 * block wholly before completed-W+1, logical blocks i < max(0, completed-W+1) /
 * block_size, is freed: its id (if >= 0) is listed in freed[b*MB ..] in block
 * order, num_freed[b] counts them, and its entry becomes -1, a hole.  W = 0
 * frees nothing.  A bad row is flagged (BAD_ROW) and frees nothing.
 */
int orc_window_free(int32_t m, const int32_t* rows, const int32_t* completed,
                    int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                    int32_t sliding_window, int32_t* freed, int32_t* num_freed, uint32_t* status)
{
    if (m < 0 || R < 0 || MB < 0 || block_size <= 0 || sliding_window < 0)
        return ORC_EINVAL;
    if (m > 0 && (rows == NULL || num_freed == NULL || (R > 0 && completed == NULL) ||
                  (MB > 0 && (freed == NULL || (R > 0 && block_table == NULL)))))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t b = 0; b < m; ++b) {
        int32_t r = rows[b];
        int32_t count = 0;
        if (r < 0 || r >= R) {
            st |= ORC_ST_BAD_ROW;
        } else if (sliding_window > 0) {
            int64_t first = (int64_t)completed[r] - sliding_window + 1;
            int64_t blocks = first > 0 ? first / block_size : 0;
            if (blocks > MB)
                blocks = MB;
            for (int64_t i = 0; i < blocks; ++i) {
                int32_t* entry = &block_table[(int64_t)r * MB + i];
                if (*entry >= 0) {
                    freed[(int64_t)b * MB + count] = *entry;
                    ++count;
                    *entry = -1;
                }
            }
        }
        num_freed[b] = count;
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * Speculative lookahead ([CF] "Scheduler.schedule()": a request advances
 * towards num_tokens_with_spec, so speculative tokens are scheduled like any
 * others; "allocate_slots()": the slots needed count computed, prefix-hit, new
 * and speculative lookahead tokens, and only the missing blocks are new).
 * R24: after this step's seq_len tokens, the next k positions seq_len ..
 * seq_len+k-1 are where the draft tokens' K/V will go: lookahead_slots[b*k +
 * j] is the slot of position seq_lens[b] + j by the same chain as the slot
 * mapping (and the same flags and -1 for a bad row, a logical block >= MB or a
 * page outside the pool).
 */
int orc_lookahead_slots(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                        const int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                        int32_t num_blocks, int32_t k, int32_t* lookahead_slots, uint32_t* status)
{
    if (n < 0 || R < 0 || MB < 0 || block_size <= 0 || num_blocks < 0 || k < 0)
        return ORC_EINVAL;
    if ((int64_t)num_blocks * block_size > (int64_t)INT32_MAX + 1)
        return ORC_EINVAL;
    if (n > 0 && k > 0 && (index_mapping == NULL || seq_lens == NULL || lookahead_slots == NULL ||
                           (R > 0 && MB > 0 && block_table == NULL)))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t b = 0; b < n; ++b) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t slot = -1;
            int32_t row = index_mapping[b];
            int64_t position = (int64_t)seq_lens[b] + j;
            if (row < 0 || row >= R) {
                st |= ORC_ST_BAD_ROW;
            } else if (position < 0 || position > INT32_MAX) {
                st |= ORC_ST_POS_OOR;
            } else {
                int64_t logic_block = position / block_size;
                int64_t offset = position % block_size;
                if (logic_block >= MB) {
                    st |= ORC_ST_LB_OOR;
                } else {
                    int32_t physical_block_id = block_table[(int64_t)row * MB + logic_block];
                    if (physical_block_id < 0 || physical_block_id >= num_blocks)
                        st |= ORC_ST_BLOCK_OOR;
                    else
                        slot = (int32_t)((int64_t)physical_block_id * block_size + offset);
                }
            }
            lookahead_slots[(int64_t)b * k + j] = slot;
        }
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}

/*
 * How many new blocks each request still needs ([CF] "allocate_slots()": from
 * computed, new and lookahead tokens the needed slots, and from them the
 * blocks actually missing).  R25: need[b] = max(0, ceil((completed[row] +
 * num_new[b] + k) / block_size) - row_blocks[row]); row_blocks counts the
 * row's logical blocks, holes included.  A bad row gives 0 (BAD_ROW); a
 * negative num_new counts as 0 (BAD_COUNT).
 */
int orc_blocks_needed(int32_t n, const int32_t* rows, const int32_t* num_new, int32_t k,
                      int32_t block_size, const int32_t* completed, const int32_t* row_blocks,
                      int32_t R, int32_t* need, uint32_t* status)
{
    if (n < 0 || k < 0 || block_size <= 0 || R < 0)
        return ORC_EINVAL;
    if (n > 0 && (rows == NULL || num_new == NULL || need == NULL ||
                  (R > 0 && (completed == NULL || row_blocks == NULL))))
        return ORC_EINVAL;
    uint32_t st = 0;
    for (int32_t b = 0; b < n; ++b) {
        int32_t r = rows[b];
        int64_t want = 0;
        if (r < 0 || r >= R) {
            st |= ORC_ST_BAD_ROW;
        } else {
            int64_t add = num_new[b];
            if (add < 0) {
                st |= ORC_ST_BAD_COUNT;
                add = 0;
            }
            int64_t tokens = (int64_t)completed[r] + add + k;
            int64_t blocks = tokens <= 0 ? 0 : (tokens + block_size - 1) / block_size;
            want = blocks - row_blocks[r];
            if (want < 0)
                want = 0;
            if (want > INT32_MAX)
                want = INT32_MAX;
        }
        need[b] = (int32_t)want;
    }
    if (status != NULL)
        *status |= st;
    return ORC_OK;
}
