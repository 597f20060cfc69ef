// state.hip -- updates of the persistent request state on the device.
//
// The worker keeps, per request_state_index, the tokens already processed,
// the request's token list and its block table ("Persistent Request Context
// Strategy" of "Deep Dive into vLLM's Scheduling Mechanism: The Complete
// CPU-to-GPU Mapping Pipeline", kongchang.com/en), plus here the number of
// logical blocks allocated to the row.  add_request initializes a row for a
// new request and update_request appends newly allocated block ids to a
// registered one ("Design Logic Behind the Dual-Index System"); after a step,
// each scheduled request's computed count advances to its seq_len and a
// sampled token is appended at the next position.
//
// Design (gfx950): all three are scatters of small records, bound by memory
// latency, not bandwidth.  add_requests gives each new request a workgroup
// whose lanes copy the prompt and the block-table row with unrolled,
// branch-free loads; append_blocks gives each request one wavefront, whose
// lanes read the row's block count together before any of them writes (no
// other workgroup touches the row, so the count cannot race); advance_state
// takes one lane per batch row.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

// Registering a request: one workgroup per request.  Long prompts take 256
// threads moving 16 KiB per round trip; prompts of at most 2048 tokens on
// average take 128 threads moving 4 KiB, so that more requests are resident
// at once (measured on MI355X, 4096 prompts of 128-2048 tokens: 12.2 -> 9.5
// us; 512 prompts of up to 16.9k tokens stay at 256 threads: 10.3 us against
// 14.7 us with 128).
constexpr int kAddShortTokens = 2048;
constexpr int kAppendThreads = 256;
constexpr int kAppendRows = kAppendThreads / kWave;
constexpr int kAdvanceThreads = 256;

__device__ inline bool bad_range(const int32_t* start, int i, int32_t total, int32_t& lo,
                                 int32_t& hi)
{
    lo = start[i];
    hi = start[i + 1];
    return lo < 0 || hi < lo || hi > total;
}

template <int kAddThreads, int kAddUnroll>
__global__ __launch_bounds__(kAddThreads) void k_add_requests(
    const int32_t* __restrict__ rows, const int32_t* __restrict__ num_computed,
    const int32_t* __restrict__ prompt_start, const int32_t* __restrict__ prompt_tokens,
    int32_t num_prompt_tokens, const int32_t* __restrict__ block_start,
    const int32_t* __restrict__ blocks, int32_t num_blocks_given, int32_t R,
    int32_t* __restrict__ completed, int32_t* __restrict__ token_ids, int64_t token_stride,
    int32_t L, int32_t* __restrict__ block_table, int32_t MB, int32_t* __restrict__ row_blocks,
    uint32_t* __restrict__ status)
{
    const int i = blockIdx.x;
    const int tid = threadIdx.x;
    uint32_t flags = 0;
    const int32_t r = rows[i];
    int32_t p_lo, p_hi, b_lo, b_hi;
    const bool bad_p = bad_range(prompt_start, i, num_prompt_tokens, p_lo, p_hi);
    const bool bad_b = bad_range(block_start, i, num_blocks_given, b_lo, b_hi);
    if (r < 0 || r >= R) {
        flags |= tid == 0 ? PKV_ST_BAD_ROW : 0u;
    } else if (bad_p || bad_b) {
        flags |= tid == 0 ? PKV_ST_BAD_RANGE : 0u;
    } else {
        const int32_t plen = p_hi - p_lo;
        const int32_t ncopy = plen < L ? plen : L;
        if (plen > L && tid == 0)
            flags |= PKV_ST_POS_OOR;
        int32_t* trow = token_ids + (int64_t)r * token_stride;
        for (int32_t j0 = 0; j0 < ncopy; j0 += kAddThreads * kAddUnroll) {
            int32_t v[kAddUnroll];
#pragma unroll
            for (int u = 0; u < kAddUnroll; ++u) {
                const int32_t j = j0 + u * kAddThreads + tid;
                v[u] = prompt_tokens[p_lo + (j < ncopy ? j : ncopy - 1)];   // clamped
            }
#pragma unroll
            for (int u = 0; u < kAddUnroll; ++u) {
                const int32_t j = j0 + u * kAddThreads + tid;
                if (j < ncopy)
                    trow[j] = v[u];
            }
        }
        int32_t given = b_hi - b_lo;
        if (given > MB) {
            flags |= tid == 0 ? PKV_ST_LB_OOR : 0u;
            given = MB;
        }
        int32_t* brow = block_table + (int64_t)r * MB;
        for (int32_t j0 = 0; j0 < MB; j0 += kAddThreads * kAddUnroll) {
            int32_t v[kAddUnroll];
#pragma unroll
            for (int u = 0; u < kAddUnroll; ++u) {
                const int32_t j = j0 + u * kAddThreads + tid;
                v[u] = given > 0 ? blocks[b_lo + (j < given ? j : given - 1)] : -1;
                if (j >= given)
                    v[u] = -1;
            }
#pragma unroll
            for (int u = 0; u < kAddUnroll; ++u) {
                const int32_t j = j0 + u * kAddThreads + tid;
                if (j < MB)
                    brow[j] = v[u];
            }
        }
        if (tid == 0) {
            completed[r] = num_computed[i];
            row_blocks[r] = given;
        }
    }
    report_status(status, flags);
}

__global__ __launch_bounds__(kAppendThreads) void k_append_blocks(
    int32_t m, const int32_t* __restrict__ rows, const int32_t* __restrict__ block_start,
    const int32_t* __restrict__ blocks, int32_t num_blocks_given, int32_t R,
    int32_t* __restrict__ block_table, int32_t MB, int32_t* __restrict__ row_blocks,
    uint32_t* __restrict__ status)
{
    const int i = blockIdx.x * kAppendRows + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t flags = 0;
    if (i < m) {
        const int32_t r = rows[i];
        int32_t lo, hi;
        if (r < 0 || r >= R) {
            flags |= lane == 0 ? PKV_ST_BAD_ROW : 0u;
        } else if (bad_range(block_start, i, num_blocks_given, lo, hi)) {
            flags |= lane == 0 ? PKV_ST_BAD_RANGE : 0u;
        } else {
            // Every lane holds the old count before lane 0 stores the new one.
            const int32_t have = row_blocks[r];
            const int32_t k = hi - lo;
            const bool room = have >= 0 && have <= MB;
            const int32_t fits = room ? (k < MB - have ? k : MB - have) : 0;
            if (k > fits)
                flags |= lane == 0 ? PKV_ST_LB_OOR : 0u;
            int32_t* brow = block_table + (int64_t)r * MB;
            for (int32_t j = lane; j < fits; j += kWave)
                brow[have + j] = blocks[lo + j];
            if (lane == 0 && room)
                row_blocks[r] = have + fits;
        }
    }
    report_status(status, flags);
}

__global__ __launch_bounds__(kAdvanceThreads) void k_advance_state(
    int32_t n, const int32_t* __restrict__ index_mapping, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sampled, int32_t R, int32_t* __restrict__ completed,
    int32_t* __restrict__ token_ids, int64_t token_stride, int32_t L,
    uint32_t* __restrict__ status)
{
    const int b = blockIdx.x * kAdvanceThreads + threadIdx.x;
    uint32_t flags = 0;
    if (b < n) {
        const int32_t r = index_mapping[b];
        const int32_t sl = seq_lens[b];
        const int32_t tok = sampled != nullptr ? sampled[b] : -1;
        if (r < 0 || r >= R) {
            flags |= PKV_ST_BAD_ROW;
        } else {
            completed[r] = sl;
            if (tok >= 0) {
                if (sl < 0 || sl >= L)
                    flags |= PKV_ST_POS_OOR;
                else
                    token_ids[(int64_t)r * token_stride + sl] = tok;
            }
        }
    }
    report_status(status, flags);
}

}  // namespace

hipError_t launch_add_requests(int32_t m, const int32_t* rows, const int32_t* num_computed,
                               const int32_t* prompt_start, const int32_t* prompt_tokens,
                               int32_t num_prompt_tokens, const int32_t* block_start,
                               const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                               int32_t* completed, int32_t* token_ids, int64_t token_stride,
                               int32_t L, int32_t* block_table, int32_t MB, int32_t* row_blocks,
                               uint32_t* status, hipStream_t stream)
{
    if (m == 0)
        return hipSuccess;
    const bool short_prompts = (int64_t)num_prompt_tokens <= (int64_t)kAddShortTokens * m;
#define PKV_ADD_LAUNCH(W, U)                                                                       \
    k_add_requests<W, U><<<dim3((unsigned)m), dim3(W), 0, stream>>>(                              \
        rows, num_computed, prompt_start, prompt_tokens, num_prompt_tokens, block_start, blocks,   \
        num_blocks_given, R, completed, token_ids, token_stride, L, block_table, MB, row_blocks,   \
        status)
    if (short_prompts)
        PKV_ADD_LAUNCH(128, 8);
    else
        PKV_ADD_LAUNCH(256, 16);
#undef PKV_ADD_LAUNCH
    return hipGetLastError();
}

hipError_t launch_append_blocks(int32_t m, const int32_t* rows, const int32_t* block_start,
                                const int32_t* blocks, int32_t num_blocks_given, int32_t R,
                                int32_t* block_table, int32_t MB, int32_t* row_blocks,
                                uint32_t* status, hipStream_t stream)
{
    if (m == 0)
        return hipSuccess;
    const unsigned grid = (unsigned)(((int64_t)m + kAppendRows - 1) / kAppendRows);
    k_append_blocks<<<dim3(grid), dim3(kAppendThreads), 0, stream>>>(
        m, rows, block_start, blocks, num_blocks_given, R, block_table, MB, row_blocks, status);
    return hipGetLastError();
}

hipError_t launch_advance_state(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                                const int32_t* sampled, int32_t R, int32_t* completed,
                                int32_t* token_ids, int64_t token_stride, int32_t L,
                                uint32_t* status, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const unsigned grid = (unsigned)(((int64_t)n + kAdvanceThreads - 1) / kAdvanceThreads);
    k_advance_state<<<dim3(grid), dim3(kAdvanceThreads), 0, stream>>>(
        n, index_mapping, seq_lens, sampled, R, completed, token_ids, token_stride, L, status);
    return hipGetLastError();
}

}  // namespace pkv
