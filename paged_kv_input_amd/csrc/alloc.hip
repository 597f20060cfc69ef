// alloc.hip -- allocation-side variants of the path: freeing the blocks a
// sliding-window group no longer needs, the slots of speculative lookahead
// positions, and the new blocks each request still needs.
//
// "从源码读 vLLM Scheduler：一轮调度如何分配请求与 KV Cache" (caffein.top):
// a request advances towards num_tokens_with_spec, so speculative draft tokens
// are scheduled like any others ("Scheduler.schedule()"); allocate_slots()
// counts the slots for computed, prefix-hit, new and speculative lookahead
// tokens, first frees the old blocks sliding-window attention no longer needs,
// and allocates only the blocks actually missing.
//
// Design (gfx950): small integer kernels bound by launch and memory latency.
// The free gives each request a wavefront, which compacts the freed ids with a
// ballot and a popcount prefix (no atomics, block order kept); the other two
// take one lane per output.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;
constexpr int kFreeRounds = 4;

__global__ __launch_bounds__(kThreads) void k_window_free(
    int32_t m, const int32_t* __restrict__ rows, const int32_t* __restrict__ completed,
    int32_t* __restrict__ block_table, int32_t R, int32_t MB, int32_t block_size, int32_t window,
    int32_t* __restrict__ freed, int32_t* __restrict__ num_freed, uint32_t* __restrict__ status)
{
    const int b = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t flags = 0;
    if (b < m) {
        const int32_t r = rows[b];
        int32_t count = 0;
        if (r < 0 || r >= R) {
            flags |= lane == 0 ? PKV_ST_BAD_ROW : 0u;
        } else if (window > 0) {
            // Blocks wholly before the first position the next token attends.
            const int64_t first = (int64_t)completed[r] - window + 1;
            int64_t blocks = first > 0 ? first / block_size : 0;
            if (blocks > MB)
                blocks = MB;
            int32_t* row = block_table + (int64_t)r * MB;
            int32_t* out = freed + (int64_t)b * MB;
            const uint64_t below = (1ull << lane) - 1;
            // Four rounds of 64 entries loaded per wait (unconditional loads
            // from clamped in-bounds addresses), then compacted in order.
            for (int64_t i0 = 0; i0 < blocks; i0 += kFreeRounds * kWave) {
                int32_t entry[kFreeRounds];
#pragma unroll
                for (int u = 0; u < kFreeRounds; ++u) {
                    const int64_t i = i0 + u * kWave + lane;
                    entry[u] = row[i < blocks ? i : 0];
                }
#pragma unroll
                for (int u = 0; u < kFreeRounds; ++u) {
                    const int64_t i = i0 + u * kWave + lane;
                    const bool take = i < blocks && entry[u] >= 0;
                    const uint64_t mask = __ballot(take);
                    if (take) {
                        out[count + __popcll(mask & below)] = entry[u];
                        row[i] = -1;
                    }
                    count += __popcll(mask);
                }
            }
        }
        if (lane == 0)
            num_freed[b] = count;
    }
    report_status(status, flags);
}

__global__ __launch_bounds__(kThreads) void k_lookahead_slots(
    int32_t n, const int32_t* __restrict__ index_mapping, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ block_table, int32_t R, int32_t MB, int32_t block_size,
    int32_t num_blocks, int32_t k, int32_t* __restrict__ out, uint32_t* __restrict__ status)
{
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t flags = 0;
    if (idx < (int64_t)n * k) {
        const int64_t b = idx / k;
        const int64_t j = idx - b * k;
        const int32_t row = index_mapping[b];
        const int64_t position = (int64_t)seq_lens[b] + j;
        int32_t slot = -1;
        if (row < 0 || row >= R) {
            flags |= PKV_ST_BAD_ROW;
        } else if (position < 0 || position > INT32_MAX) {
            flags |= PKV_ST_POS_OOR;
        } else {
            const int64_t lb = position / block_size;
            if (lb >= MB) {
                flags |= PKV_ST_LB_OOR;
            } else {
                const int32_t blk = block_table[(int64_t)row * MB + lb];
                if (blk < 0 || blk >= num_blocks)
                    flags |= PKV_ST_BLOCK_OOR;
                else
                    slot = (int32_t)((int64_t)blk * block_size + (position - lb * block_size));
            }
        }
        out[idx] = slot;
    }
    report_status(status, flags);
}

__global__ __launch_bounds__(kThreads) void k_blocks_needed(
    int32_t n, const int32_t* __restrict__ rows, const int32_t* __restrict__ num_new, int32_t k,
    int32_t block_size, const int32_t* __restrict__ completed,
    const int32_t* __restrict__ row_blocks, int32_t R, int32_t* __restrict__ need,
    uint32_t* __restrict__ status)
{
    const int b = blockIdx.x * kThreads + threadIdx.x;
    uint32_t flags = 0;
    if (b < n) {
        const int32_t r = rows[b];
        int64_t want = 0;
        if (r < 0 || r >= R) {
            flags |= PKV_ST_BAD_ROW;
        } else {
            int64_t add = num_new[b];
            if (add < 0) {
                flags |= PKV_ST_BAD_COUNT;
                add = 0;
            }
            const int64_t tokens = (int64_t)completed[r] + add + k;
            const int64_t blocks = tokens <= 0 ? 0 : (tokens + block_size - 1) / block_size;
            want = blocks - row_blocks[r];
            want = want < 0 ? 0 : (want > INT32_MAX ? INT32_MAX : want);
        }
        need[b] = (int32_t)want;
    }
    report_status(status, flags);
}

}  // namespace

hipError_t launch_window_free(int32_t m, const int32_t* rows, const int32_t* completed,
                              int32_t* block_table, int32_t R, int32_t MB, int32_t block_size,
                              int32_t sliding_window, int32_t* freed, int32_t* num_freed,
                              uint32_t* status, hipStream_t stream)
{
    if (m == 0)
        return hipSuccess;
    const unsigned grid = (unsigned)(((int64_t)m + kRowsPerBlock - 1) / kRowsPerBlock);
    k_window_free<<<dim3(grid), dim3(kThreads), 0, stream>>>(
        m, rows, completed, block_table, R, MB, block_size, sliding_window, freed, num_freed,
        status);
    return hipGetLastError();
}

hipError_t launch_lookahead_slots(int32_t n, const int32_t* index_mapping, const int32_t* seq_lens,
                                  const int32_t* block_table, int32_t R, int32_t MB,
                                  int32_t block_size, int32_t num_blocks, int32_t k,
                                  int32_t* lookahead_slots, uint32_t* status, hipStream_t stream)
{
    const int64_t total = (int64_t)n * k;
    if (total == 0)
        return hipSuccess;
    const int64_t grid = (total + kThreads - 1) / kThreads;
    if (grid > INT32_MAX)
        return hipErrorInvalidConfiguration;
    k_lookahead_slots<<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        n, index_mapping, seq_lens, block_table, R, MB, block_size, num_blocks, k,
        lookahead_slots, status);
    return hipGetLastError();
}

hipError_t launch_blocks_needed(int32_t n, const int32_t* rows, const int32_t* num_new, int32_t k,
                                int32_t block_size, const int32_t* completed,
                                const int32_t* row_blocks, int32_t R, int32_t* need,
                                uint32_t* status, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const unsigned grid = (unsigned)(((int64_t)n + kThreads - 1) / kThreads);
    k_blocks_needed<<<dim3(grid), dim3(kThreads), 0, stream>>>(n, rows, num_new, k, block_size,
                                                             completed, row_blocks, R, need,
                                                             status);
    return hipGetLastError();
}

}  // namespace pkv
