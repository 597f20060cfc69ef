// slots.hip -- write slots and visible pages of one KV-cache group, one launch.
//
// The chain of "Multi-Layer Coordinate Conversion Pipeline" of "Deep Dive into
// vLLM's Scheduling Mechanism: The Complete CPU-to-GPU Mapping Pipeline"
// (kongchang.com/en): batch_index -> request_state_index through index_mapping,
// flat token -> position, position -> (logical block, offset) by division and
// remainder, (row, logical block) -> physical block through the block table,
// physical block * block_size + offset -> slot id ("Address Calculation
// Example").  The visible pages per request (input_block_tables) come from its
// "Complete Input Preparation for the Attention Module"; in a sliding-window
// group the pages before every window of the step may be -1 holes, the blocks
// freed once the window moved past them ("allocate_slots()" of the
// caffein.top scheduler page).
//
// Design (gfx950): the grid has two kinds of workgroups.  Token workgroups
// stage query_start_loc and index_mapping in LDS, find each token's request by
// binary search there, and look the block up with one global load per token
// (lanes of a prefill run share a block-table word, so the load coalesces to a
// handful of lines per wave).  Page workgroups copy the visible prefix of one
// block-table row per wavefront.  Power-of-two block sizes use shift and mask.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

constexpr int kSlotThreads = 256;
constexpr int kSlotTokensPerThread = 4;
constexpr int kSlotTokensPerBlock = kSlotThreads * kSlotTokensPerThread;
constexpr int kPageRowsPerBlock = kSlotThreads / kWave;   // one batch row per wave
constexpr int kPageUnroll = 4;
constexpr int kStageLoads = PKV_MAX_BATCH / kSlotThreads + 1;   // query_start_loc has n + 1

__global__ __launch_bounds__(kSlotThreads) void k_slots(
    int32_t n, int32_t T, const int32_t* __restrict__ index_mapping,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ block_table, int32_t R,
    int32_t MB, int32_t block_size, int32_t bs_shift, int32_t num_blocks, int32_t window,
    int32_t* __restrict__ slot_mapping, int32_t* __restrict__ input_block_tables,
    uint32_t* __restrict__ status, int32_t token_blocks)
{
    __shared__ int32_t s_qsl[PKV_MAX_BATCH + 1];
    __shared__ int32_t s_row[PKV_MAX_BATCH];

    const int tid = threadIdx.x;
    uint32_t flags = 0;

    if ((int)blockIdx.x < token_blocks) {
        const int64_t t0 = (int64_t)blockIdx.x * kSlotTokensPerBlock + tid;
        int32_t pos[kSlotTokensPerThread];
        // Unconditional loads from clamped in-bounds addresses throughout: a
        // load under a divergent branch is issued only after a full wait.
#pragma unroll
        for (int u = 0; u < kSlotTokensPerThread; ++u) {
            const int64_t t = t0 + u * kSlotThreads;
            pos[u] = positions[t < T ? t : T - 1];
        }
        // The whole batch's boundaries and rows, every load of a thread in
        // flight together (a load-then-store loop waits once per iteration).
        int32_t q[kStageLoads];
        int32_t r[kStageLoads];
        // Rounds past the batch are skipped as a whole (a uniform test).
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int i = u * kSlotThreads + tid;
            if (u * kSlotThreads <= n) {
                q[u] = query_start_loc[i <= n ? i : 0];
                r[u] = n > 0 ? index_mapping[i < n ? i : 0] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int i = u * kSlotThreads + tid;
            if (u * kSlotThreads <= n) {
                if (i <= n)
                    s_qsl[i] = q[u];
                if (i < n)
                    s_row[i] = r[u];
            }
        }
        __syncthreads();

        int64_t src[kSlotTokensPerThread];
        int32_t off[kSlotTokensPerThread];
#pragma unroll
        for (int u = 0; u < kSlotTokensPerThread; ++u) {
            const int64_t t = t0 + u * kSlotThreads;
            src[u] = -1;
            off[u] = 0;
            if (t >= T)
                continue;
            const int b = owner_of(s_qsl, n, t);
            if (b < 0 || b >= n)
                continue;                                   // no request: slot -1
            const int32_t row = s_row[b];
            const int32_t p = pos[u];
            if (row < 0 || row >= R) {
                flags |= PKV_ST_BAD_ROW;
            } else if (p < 0) {
                flags |= PKV_ST_POS_OOR;
            } else {
                const int32_t lb = bs_shift >= 0 ? (p >> bs_shift) : p / block_size;
                off[u] = p - lb * block_size;
                if (lb >= MB)
                    flags |= PKV_ST_LB_OOR;
                else
                    src[u] = (int64_t)row * MB + lb;
            }
        }
        const bool have_bt = R > 0 && MB > 0;                // uniform
        int32_t blk[kSlotTokensPerThread];
#pragma unroll
        for (int u = 0; u < kSlotTokensPerThread; ++u) {
            blk[u] = have_bt ? block_table[src[u] >= 0 ? src[u] : 0] : -1;
            if (src[u] < 0)
                blk[u] = -1;
        }
#pragma unroll
        for (int u = 0; u < kSlotTokensPerThread; ++u) {
            const int64_t t = t0 + u * kSlotThreads;
            if (t >= T)
                continue;
            int32_t slot = -1;
            if (src[u] >= 0) {
                if (blk[u] < 0 || blk[u] >= num_blocks)
                    flags |= PKV_ST_BLOCK_OOR;
                else
                    slot = blk[u] * block_size + off[u];
            }
            slot_mapping[t] = slot;
        }
    } else {
        // Visible pages: one wavefront per batch row.
        const int b = ((int)blockIdx.x - token_blocks) * kPageRowsPerBlock + tid / kWave;
        const int lane = tid & (kWave - 1);
        if (b < n) {
            int32_t row = index_mapping[b];
            int32_t sl = seq_lens[b];
            // Both loads issued before the branch that needs sl (otherwise it
            // is sunk there, a second round trip after the row's).
            __asm__ volatile("" : "+v"(row), "+v"(sl));
            if (row < 0 || row >= R) {
                flags |= PKV_ST_BAD_ROW;
            } else {
                int64_t visible = sl <= 0 ? 0 : ((int64_t)sl + block_size - 1) / block_size;
                if (visible > MB) {
                    flags |= PKV_ST_LB_OOR;
                    visible = MB;
                }
                // Pages before the window may be -1 holes (freed blocks).
                int64_t first_block = 0;
                if (window > 0) {                                   // uniform
                    const int64_t count = (int64_t)query_start_loc[b + 1] - query_start_loc[b];
                    first_block = window_first(sl, count, window) / block_size;
                }
                const int32_t* src = block_table + (int64_t)row * MB;
                int32_t* dst = input_block_tables + (int64_t)b * MB;
                for (int64_t i0 = 0; i0 < visible; i0 += kWave * kPageUnroll) {
                    int32_t v[kPageUnroll];
#pragma unroll
                    for (int u = 0; u < kPageUnroll; ++u) {
                        const int64_t i = i0 + u * kWave + lane;
                        v[u] = src[i < visible ? i : visible - 1];   // clamped, unconditional
                    }
#pragma unroll
                    for (int u = 0; u < kPageUnroll; ++u) {
                        const int64_t i = i0 + u * kWave + lane;
                        if (i < visible) {
                            const bool hole = i < first_block && v[u] == -1;
                            if ((v[u] < 0 || v[u] >= num_blocks) && !hole)
                                flags |= PKV_ST_BLOCK_OOR;
                            dst[i] = v[u];
                        }
                    }
                }
            }
        }
    }
    report_status(status, flags);
}

}  // namespace

hipError_t launch_slots(int32_t n, int32_t T, const int32_t* index_mapping,
                        const int32_t* query_start_loc, const int32_t* seq_lens,
                        const int32_t* positions, const int32_t* block_table, int32_t R,
                        int32_t MB, int32_t block_size, int32_t num_blocks,
                        int32_t sliding_window, int32_t* slot_mapping,
                        int32_t* input_block_tables, uint32_t* status, hipStream_t stream)
{
    const int64_t token_blocks = ((int64_t)T + kSlotTokensPerBlock - 1) / kSlotTokensPerBlock;
    const int64_t page_blocks =
        input_block_tables != nullptr
            ? ((int64_t)n + kPageRowsPerBlock - 1) / kPageRowsPerBlock
            : 0;
    const int64_t blocks = token_blocks + page_blocks;
    if (blocks == 0)
        return hipSuccess;
    int32_t bs_shift = -1;
    if ((block_size & (block_size - 1)) == 0)
        bs_shift = __builtin_ctz((unsigned)block_size);
    k_slots<<<dim3((unsigned)blocks), dim3(kSlotThreads), 0, stream>>>(
        n, T, index_mapping, query_start_loc, seq_lens, positions, block_table, R, MB, block_size,
        bs_shift, num_blocks, sliding_window, slot_mapping, input_block_tables, status,
        (int32_t)token_blocks);
    return hipGetLastError();
}

}  // namespace pkv
