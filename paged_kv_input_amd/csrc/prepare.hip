// prepare.hip -- batch assembly and flattening in one launch.
//
// Batch order, prefix sums and seq_lens follow "Batch Construction and Sequence
// Flattening" and "Contiguous Token Sequence Processing" of "Deep Dive into
// vLLM's Scheduling Mechanism: The Complete CPU-to-GPU Mapping Pipeline"
// (kongchang.com/en); seq_lens as in its "Complete Input Preparation for the
// Attention Module".
//
// Design (gfx950): every workgroup orders the whole batch itself in LDS (a
// bitonic sort of 64-bit keys (count << 32 | biased row), at most
// PKV_MAX_BATCH keys), scans the sorted counts with a wave-level scan plus a
// cross-wave pass, and then expands its own slice of flat tokens by binary
// search over query_start_loc held in LDS.  Each lane's dependent loads are
// issued together, so the kernel's time is about three memory round trips
// (schedule, completed counts, token table) plus the launch.  Redoing the small sort per
// workgroup costs a few microseconds at most and removes the grid-wide barrier
// that would otherwise need a second launch or a device-side counter.
// Workgroup 0 alone writes the per-request outputs and the per-request flags.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepTokensPerThread = 4;
constexpr int kPrepTokensPerBlock = kPrepThreads * kPrepTokensPerThread;   // tokens per workgroup

__global__ __launch_bounds__(kPrepThreads) void k_prepare(
    int32_t n, int32_t T, const int32_t* __restrict__ sched_rows,
    const int32_t* __restrict__ num_scheduled, const int32_t* __restrict__ completed, int32_t R,
    const int32_t* __restrict__ token_ids, int64_t token_stride, int32_t L,
    int32_t* __restrict__ index_mapping, int32_t* __restrict__ query_start_loc,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ positions,
    int32_t* __restrict__ input_ids, uint32_t* __restrict__ status)
{
    __shared__ BatchLds<PKV_MAX_BATCH, kPrepThreads / kWave> lds;
    const bool leader = blockIdx.x == 0;
    uint32_t flags = 0;
    order_batch<kPrepThreads, PKV_MAX_BATCH, false>(lds, n, T, sched_rows, num_scheduled,
                                                    completed, R, leader, index_mapping,
                                                    query_start_loc, seq_lens, flags);
    if (!leader)
        flags = 0;      // per-request flags come from workgroup 0 only
    const int32_t* s_row = lds.row();
    const int32_t* s_done = lds.done();

    // Expand this workgroup's flat tokens: every lane resolves its tokens'
    // requests first, then issues all its token-table loads together.
    const int64_t t0 = (int64_t)blockIdx.x * kPrepTokensPerBlock + threadIdx.x;
    int32_t pos_out[kPrepTokensPerThread];
    int64_t src[kPrepTokensPerThread];
#pragma unroll
    for (int u = 0; u < kPrepTokensPerThread; ++u) {
        const int64_t t = t0 + (int64_t)u * kPrepThreads;
        pos_out[u] = -1;
        src[u] = -1;
        if (t >= T)
            continue;
        const int b = owner_of(lds.qsl, n, t);
        if (b < 0 || b >= n)
            continue;                               // past the last request
        const int32_t row = s_row[b];
        if (row < 0 || row >= R)
            continue;                               // flagged by workgroup 0
        const int64_t p = (int64_t)s_done[b] + (t - lds.qsl[b]);
        pos_out[u] = (int32_t)(uint32_t)(uint64_t)p;
        if (p < 0 || (input_ids != nullptr && p >= L))
            flags |= PKV_ST_POS_OOR;
        else if (input_ids != nullptr)
            src[u] = (int64_t)row * token_stride + p;
    }
    const bool have_ids = input_ids != nullptr && R > 0 && L > 0;
    int32_t id_out[kPrepTokensPerThread];
#pragma unroll
    for (int u = 0; u < kPrepTokensPerThread; ++u) {
        id_out[u] = have_ids ? token_ids[src[u] >= 0 ? src[u] : 0] : -1;
        if (src[u] < 0)
            id_out[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < kPrepTokensPerThread; ++u) {
        const int64_t t = t0 + (int64_t)u * kPrepThreads;
        if (t < T) {
            positions[t] = pos_out[u];
            if (input_ids != nullptr)
                input_ids[t] = id_out[u];
        }
    }
    report_status(status, flags);
}

}  // namespace

hipError_t launch_prepare(int32_t n, int32_t T, const int32_t* sched_rows,
                          const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                          const int32_t* token_ids, int64_t token_stride, int32_t L,
                          int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                          int32_t* positions, int32_t* input_ids, uint32_t* status,
                          hipStream_t stream)
{
    const int64_t blocks64 = ((int64_t)T + kPrepTokensPerBlock - 1) / kPrepTokensPerBlock;
    const unsigned blocks = blocks64 > 0 ? (unsigned)blocks64 : 1u;
    k_prepare<<<dim3(blocks), dim3(kPrepThreads), 0, stream>>>(
        n, T, sched_rows, num_scheduled, completed, R, token_ids, token_stride, L, index_mapping,
        query_start_loc, seq_lens, positions, input_ids, status);
    return hipGetLastError();
}

}  // namespace pkv
