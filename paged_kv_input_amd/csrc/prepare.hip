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
// search over query_start_loc held in LDS.  Redoing the small sort per
// workgroup costs a few microseconds at most and removes the grid-wide barrier
// that would otherwise need a second launch or a device-side counter.
// Workgroup 0 alone writes the per-request outputs and the per-request flags.
#include "internal.h"

namespace pkv {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepTokensPerBlock = 4096;   // flat tokens expanded per workgroup
constexpr int kPrepWaves = kPrepThreads / kWave;
constexpr int kPrepPerThread = PKV_MAX_BATCH / kPrepThreads;   // batch rows per thread

static_assert(PKV_MAX_BATCH % kPrepThreads == 0, "batch rows split evenly over threads");

// Ascending order of (count, row) as unsigned 64-bit keys: the count (>= 0) in
// the high word, the row with its sign bit flipped in the low word so that
// signed row order equals unsigned key order.
__device__ inline uint64_t sort_key(int32_t count, int32_t row)
{
    return ((uint64_t)(uint32_t)count << 32) | (uint32_t)(row ^ INT32_MIN);
}
__device__ inline int32_t key_count(uint64_t key) { return (int32_t)(key >> 32); }
__device__ inline int32_t key_row(uint64_t key) { return (int32_t)((uint32_t)key ^ 0x80000000u); }

__global__ __launch_bounds__(kPrepThreads) void k_prepare(
    int32_t n, int32_t T, const int32_t* __restrict__ sched_rows,
    const int32_t* __restrict__ num_scheduled, const int32_t* __restrict__ completed, int32_t R,
    const int32_t* __restrict__ token_ids, int64_t token_stride, int32_t L,
    int32_t* __restrict__ index_mapping, int32_t* __restrict__ query_start_loc,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ positions,
    int32_t* __restrict__ input_ids, uint32_t* __restrict__ status)
{
    // s_key holds the keys while sorting, then (reinterpreted) the batch rows
    // and their completed counts for the expansion.
    __shared__ uint64_t s_key[PKV_MAX_BATCH];
    __shared__ int32_t s_qsl[PKV_MAX_BATCH + 1];
    __shared__ int64_t s_wave_total[kPrepWaves];
    int32_t* s_row = reinterpret_cast<int32_t*>(s_key);
    int32_t* s_done = s_row + PKV_MAX_BATCH;

    const int tid = threadIdx.x;
    const bool leader = blockIdx.x == 0;
    uint32_t flags = 0;

    int n_pad = 1;
    while (n_pad < n)
        n_pad <<= 1;

    // Gather the scheduled requests as sort keys.
    for (int i = tid; i < n_pad; i += kPrepThreads) {
        uint64_t key = ~0ull;                       // padding sorts last
        if (i < n) {
            int32_t c = num_scheduled[i];
            if (c < 0) {
                flags |= PKV_ST_BAD_COUNT;
                c = 0;
            }
            key = sort_key(c, sched_rows[i]);
        }
        s_key[i] = key;
    }
    __syncthreads();

    // Bitonic sort, ascending.  Pair i of a stage with distance j compares
    // element lo (bit log2(j) cleared) with lo + j; the sub-sequence direction
    // comes from bit log2(k) of lo.
    for (int k = 2; k <= n_pad; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < (n_pad >> 1); i += kPrepThreads) {
                const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
                const int hi = lo + j;
                const bool ascending = (lo & k) == 0;
                const uint64_t a = s_key[lo];
                const uint64_t b = s_key[hi];
                if ((a > b) == ascending) {
                    s_key[lo] = b;
                    s_key[hi] = a;
                }
            }
            __syncthreads();
        }
    }

    // Each thread owns kPrepPerThread consecutive batch rows.
    uint64_t keys[kPrepPerThread];
    int64_t local = 0;
    const int first = tid * kPrepPerThread;
#pragma unroll
    for (int e = 0; e < kPrepPerThread; ++e) {
        const int b = first + e;
        keys[e] = b < n ? s_key[b] : 0ull;
        local += b < n ? key_count(keys[e]) : 0;
    }

    // Block-wide exclusive scan of the per-thread sums.
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t incl = wave_inclusive_scan(local);
    if (lane == kWave - 1)
        s_wave_total[wave] = incl;
    __syncthreads();      // also: every key is now in registers, s_key may be reused
    if (wave == 0) {
        int64_t w = lane < kPrepWaves ? s_wave_total[lane] : 0;
        w = wave_inclusive_scan(w);
        if (lane < kPrepWaves)
            s_wave_total[lane] = w;
    }
    __syncthreads();
    int64_t run = (wave > 0 ? s_wave_total[wave - 1] : 0) + incl - local;
    const int64_t total = s_wave_total[kPrepWaves - 1];

#pragma unroll
    for (int e = 0; e < kPrepPerThread; ++e) {
        const int b = first + e;
        if (b >= n)
            break;
        const int32_t c = key_count(keys[e]);
        const int32_t row = key_row(keys[e]);
        run += c;
        const int32_t end = run > INT32_MAX ? INT32_MAX : (int32_t)run;
        s_qsl[b + 1] = end;
        const bool row_ok = row >= 0 && row < R;
        const int32_t done = row_ok ? completed[row] : 0;
        s_row[b] = row;
        s_done[b] = done;
        if (leader) {
            index_mapping[b] = row;
            query_start_loc[b + 1] = end;
            if (row_ok) {
                seq_lens[b] = (int32_t)(uint32_t)(uint64_t)((int64_t)done + c);
            } else {
                seq_lens[b] = -1;
                flags |= PKV_ST_BAD_ROW;
            }
        }
    }
    if (tid == 0) {
        s_qsl[0] = 0;
        if (leader) {
            query_start_loc[0] = 0;
            if (total != (int64_t)T)
                flags |= PKV_ST_TOKEN_SUM;
        }
    }
    if (!leader)
        flags = 0;      // per-request flags come from workgroup 0 only
    __syncthreads();

    // Expand this workgroup's flat tokens.
    const int64_t t_begin = (int64_t)blockIdx.x * kPrepTokensPerBlock;
    const int64_t t_end = t_begin + kPrepTokensPerBlock < T ? t_begin + kPrepTokensPerBlock : T;
    for (int64_t t = t_begin + tid; t < t_end; t += kPrepThreads) {
        int32_t pos_out = -1;
        int32_t id_out = -1;
        const int b = owner_of(s_qsl, n, t);
        if (b >= 0 && b < n) {
            const int32_t row = s_row[b];
            if (row >= 0 && row < R) {
                const int64_t p = (int64_t)s_done[b] + (t - s_qsl[b]);
                pos_out = (int32_t)(uint32_t)(uint64_t)p;
                if (p >= 0 && p < L) {
                    if (input_ids != nullptr)
                        id_out = token_ids[(int64_t)row * token_stride + p];
                } else {
                    flags |= PKV_ST_POS_OOR;
                }
            }
        }
        positions[t] = pos_out;
        if (input_ids != nullptr)
            input_ids[t] = id_out;
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
