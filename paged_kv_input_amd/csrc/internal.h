// internal.h -- device helpers and launcher declarations shared by the HIP
// sources of libpagedkv (gfx950, wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

constexpr int kWave = 64;

// Inclusive prefix sum across the 64 lanes of a wavefront (Hillis-Steele over
// __shfl_up; the 64-bit value moves as two 32-bit halves).
__device__ inline int64_t wave_inclusive_scan(int64_t x)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t lo = (uint32_t)(uint64_t)x;
        uint32_t hi = (uint32_t)((uint64_t)x >> 32);
        lo = __shfl_up(lo, d, kWave);
        hi = __shfl_up(hi, d, kWave);
        int64_t y = (int64_t)(((uint64_t)hi << 32) | lo);
        if (lane >= d)
            x += y;
    }
    return x;
}

// OR a lane's status flags into the caller's word: one atomic per wave that
// has any flag set (data errors only; the clean path issues none).
__device__ inline void report_status(uint32_t* status, uint32_t flags)
{
    if (status == nullptr)
        return;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1)
        flags |= __shfl_xor(flags, d, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0 && flags != 0)
        atomicOr(status, flags);
}

// Largest b in [0, n] with qsl[b] <= t, or -1 when qsl[0] > t.  qsl is
// non-decreasing, so that b is the request owning flat token t (b == n: past
// the last request).
__device__ inline int owner_of(const int32_t* qsl, int n, int64_t t)
{
    if ((int64_t)qsl[0] > t)
        return -1;
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)qsl[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Launchers (host side).  Arguments are already validated; each returns a
// hipError_t from the launch.
hipError_t launch_prepare(int32_t n, int32_t T, const int32_t* sched_rows,
                          const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                          const int32_t* token_ids, int64_t token_stride, int32_t L,
                          int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                          int32_t* positions, int32_t* input_ids, uint32_t* status,
                          hipStream_t stream);

hipError_t launch_slots(int32_t n, int32_t T, const int32_t* index_mapping,
                        const int32_t* query_start_loc, const int32_t* seq_lens,
                        const int32_t* positions, const int32_t* block_table, int32_t R,
                        int32_t MB, int32_t block_size, int32_t num_blocks,
                        int32_t* slot_mapping, int32_t* input_block_tables, uint32_t* status,
                        hipStream_t stream);

hipError_t launch_scatter(int32_t T, int64_t row_bytes, const void* k, int64_t k_stride,
                          const void* v, int64_t v_stride, void* k_cache, void* v_cache,
                          int64_t num_slots, const int32_t* slot_mapping, uint32_t* status,
                          hipStream_t stream);

}  // namespace pkv
