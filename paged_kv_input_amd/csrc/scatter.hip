// scatter.hip -- write each new token's K and V rows into a paged cache.
//
// slot_mapping is the write destination of this step's new K/V ("Multi-Layer
// Coordinate Conversion Pipeline" of "Deep Dive into vLLM's Scheduling
// Mechanism: The Complete CPU-to-GPU Mapping Pipeline", kongchang.com/en); a
// slot is one token's K and V over all heads ("Address Calculation Example"),
// here two caches of [num_slots][row_bytes].
//
// Design (gfx950): a pure HBM stream, no arithmetic.  Each workgroup moves one
// payload: the first half of the grid K, the second half V, each walking the
// T x (row_bytes / 16) 16-byte chunks in flat order, so each wavefront reads
// 1 KiB of consecutive bytes and writes whole cache rows.  Every lane issues
// kScatterUnroll loads before its first store, keeping enough bytes in flight
// per CU for HBM3E; the slot load of a token is shared by its lanes.  One
// payload per workgroup streams from one source span to one cache row at a
// time (measured on MI355X against a workgroup moving the same tokens' K and
// V together: the 32k-token prefill 51.9 -> 50.8 us, 512 requests in two
// groups 110.7 -> 108.4 us, the mixed batch 13.5 -> 13.1 us).  Loads and
// stores are non-temporal: the payload is touched once and the cache rows are
// not read back by this step.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#ifndef PKV_SCATTER_THREADS
#define PKV_SCATTER_THREADS 256
#endif
#ifndef PKV_SCATTER_UNROLL
#define PKV_SCATTER_UNROLL 8              // 16-byte chunks of one payload per lane
#endif
#ifndef PKV_SCATTER_NT_LOAD
#define PKV_SCATTER_NT_LOAD 1
#endif
#ifndef PKV_SCATTER_NT_STORE
#define PKV_SCATTER_NT_STORE 1
#endif

constexpr int kScatterThreads = PKV_SCATTER_THREADS;
constexpr int kScatterUnroll = PKV_SCATTER_UNROLL;
constexpr int kChunksPerBlock = kScatterThreads * kScatterUnroll;

__device__ inline u32x4 load16(const u32x4* p)
{
#if PKV_SCATTER_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

__device__ inline void store16(u32x4 x, u32x4* p)
{
#if PKV_SCATTER_NT_STORE
    __builtin_nontemporal_store(x, p);
#else
    *p = x;
#endif
}

template <bool kPow2Row, bool kFull>
__device__ inline void scatter_chunks(int64_t base, int64_t total_chunks, int32_t chunks_per_row,
                                      int32_t row_shift, const u32x4* __restrict__ src,
                                      int64_t stride16, u32x4* __restrict__ cache,
                                      int64_t num_slots, const int32_t* __restrict__ slot_mapping,
                                      uint32_t& flags)
{
    int32_t slot[kScatterUnroll];
    int64_t chunk[kScatterUnroll];
    u32x4 x[kScatterUnroll];

    // Issue every load (slot words and payload) before the first use of any.
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
        int64_t idx = base + (int64_t)u * kScatterThreads;
        const bool live = kFull || idx < total_chunks;
        if (!live)
            idx = 0;                    // a safe in-bounds address; result unused
        const int64_t t = kPow2Row ? (idx >> row_shift) : idx / chunks_per_row;
        chunk[u] = idx - t * chunks_per_row;
        slot[u] = live ? slot_mapping[t] : -1;
        x[u] = load16(src + t * stride16 + chunk[u]);
    }
    // Pin the payload in registers here.  Without this the compiler sinks the
    // loads into the store branches below, after the slot test, and the lane
    // then has one load in flight at a time instead of kScatterUnroll.
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u)
        __asm__ volatile("" : "+v"(x[u]));
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
        if (slot[u] < 0)
            continue;                   // padding token: nothing to write
        if ((int64_t)slot[u] >= num_slots) {
            flags |= PKV_ST_SLOT_OOR;
            continue;
        }
        store16(x[u], cache + (int64_t)slot[u] * chunks_per_row + chunk[u]);
    }
}

// Workgroups [0, half) write K, [half, 2 half) write V; workgroup w of either
// half moves chunks [w, w + 1) * kChunksPerBlock.  The slot range is reported
// once, by the K half.
template <bool kPow2Row>
__global__ __launch_bounds__(kScatterThreads) void k_scatter(
    int64_t total_chunks, int32_t chunks_per_row, int32_t row_shift,
    const u32x4* __restrict__ k, int64_t k_stride16, const u32x4* __restrict__ v,
    int64_t v_stride16, u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
    int64_t num_slots, const int32_t* __restrict__ slot_mapping, uint32_t* __restrict__ status)
{
    const int64_t half = (total_chunks + kChunksPerBlock - 1) / kChunksPerBlock;
    const bool is_v = (int64_t)blockIdx.x >= half;              // uniform
    const int64_t w = is_v ? (int64_t)blockIdx.x - half : (int64_t)blockIdx.x;
    const int64_t block0 = w * kChunksPerBlock;
    const u32x4* src = is_v ? v : k;
    const int64_t stride16 = is_v ? v_stride16 : k_stride16;
    u32x4* cache = is_v ? v_cache : k_cache;
    uint32_t flags = 0;
    if (block0 + kChunksPerBlock <= total_chunks)
        scatter_chunks<kPow2Row, true>(block0 + threadIdx.x, total_chunks, chunks_per_row,
                                       row_shift, src, stride16, cache, num_slots, slot_mapping,
                                       flags);
    else
        scatter_chunks<kPow2Row, false>(block0 + threadIdx.x, total_chunks, chunks_per_row,
                                        row_shift, src, stride16, cache, num_slots, slot_mapping,
                                        flags);
    if (is_v)
        flags &= ~(uint32_t)PKV_ST_SLOT_OOR;   // the K half reports the same slots
    report_status(status, flags);
}

}  // namespace

hipError_t launch_scatter(int32_t T, int64_t row_bytes, const void* k, int64_t k_stride,
                          const void* v, int64_t v_stride, void* k_cache, void* v_cache,
                          int64_t num_slots, const int32_t* slot_mapping, uint32_t* status,
                          hipStream_t stream)
{
    const int64_t chunks_per_row = row_bytes / 16;
    const int64_t total = (int64_t)T * chunks_per_row;
    if (total == 0)
        return hipSuccess;
    const int64_t blocks = 2 * ((total + kChunksPerBlock - 1) / kChunksPerBlock);   // K, then V
    const bool pow2 = (chunks_per_row & (chunks_per_row - 1)) == 0;
    const int32_t shift = pow2 ? __builtin_ctzll((unsigned long long)chunks_per_row) : 0;
    const u32x4* kp = static_cast<const u32x4*>(k);
    const u32x4* vp = static_cast<const u32x4*>(v);
    u32x4* kc = static_cast<u32x4*>(k_cache);
    u32x4* vc = static_cast<u32x4*>(v_cache);
    if (pow2)
        k_scatter<true><<<dim3((unsigned)blocks), dim3(kScatterThreads), 0, stream>>>(
            total, (int32_t)chunks_per_row, shift, kp, k_stride / 16, vp, v_stride / 16, kc, vc,
            num_slots, slot_mapping, status);
    else
        k_scatter<false><<<dim3((unsigned)blocks), dim3(kScatterThreads), 0, stream>>>(
            total, (int32_t)chunks_per_row, shift, kp, k_stride / 16, vp, v_stride / 16, kc, vc,
            num_slots, slot_mapping, status);
    return hipGetLastError();
}

}  // namespace pkv
