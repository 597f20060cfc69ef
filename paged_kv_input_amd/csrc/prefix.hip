// prefix.hip -- prefix-cache block hashes and the prefix index.
//
// A request's full token blocks are hashed together with their prefix context
// and looked up in the block pool's hash index; hit blocks are reused as they
// are and only the rest is computed; blocks whose contents are settled are
// registered ("Prefix Cache" and "allocate_slots()" of "从源码读 vLLM
// Scheduler：一轮调度如何分配请求与 KV Cache", caffein.top).
//
// The hash (the pages fix only what it covers): FNV-1a 64 (Fowler, Noll, Vo)
// of each full block's little-endian token bytes, c_i; the prefix context
// s_i = s_{i-1} * P + c_i (mod 2^64, P = the FNV-1a 64 prime, s_{-1} = 0);
// the block's hash h_i = FNV-1a 64 of s_i's 8 little-endian bytes, 0 replaced
// by 1 (0 marks an unused index entry).
//
// Design (gfx950): every block's content hash is independent, and the chain
// is an affine recurrence, s_i = A(s_{i-1}) with A(x) = x * P + c_i; affine
// maps compose associatively, so one workgroup per request hashes 256 blocks
// at a time and chains them with a workgroup scan of (multiplier, addend)
// pairs instead of walking the blocks one after another.  The index is an
// open-addressing table of power-of-two capacity: 64-bit keys (0 = unused),
// int32 blocks (INT32_MAX = none), linear probing from the key's low bits.
// Registration claims a slot with a 64-bit compare-and-swap and keeps the
// smallest block with atomicMin, so concurrent registrations of one hash end
// the same way in any order.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

constexpr uint64_t kFnvBasis = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;
constexpr int32_t kNoBlock = INT32_MAX;
// One workgroup per request, of as many threads as the block-table width
// (MB, the most blocks a request can have) needs, at least one wavefront and
// at most: 256 for hashing, which is bound by the byte-serial FNV multiplies;
// 1024 for the index probes, which are bound by memory latency, so that a long
// request's blocks take fewer rounds (measured on MI355X, 512 requests of up
// to 1056 blocks: lookup 16 -> 12 us, insert 19.6 -> 16.6 us; 1024-thread
// hashing was slower).  Narrow tables get narrow workgroups, so that more
// requests are resident at once (4096 requests with tables of 128 blocks:
// lookup 28.9 -> 11.2 us, hashing 19.3 -> 12.3 us).
constexpr int kHashMaxThreads = 256;
constexpr int kIndexMaxThreads = 1024;
constexpr int kFlatThreads = 256;         // flat grids: eviction, clearing

__device__ inline uint64_t fnv_byte(uint64_t h, uint32_t byte)
{
    return (h ^ byte) * kFnvPrime;
}

__device__ inline uint64_t fnv_word(uint64_t h, uint32_t w)      // 4 little-endian bytes
{
    h = fnv_byte(h, w & 0xffu);
    h = fnv_byte(h, (w >> 8) & 0xffu);
    h = fnv_byte(h, (w >> 16) & 0xffu);
    return fnv_byte(h, w >> 24);
}

__device__ inline uint64_t shfl_up64(uint64_t x, int d)
{
    const uint32_t lo = __shfl_up((uint32_t)x, d, kWave);
    const uint32_t hi = __shfl_up((uint32_t)(x >> 32), d, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive scan of affine maps x -> x * a + b across a wavefront: lane l ends
// with the composition of lanes 0..l (lane 0's map applied first).
__device__ inline void wave_affine_scan(uint64_t& a, uint64_t& b)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t pa = shfl_up64(a, d);
        const uint64_t pb = shfl_up64(b, d);
        if (lane >= d) {          // (earlier map) then (this map)
            b = pb * a + b;
            a = pa * a;
        }
    }
}

template <int kHashThreads>
__global__ __launch_bounds__(kHashThreads) void k_hash_blocks(
    const int32_t* __restrict__ tokens, int64_t total, const int64_t* __restrict__ starts,
    const int32_t* __restrict__ lengths, int32_t block_size, int32_t MB,
    uint64_t* __restrict__ hashes, int32_t* __restrict__ num_full, uint32_t* __restrict__ status)
{
    __shared__ uint64_t s_a[kHashThreads / kWave];
    __shared__ uint64_t s_b[kHashThreads / kWave];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    uint32_t flags = 0;
    int64_t len = lengths[b];
    const int64_t start = starts[b];
    if (len < 0) {
        flags |= tid == 0 ? PKV_ST_BAD_COUNT : 0u;
        len = 0;
    }
    int64_t full = 0;
    if (start < 0 || start + len > total) {
        flags |= tid == 0 ? PKV_ST_BAD_RANGE : 0u;
    } else {
        full = len / block_size;
        if (full > MB) {
            flags |= tid == 0 ? PKV_ST_LB_OOR : 0u;
            full = MB;
        }
    }
    uint64_t carry = 0;                               // s of the block before the chunk
    for (int64_t i0 = 0; i0 < full; i0 += kHashThreads) {
        const int64_t i = i0 + tid;
        // Content hash of block i (lanes past the last block hash block i0).
        const int32_t* blk = tokens + start + (i < full ? i : i0) * block_size;
        uint64_t c = kFnvBasis;
        // Eight token loads in flight per wait, then their bytes in order.
        int32_t j = 0;
        for (; j + 8 <= block_size; j += 8) {
            uint32_t t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                t[u] = (uint32_t)blk[j + u];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                c = fnv_word(c, t[u]);
        }
        for (; j < block_size; ++j)
            c = fnv_word(c, (uint32_t)blk[j]);
        // Compose the chunk's maps x -> x * P + c_i.
        uint64_t a = kFnvPrime, add = c;
        wave_affine_scan(a, add);
        if (lane == kWave - 1) {
            s_a[wave] = a;
            s_b[wave] = add;
        }
        __syncthreads();
        uint64_t x = carry;                           // s before this wavefront's lanes
        for (int w = 0; w < wave; ++w)
            x = x * s_a[w] + s_b[w];
        const uint64_t s = x * a + add;
        uint64_t h = kFnvBasis;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            h = fnv_byte(h, (uint32_t)(s >> (8 * k)) & 0xffu);
        if (i < full)
            hashes[(int64_t)b * MB + i] = h == 0 ? 1 : h;
        // The carry for the next chunk: s after the chunk's last block.
        uint64_t last = carry;
        for (int w = 0; w < kHashThreads / kWave; ++w)
            last = last * s_a[w] + s_b[w];
        carry = last;
        __syncthreads();                              // s_a / s_b are reused
    }
    if (tid == 0 && num_full != nullptr)
        num_full[b] = (int32_t)full;
    report_status(status, flags);
}

// Slot of `key` in the table, or -1 when it is not there (an unused slot, or
// every slot probed).
__device__ inline int64_t probe(const uint64_t* keys, int64_t capacity, uint64_t key)
{
    const int64_t mask = capacity - 1;
    int64_t slot = (int64_t)(key & (uint64_t)mask);
    for (int64_t n = 0; n < capacity; ++n) {
        const uint64_t k = keys[slot];
        if (k == key)
            return slot;
        if (k == 0)
            return -1;
        slot = (slot + 1) & mask;
    }
    return -1;
}

template <int kLookupThreads>
__global__ __launch_bounds__(kLookupThreads) void k_prefix_lookup(
    const uint64_t* __restrict__ hashes, int32_t MB, const int32_t* __restrict__ lengths,
    int32_t block_size, const uint64_t* __restrict__ keys, const int32_t* __restrict__ vals,
    int64_t capacity, int32_t* __restrict__ hit_blocks, int32_t* __restrict__ num_computed,
    uint32_t* __restrict__ status)
{
    __shared__ int32_t s_first_miss;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    uint32_t flags = 0;
    int64_t len = lengths[b];
    if (len < 0) {
        flags |= tid == 0 ? PKV_ST_BAD_COUNT : 0u;
        len = 0;
    }
    int64_t cap = len > 0 ? (len - 1) / block_size : 0;   // a hit never covers the last token
    if (cap > MB)
        cap = MB;
    int64_t hits = 0;
    for (int64_t i0 = 0; i0 < cap; i0 += kLookupThreads) {
        const int chunk = (int)(cap - i0 < kLookupThreads ? cap - i0 : kLookupThreads);
        if (tid == 0)
            s_first_miss = chunk;
        __syncthreads();
        int32_t block = kNoBlock;
        if (tid < chunk) {
            const uint64_t key = hashes[(int64_t)b * MB + i0 + tid];
            const int64_t at = key != 0 && capacity > 0 ? probe(keys, capacity, key) : -1;
            if (at >= 0)
                block = vals[at];
            if (block == kNoBlock)
                atomicMin(&s_first_miss, tid);
        }
        __syncthreads();
        const int first_miss = s_first_miss;         // uniform
        if (tid < first_miss && hit_blocks != nullptr)
            hit_blocks[(int64_t)b * MB + i0 + tid] = block;
        hits += first_miss;
        __syncthreads();                              // s_first_miss is reused
        if (first_miss < chunk)
            break;
    }
    if (tid == 0)
        num_computed[b] = (int32_t)(hits * block_size);
    report_status(status, flags);
}

template <int kInsertThreads>
__global__ __launch_bounds__(kInsertThreads) void k_prefix_insert(
    const uint64_t* __restrict__ hashes, int32_t MB, const int32_t* __restrict__ lo,
    const int32_t* __restrict__ hi, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ block_table, int32_t R, uint64_t* __restrict__ keys,
    int32_t* __restrict__ vals, int64_t capacity, uint32_t* __restrict__ status)
{
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    uint32_t flags = 0;
    const int32_t r = rows[b];
    const int32_t first = lo[b], last = hi[b];
    if (r < 0 || r >= R) {
        flags |= tid == 0 ? PKV_ST_BAD_ROW : 0u;
    } else if (first < 0 || last < first || last > MB) {
        flags |= tid == 0 ? PKV_ST_BAD_RANGE : 0u;
    } else {
        const int64_t mask = capacity - 1;
        for (int32_t i = first + tid; i < last; i += kInsertThreads) {
            const int32_t block = block_table[(int64_t)r * MB + i];
            const uint64_t key = hashes[(int64_t)b * MB + i];
            if (block < 0 || block == kNoBlock) {
                flags |= PKV_ST_BLOCK_OOR;
                continue;
            }
            if (key == 0)
                continue;                             // marks unused slots; never a hash
            int64_t slot = (int64_t)(key & (uint64_t)mask);
            bool done = false;
            for (int64_t n = 0; n < capacity && !done; ++n) {
                uint64_t k = keys[slot];
                if (k == 0) {
                    k = atomicCAS((unsigned long long*)&keys[slot], 0ull,
                                  (unsigned long long)key);
                    if (k == 0)
                        k = key;                      // claimed it
                }
                if (k == key) {
                    atomicMin(&vals[slot], block);
                    done = true;
                } else {
                    slot = (slot + 1) & mask;
                }
            }
            if (!done)
                flags |= PKV_ST_TABLE_FULL;
        }
    }
    report_status(status, flags);
}

__global__ __launch_bounds__(kFlatThreads) void k_prefix_evict(
    int32_t count, const uint64_t* __restrict__ hashes, const int32_t* __restrict__ blocks,
    const uint64_t* __restrict__ keys, int32_t* __restrict__ vals, int64_t capacity)
{
    const int64_t i = (int64_t)blockIdx.x * kFlatThreads + threadIdx.x;
    if (i >= count)
        return;
    const uint64_t key = hashes[i];
    const int64_t at = key != 0 ? probe(keys, capacity, key) : -1;
    if (at >= 0)
        atomicCAS(&vals[at], blocks[i], kNoBlock);
}

__global__ __launch_bounds__(kFlatThreads) void k_prefix_clear(uint64_t* __restrict__ keys,
                                                                 int32_t* __restrict__ vals,
                                                                 int64_t capacity)
{
    const int64_t stride = (int64_t)gridDim.x * kFlatThreads;
    for (int64_t i = (int64_t)blockIdx.x * kFlatThreads + threadIdx.x; i < capacity; i += stride) {
        keys[i] = 0;
        vals[i] = kNoBlock;
    }
}

// Threads of a request's workgroup: the smallest power of two from one
// wavefront up to `most` that covers MB blocks.
__host__ inline int request_threads(int32_t MB, int most)
{
    int t = kWave;
    while (t < most && t < MB)
        t *= 2;
    return t;
}

}  // namespace

hipError_t launch_hash_blocks(int32_t m, const int32_t* tokens, int64_t total,
                              const int64_t* starts, const int32_t* lengths, int32_t block_size,
                              int32_t MB, uint64_t* hashes, int32_t* num_full, uint32_t* status,
                              hipStream_t stream)
{
    if (m == 0)
        return hipSuccess;
#define PKV_HASH_LAUNCH(W)                                                                         \
    k_hash_blocks<W><<<dim3((unsigned)m), dim3(W), 0, stream>>>(tokens, total, starts, lengths,    \
                                                                block_size, MB, hashes, num_full, \
                                                                status)
    switch (request_threads(MB, kHashMaxThreads)) {
    case 64: PKV_HASH_LAUNCH(64); break;
    case 128: PKV_HASH_LAUNCH(128); break;
    default: PKV_HASH_LAUNCH(256); break;
    }
#undef PKV_HASH_LAUNCH
    return hipGetLastError();
}

hipError_t launch_prefix_lookup(int32_t m, const uint64_t* hashes, int32_t MB,
                                const int32_t* lengths, int32_t block_size, const uint64_t* keys,
                                const int32_t* vals, int64_t capacity, int32_t* hit_blocks,
                                int32_t* num_computed, uint32_t* status, hipStream_t stream)
{
    if (m == 0)
        return hipSuccess;
#define PKV_LOOKUP_LAUNCH(W)                                                                       \
    k_prefix_lookup<W><<<dim3((unsigned)m), dim3(W), 0, stream>>>(                                \
        hashes, MB, lengths, block_size, keys, vals, capacity, hit_blocks, num_computed, status)
    switch (request_threads(MB, kIndexMaxThreads)) {
    case 64: PKV_LOOKUP_LAUNCH(64); break;
    case 128: PKV_LOOKUP_LAUNCH(128); break;
    case 256: PKV_LOOKUP_LAUNCH(256); break;
    case 512: PKV_LOOKUP_LAUNCH(512); break;
    default: PKV_LOOKUP_LAUNCH(1024); break;
    }
#undef PKV_LOOKUP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_prefix_insert(int32_t m, const uint64_t* hashes, int32_t MB, const int32_t* lo,
                                const int32_t* hi, const int32_t* rows,
                                const int32_t* block_table, int32_t R, uint64_t* keys,
                                int32_t* vals, int64_t capacity, uint32_t* status,
                                hipStream_t stream)
{
    if (m == 0)
        return hipSuccess;
#define PKV_INSERT_LAUNCH(W)                                                                       \
    k_prefix_insert<W><<<dim3((unsigned)m), dim3(W), 0, stream>>>(                                \
        hashes, MB, lo, hi, rows, block_table, R, keys, vals, capacity, status)
    switch (request_threads(MB, kIndexMaxThreads)) {
    case 64: PKV_INSERT_LAUNCH(64); break;
    case 128: PKV_INSERT_LAUNCH(128); break;
    case 256: PKV_INSERT_LAUNCH(256); break;
    case 512: PKV_INSERT_LAUNCH(512); break;
    default: PKV_INSERT_LAUNCH(1024); break;
    }
#undef PKV_INSERT_LAUNCH
    return hipGetLastError();
}

hipError_t launch_prefix_evict(int32_t count, const uint64_t* hashes, const int32_t* blocks,
                               uint64_t* keys, int32_t* vals, int64_t capacity,
                               hipStream_t stream)
{
    if (count == 0)
        return hipSuccess;
    const unsigned grid = (unsigned)(((int64_t)count + kFlatThreads - 1) / kFlatThreads);
    k_prefix_evict<<<dim3(grid), dim3(kFlatThreads), 0, stream>>>(count, hashes, blocks, keys,
                                                                   vals, capacity);
    return hipGetLastError();
}

hipError_t launch_prefix_clear(uint64_t* keys, int32_t* vals, int64_t capacity, hipStream_t stream)
{
    if (capacity == 0)
        return hipSuccess;
    const int64_t want = (capacity + kFlatThreads - 1) / kFlatThreads;
    const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
    k_prefix_clear<<<dim3(grid), dim3(kFlatThreads), 0, stream>>>(keys, vals, capacity);
    return hipGetLastError();
}

}  // namespace pkv
