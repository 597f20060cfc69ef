// gather.hip -- the paged K/V read: every position below seq_len, through the
// visible pages, into one contiguous varlen array.
//
// Attention reads each request's KV range (seq_lens: history plus the new
// tokens) through its visible pages (input_block_tables) by indirect
// addressing ("Complete Input Preparation for the Attention Module" of "Deep
// Dive into vLLM's Scheduling Mechanism: The Complete CPU-to-GPU Mapping
// Pipeline", kongchang.com/en).  For position p of batch row b the address
// chain of its "Multi-Layer Coordinate Conversion Pipeline" runs again: logical
// block p / block_size, offset p % block_size, the physical block from the
// visible pages, slot = block * block_size + offset.  The K and V rows at that
// slot go to row kv_start[b] + p of the outputs, kv_start being the running sum
// of the seq_lens.  It is the exact inverse of the scatter.  For a
// sliding-window group only the positions some new token attends are read,
// from first = max(0, seq_len - count - W + 1) on.
//
// Design (gfx950): a persistent grid of one 512-thread workgroup per compute
// unit.  Every workgroup first forms the running sum of the seq_lens in LDS (at
// most PKV_MAX_BATCH values, 8 per thread, wave scans combined across the eight
// wavefronts).  Then, as in the fused step kernel, copy wavefronts (seven here)
// and one index wavefront split the work: the index wavefront resolves the rows
// of the next tile of at most 256 rows (owner by binary search in LDS, page
// lookup) while the copy wavefronts move the current tile.  Tiles are
// shortened for short reads, so that even those spread over the whole chip.
// Here the loads depend on the slots and the stores do not: the copy
// wavefronts read whole 16-byte chunks of the cache rows at the tile's slots
// (consecutive positions of a page are consecutive slots, so a page is one
// contiguous span) and write the output rows in order.  The index wavefront's
// page loads never queue behind the payload, since a wavefront's memory
// counter only covers its own accesses.  Measured on MI355X, one workgroup of
// seven copy wavefronts per compute unit streams 4-14 % faster than four
// workgroups of three (the fused step's shape), although fewer loads are in
// flight per compute unit.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#ifndef PKV_GATHER_UNROLL
#define PKV_GATHER_UNROLL 6
#endif
#ifndef PKV_GATHER_WGS
#define PKV_GATHER_WGS 256                 // persistent workgroups, at most: one per CU
#endif
#ifndef PKV_GATHER_TARGET_TILES
#define PKV_GATHER_TARGET_TILES 2048       // tiles are shortened until there are this many
#endif
#ifndef PKV_GATHER_MIN_TILE
#define PKV_GATHER_MIN_TILE 16
#endif

constexpr int kCopyWaves = 7;
constexpr int kCopyThreads = kCopyWaves * kWave;
constexpr int kThreads = kCopyThreads + kWave;
constexpr int kUnroll = PKV_GATHER_UNROLL;
constexpr int kChunks = kCopyThreads * kUnroll;     // 16-byte chunks per round
constexpr int kTile = 256;                          // output rows per tile, at most
constexpr int kRowsPerLane = kTile / kWave;
constexpr int kScanPer = PKV_MAX_BATCH / kThreads;  // seq_lens per thread in the scan
static_assert(kScanPer * kThreads == PKV_MAX_BATCH, "the scan covers every batch row");

struct GatherArgs {
    const int32_t* seq_lens;
    const int32_t* qsl;              // query_start_loc (read only for a sliding window)
    const int32_t* pages;            // input_block_tables [n, MB]
    const u32x4* k_cache;
    const u32x4* v_cache;
    u32x4* k_out;
    u32x4* v_out;
    int32_t* kv_start;
    uint32_t* status;
    int64_t k_out_stride16;
    int64_t v_out_stride16;
    int32_t n;
    int32_t MB;
    int32_t block_size;
    int32_t bs_shift;                // log2(block_size), or -1
    int32_t num_blocks;
    int32_t chunks_per_row;
    int32_t row_shift;               // log2(chunks_per_row), or -1
    int32_t window;                  // sliding window, 0 = full attention
    int32_t tile;                    // output rows per tile (a power of two <= kTile)
    int32_t out_tokens;
};

__device__ inline u32x4 nt_load(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ inline void nt_store(u32x4 x, u32x4* p) { __builtin_nontemporal_store(x, p); }

__device__ inline bool is_index_wave()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)) == kCopyWaves;
}

// Running sum of the seq_lens into s_start[0..n] (clamped to out_tokens: rows
// at or past it are never written), by every thread of the workgroup.
// Workgroup 0 also writes kv_start (saturated at INT32_MAX) and the flags of
// the batch as a whole.
template <bool kWindow>
__device__ inline void start_offsets(const GatherArgs& a, int32_t* s_start, int64_t* s_wave,
                                     uint32_t& flags)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int i0 = tid * kScanPer;
    int64_t v[kScanPer];
    // Unconditional loads from clamped in-bounds addresses (n > 0 is uniform).
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
        const int i = i0 + k;
        v[k] = a.n > 0 ? a.seq_lens[i < a.n ? i : a.n - 1] : 0;
        if (i >= a.n)
            v[k] = 0;
    }
    int32_t q[kScanPer + 1];
    const bool windowed = kWindow && a.n > 0;         // uniform; qsl is read only then
    if (windowed) {
#pragma unroll
        for (int k = 0; k <= kScanPer; ++k) {
            const int i = i0 + k;
            q[k] = a.qsl[i < a.n ? i : a.n];
        }
    }
    int64_t total = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
        if (v[k] < 0) {
            flags |= PKV_ST_BAD_COUNT;
            v[k] = 0;
        }
        // A sliding window reads only from the first attended position on.
        if (windowed && i0 + k < a.n)
            v[k] -= window_first(v[k], (int64_t)q[k + 1] - q[k], a.window);
        total += v[k];
    }
    const int64_t incl = wave_inclusive_scan(total);
    if (lane == kWave - 1)
        s_wave[wave] = incl;
    __syncthreads();
    int64_t before = incl - total;
    for (int w = 0; w < wave; ++w)
        before += s_wave[w];
    const bool first = blockIdx.x == 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
        const int i = i0 + k;
        if (i <= a.n) {            // i == n: the grand total
            s_start[i] = (int32_t)(before < a.out_tokens ? before : a.out_tokens);
            if (first && a.kv_start != nullptr)
                a.kv_start[i] = (int32_t)(before < INT32_MAX ? before : INT32_MAX);
        }
        before += v[k];
    }
    if (i0 + kScanPer == PKV_MAX_BATCH && a.n == PKV_MAX_BATCH) {   // last thread, full batch
        s_start[a.n] = (int32_t)(before < a.out_tokens ? before : a.out_tokens);
        if (first && a.kv_start != nullptr)
            a.kv_start[a.n] = (int32_t)(before < INT32_MAX ? before : INT32_MAX);
    }
    if (first && before > a.out_tokens && tid == kThreads - 1)
        flags |= PKV_ST_TOKEN_SUM;
    if (!first)
        flags &= ~(uint32_t)PKV_ST_BAD_COUNT;    // batch-wide flags: workgroup 0 only
}

// Index wavefront: the source slot of each row of a tile, -1 where no page
// can be read (flagged).  All of a lane's page loads are issued together.
template <bool kWindow>
__device__ inline void tile_slots(const GatherArgs& a, const int32_t* s_start, int64_t u0,
                                  int len, int32_t* s_slot, uint32_t& flags)
{
    const int lane = threadIdx.x & (kWave - 1);
    int64_t src[kRowsPerLane];
    int32_t off[kRowsPerLane];
    int owner[kRowsPerLane];
    int64_t first[kRowsPerLane];
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
        const int j = k * kWave + lane;
        owner[k] = j < len ? owner_of(s_start, a.n, u0 + j) : 0;   // in [0, n): u < s_start[n]
        first[k] = 0;
    }
    if (kWindow) {                                    // the window's first position
        int32_t sl[kRowsPerLane], q0[kRowsPerLane], q1[kRowsPerLane];
#pragma unroll
        for (int k = 0; k < kRowsPerLane; ++k) {
            sl[k] = a.seq_lens[owner[k]];
            q0[k] = a.qsl[owner[k]];
            q1[k] = a.qsl[owner[k] + 1];
        }
#pragma unroll
        for (int k = 0; k < kRowsPerLane; ++k)
            first[k] = window_first(sl[k] > 0 ? sl[k] : 0, (int64_t)q1[k] - q0[k], a.window);
    }
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
        const int j = k * kWave + lane;
        src[k] = -1;
        off[k] = 0;
        if (j >= len)
            continue;
        const int64_t u = u0 + j;
        const int b = owner[k];
        const int32_t p = (int32_t)(u - s_start[b] + first[k]);
        const int32_t lb = a.bs_shift >= 0 ? (p >> a.bs_shift) : p / a.block_size;
        off[k] = p - lb * a.block_size;
        if (lb >= a.MB)
            flags |= PKV_ST_LB_OOR;
        else
            src[k] = (int64_t)b * a.MB + lb;
    }
    const bool have_pages = a.MB > 0;                 // uniform
    int32_t blk[kRowsPerLane];
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
        blk[k] = have_pages ? a.pages[src[k] >= 0 ? src[k] : 0] : -1;
        if (src[k] < 0)
            blk[k] = -1;
    }
#pragma unroll
    for (int k = 0; k < kRowsPerLane; ++k) {
        const int j = k * kWave + lane;
        if (j >= len)
            continue;
        int32_t slot = -1;
        if (src[k] >= 0) {
            if (blk[k] < 0 || blk[k] >= a.num_blocks)
                flags |= PKV_ST_BLOCK_OOR;
            else
                slot = blk[k] * a.block_size + off[k];
        }
        s_slot[j] = slot;
    }
}

// Chunk u of round r: its row within the tile, its 16-byte chunk within the
// row, the source slot (-1: nothing to copy) and the cache chunk to load (the
// first chunk of slot 0 when there is nothing to copy, so the load needs no
// branch).
template <bool kPow2Row>
__device__ inline void chunk_at(const GatherArgs& a, const int32_t* s_slot, int len, int r, int u,
                                int& tok, int& c, int32_t& slot, int64_t& src)
{
    const int idx = r * kChunks + u * kCopyThreads + (int)threadIdx.x;
    tok = kPow2Row ? (idx >> a.row_shift) : idx / a.chunks_per_row;
    c = idx - tok * a.chunks_per_row;
    slot = tok < len ? s_slot[tok] : -1;
    src = (int64_t)(slot >= 0 ? slot : 0) * a.chunks_per_row + c;
}

template <bool kPow2Row>
__device__ inline void load_round(const GatherArgs& a, const int32_t* s_slot, int len, int r,
                                  u32x4 (&kv)[kUnroll], u32x4 (&vv)[kUnroll])
{
    const bool have_cache = a.num_blocks > 0;         // uniform
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        int tok, c;
        int32_t slot;
        int64_t src;
        chunk_at<kPow2Row>(a, s_slot, len, r, u, tok, c, slot, src);
        if (have_cache) {
            kv[u] = nt_load(a.k_cache + src);
            vv[u] = nt_load(a.v_cache + src);
        } else {
            kv[u] = u32x4{0, 0, 0, 0};
            vv[u] = kv[u];
        }
    }
}

template <bool kPow2Row>
__device__ inline void store_round(const GatherArgs& a, const int32_t* s_slot, int len, int r,
                                   u32x4* kb, u32x4* vb, u32x4 (&kv)[kUnroll],
                                   u32x4 (&vv)[kUnroll])
{
    // Keep the payload in registers here, so the loads are not sunk into the
    // store branches below.
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        __asm__ volatile("" : "+v"(kv[u]), "+v"(vv[u]));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        int tok, c;
        int32_t slot;
        int64_t src;
        chunk_at<kPow2Row>(a, s_slot, len, r, u, tok, c, slot, src);
        if (slot < 0)
            continue;
        nt_store(kv[u], kb + (int64_t)tok * a.k_out_stride16 + c);
        nt_store(vv[u], vb + (int64_t)tok * a.v_out_stride16 + c);
    }
}

// One payload (K or V) of a tile, two rounds' chunks per lane at a time: all
// 2 * kUnroll loads of a step in flight, then their stores.
template <bool kPow2Row>
__device__ inline void copy_payload(const GatherArgs& a, const int32_t* s_slot, int len,
                                    int rounds, const u32x4* cache, u32x4* out, int64_t stride16)
{
    const bool have_cache = a.num_blocks > 0;         // uniform
    for (int r = 0; r < rounds; r += 2) {
        u32x4 x[2 * kUnroll];
#pragma unroll
        for (int u = 0; u < 2 * kUnroll; ++u) {
            int tok, c;
            int32_t slot;
            int64_t src;
            chunk_at<kPow2Row>(a, s_slot, len, r + u / kUnroll, u % kUnroll, tok, c, slot, src);
            x[u] = have_cache ? nt_load(cache + src) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 2 * kUnroll; ++u)
            __asm__ volatile("" : "+v"(x[u]));           // loads ahead of the store branches
#pragma unroll
        for (int u = 0; u < 2 * kUnroll; ++u) {
            int tok, c;
            int32_t slot;
            int64_t src;
            chunk_at<kPow2Row>(a, s_slot, len, r + u / kUnroll, u % kUnroll, tok, c, slot, src);
            if (slot < 0)
                continue;
            nt_store(x[u], out + (int64_t)tok * stride16 + c);
        }
    }
}

// kSplit (tiles of two rounds or more): all of K, then all of V, two rounds
// per step, so that a workgroup streams one payload at a time (measured on
// MI355X, 256 workgroups: the decode read of 1.07 M rows 1661 -> 1644 us, the
// mixed read of 158k rows 246.7 -> 237.8 us).  Otherwise a round's K and V
// chunks together: a tile of one round would take two round trips instead of
// one, so the 32k-row reads (one round per tile) keep the joint copy, in
// instantiations of their own that keep its register budget.
template <bool kPow2Row, bool kSplit>
__device__ inline void copy_tile(const GatherArgs& a, const int32_t* s_slot, int64_t u0, int len)
{
    u32x4* kb = a.k_out + u0 * a.k_out_stride16;
    u32x4* vb = a.v_out + u0 * a.v_out_stride16;
    const int rounds = (int)(((int64_t)len * a.chunks_per_row + kChunks - 1) / kChunks);
    if constexpr (kSplit) {
        copy_payload<kPow2Row>(a, s_slot, len, rounds, a.k_cache, kb, a.k_out_stride16);
        copy_payload<kPow2Row>(a, s_slot, len, rounds, a.v_cache, vb, a.v_out_stride16);
    } else {
        for (int r = 0; r < rounds; ++r) {
            u32x4 kv[kUnroll];
            u32x4 vv[kUnroll];
            load_round<kPow2Row>(a, s_slot, len, r, kv, vv);
            store_round<kPow2Row>(a, s_slot, len, r, kb, vb, kv, vv);
        }
    }
}

template <bool kPow2Row, bool kWindow, bool kSplit>
__global__ __launch_bounds__(kThreads) void k_gather(const GatherArgs a)
{
    __shared__ int32_t s_start[PKV_MAX_BATCH + 1];
    __shared__ int64_t s_wave[kThreads / kWave];
    __shared__ int32_t s_slot[2 * kTile];

    uint32_t flags = 0;
    start_offsets<kWindow>(a, s_start, s_wave, flags);
    __syncthreads();
    const int64_t rows = s_start[a.n];                   // rows to write (uniform)
    const int64_t tiles = (rows + a.tile - 1) / a.tile;
    const int64_t G = gridDim.x;
    auto tile_len = [&](int64_t t) {
        const int64_t u0 = t * a.tile;
        return (int)(rows - u0 < a.tile ? rows - u0 : a.tile);
    };
    // Barriers per role: one after the first tile's slots, then one per tile.
    int buf = 0;
    if (is_index_wave()) {
        int64_t tile = blockIdx.x;
        if (tile < tiles)
            tile_slots<kWindow>(a, s_start, tile * a.tile, tile_len(tile), s_slot, flags);
        __syncthreads();
        for (; tile < tiles; tile += G) {
            const int64_t next = tile + G;
            if (next < tiles)
                tile_slots<kWindow>(a, s_start, next * a.tile, tile_len(next),
                                    s_slot + (buf ^ 1) * kTile, flags);
            __syncthreads();
            buf ^= 1;
        }
    } else {
        __syncthreads();
        for (int64_t tile = blockIdx.x; tile < tiles; tile += G) {
            copy_tile<kPow2Row, kSplit>(a, s_slot + buf * kTile, tile * a.tile, tile_len(tile));
            __syncthreads();
            buf ^= 1;
        }
    }
    report_status(a.status, flags);
}

}  // namespace

hipError_t launch_gather(int32_t n, const int32_t* seq_lens, const int32_t* query_start_loc,
                         int32_t sliding_window, const int32_t* input_block_tables, int32_t MB,
                         int32_t block_size, int32_t num_blocks, int64_t row_bytes,
                         const void* k_cache, const void* v_cache, int32_t out_tokens,
                         void* k_out, int64_t k_out_stride, void* v_out, int64_t v_out_stride,
                         int32_t* kv_start, uint32_t* status, hipStream_t stream)
{
    if (n == 0 && kv_start == nullptr)
        return hipSuccess;
    GatherArgs a;
    a.seq_lens = seq_lens;
    a.qsl = query_start_loc;
    a.window = sliding_window;
    a.pages = input_block_tables;
    a.k_cache = static_cast<const u32x4*>(k_cache);
    a.v_cache = static_cast<const u32x4*>(v_cache);
    a.k_out = static_cast<u32x4*>(k_out);
    a.v_out = static_cast<u32x4*>(v_out);
    a.kv_start = kv_start;
    a.status = status;
    a.k_out_stride16 = k_out_stride / 16;
    a.v_out_stride16 = v_out_stride / 16;
    a.n = n;
    a.MB = MB;
    a.block_size = block_size;
    a.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
    a.num_blocks = num_blocks;
    a.chunks_per_row = (int32_t)(row_bytes / 16);
    a.row_shift = (a.chunks_per_row & (a.chunks_per_row - 1)) == 0
                      ? __builtin_ctz((unsigned)a.chunks_per_row) : -1;
    // Tiles as long as kTile rows, shortened (by halves) while the output has
    // fewer than PKV_GATHER_TARGET_TILES of them, so a short read still spreads
    // over the whole chip; but never below PKV_GATHER_MIN_TILE rows nor below
    // the largest power of two of rows that one round of the copy wavefronts
    // moves (128 rows of 256 bytes: a 32k-row read of such rows is one tile per
    // workgroup, 9.4 us on MI355X; with tiles of 16 rows such reads took
    // 13.5-15 us).
    int min_tile = PKV_GATHER_MIN_TILE;
    while (min_tile < kTile && (int64_t)min_tile * 2 * a.chunks_per_row <= kChunks)
        min_tile <<= 1;
    a.tile = kTile;
    while (a.tile > min_tile &&
           ((int64_t)out_tokens + a.tile - 1) / a.tile < PKV_GATHER_TARGET_TILES)
        a.tile >>= 1;
    a.out_tokens = out_tokens;
    const int64_t tiles = ((int64_t)out_tokens + a.tile - 1) / a.tile;
    const int64_t grid = tiles < 1 ? 1 : (tiles < PKV_GATHER_WGS ? tiles : PKV_GATHER_WGS);
    // The window's extra index work gets instantiations of its own, so that
    // full-attention reads keep their register budget; so does the payload
    // order (K then V once a full tile takes two rounds or more).
    const dim3 g((unsigned)grid), b(kThreads);
    const bool split = (int64_t)a.tile * a.chunks_per_row > kChunks;
#define PKV_GATHER_LAUNCH(P, W)                                                                    \
    do {                                                                                           \
        if (split)                                                                                 \
            k_gather<P, W, true><<<g, b, 0, stream>>>(a);                                          \
        else                                                                                       \
            k_gather<P, W, false><<<g, b, 0, stream>>>(a);                                         \
    } while (0)
    if (a.row_shift >= 0 && a.window == 0)
        PKV_GATHER_LAUNCH(true, false);
    else if (a.row_shift >= 0)
        PKV_GATHER_LAUNCH(true, true);
    else if (a.window == 0)
        PKV_GATHER_LAUNCH(false, false);
    else
        PKV_GATHER_LAUNCH(false, true);
#undef PKV_GATHER_LAUNCH
    return hipGetLastError();
}

}  // namespace pkv
