// step.hip -- a whole step in one launch: batch assembly and flattening, every
// KV-cache group's write slots and visible pages, and every group's K/V write
// for one layer.  Its results are exactly those of pkv_prepare_batch followed by
// pkv_compute_slot_mapping and pkv_scatter_kv for each group (the chain of
// "Deep Dive into vLLM's Scheduling Mechanism: The Complete CPU-to-GPU Mapping
// Pipeline", kongchang.com/en: batch construction, flattening, the
// coordinate-conversion pipeline and the K/V write at slot_mapping).
//
// Design (gfx950): the grid is the K/V copy.  Each workgroup owns a tile of
// flat tokens of one group and has three copy wavefronts plus one index
// wavefront, one per SIMD.  The copy wavefronts issue the tile's K/V loads at
// once (18 KiB of each per round; they depend on nothing) and wait at a
// single barrier.
// Meanwhile the index wavefront orders the batch itself (wave_gather /
// rank_sort_wave or block_sort / wave_finish: for at most 64 requests the
// index wavefront alone ranks every key by counting the keys before it, in
// LDS; for more, every wavefront joins a bitonic sort held in registers, with
// one to three exchanges through LDS; then a wave-level scan), resolves the
// tile's tokens to requests by binary search, and computes positions, input
// ids and slots.  After the
// barrier the copy wavefronts write the held rows to their slots.  Splitting
// the roles across wavefronts matters: a wavefront's loads complete in issue
// order, so index loads issued behind the payload would wait for all of it.
// No grid-wide barrier, second launch or device-side counter is needed.
// Workgroup 0 writes the per-request outputs; group 0's workgroups write
// positions and input ids; extra workgroups per group copy the visible
// block-table prefixes (one wavefront per batch row).
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Launch geometry (geometry.h): kStepThreads threads per workgroup, kStepChunks
// 16-byte chunks of K (and of V) per round, tiles of step_tile_tokens() rows.
constexpr int kCopyThreads = kStepCopyThreads;
constexpr int kTokensPerLane = kStepMaxTile / kWave;
constexpr int kPageRows = kStepPageRows;

struct StepGroup {
    const int32_t* block_table;
    int32_t* slot_mapping;
    int32_t* input_block_tables;
    const u32x4* k;
    const u32x4* v;
    u32x4* k_cache;
    u32x4* v_cache;
    int64_t k_stride16;
    int64_t v_stride16;
    int64_t num_slots;
    int32_t MB;
    int32_t block_size;
    int32_t bs_shift;        // log2(block_size), or -1
    int32_t num_blocks;
    int32_t chunks_per_row;
    int32_t row_shift;       // log2(chunks_per_row), or -1
    int32_t tile_tokens;
    int32_t rounds;          // ceil(tile_tokens * chunks_per_row / kStepChunks)
    int32_t first_block;     // first workgroup of this group's tiles
    int32_t tiles;           // ceil(T / tile_tokens)
    int32_t tile_blocks;     // persistent workgroups walking those tiles
    int32_t page_blocks;
    int32_t window;          // sliding window, 0 = full attention
};

struct StepArgs {
    const int32_t* sched_rows;
    const int32_t* num_scheduled;
    const int32_t* completed;
    const int32_t* token_ids;
    int32_t* index_mapping;
    int32_t* query_start_loc;
    int32_t* seq_lens;
    int32_t* positions;
    int32_t* input_ids;
    uint32_t* status;
    int64_t token_stride;
    int32_t n;
    int32_t T;
    int32_t R;
    int32_t L;
    int32_t num_groups;
    StepGroup g[PKV_STEP_MAX_GROUPS];
};

__device__ inline u32x4 nt_load(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ inline void nt_store(u32x4 x, u32x4* p) { __builtin_nontemporal_store(x, p); }

// Token within the tile and 16-byte chunk within its row of lane chunk u of a
// round; tok = -1 past the tile.  Recomputed where needed instead of kept in
// registers.
template <bool kPow2Row>
__device__ inline void chunk_of(const StepGroup& g, int tile_len, int round, int u, int& tok,
                                int& c)
{
    const int idx = round * kStepChunks + u * kCopyThreads + (int)threadIdx.x;
    tok = kPow2Row ? (idx >> g.row_shift) : idx / g.chunks_per_row;
    c = idx - tok * g.chunks_per_row;
    if (tok >= tile_len) {
        tok = -1;
        c = 0;
    }
}

// Issue one round of a tile's K/V loads; chunks past the tile load the
// tile's first chunk instead (harmless, keeps the code branch-free).
template <bool kPow2Row>
__device__ inline void load_round(const StepGroup& g, int64_t t0, int tile_len, int round,
                                  u32x4 (&kv)[kStepUnroll], u32x4 (&vv)[kStepUnroll])
{
    // Uniform tile bases plus 32-bit offsets (the host keeps a tile's span
    // under 4 GiB): one address register per load instead of two.
    const u32x4* kb = g.k + t0 * g.k_stride16;
    const u32x4* vb = g.v + t0 * g.v_stride16;
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u) {
        int tok, c;
        chunk_of<kPow2Row>(g, tile_len, round, u, tok, c);
        const uint32_t t = (uint32_t)(tok >= 0 ? tok : 0);
        kv[u] = nt_load(kb + (t * (uint32_t)g.k_stride16 + (uint32_t)c));
        vv[u] = nt_load(vb + (t * (uint32_t)g.v_stride16 + (uint32_t)c));
    }
}

template <bool kPow2Row>
__device__ inline void store_round(const StepGroup& g, const int32_t* s_slot, int tile_len,
                                   int round, u32x4 (&kv)[kStepUnroll], u32x4 (&vv)[kStepUnroll],
                                   uint32_t& flags)
{
    // Pin the payload in registers here, so the loads stay ahead of the slot
    // tests instead of being sunk into the store branches.
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u)
        __asm__ volatile("" : "+v"(kv[u]), "+v"(vv[u]));
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u) {
        int tok, c;
        chunk_of<kPow2Row>(g, tile_len, round, u, tok, c);
        if (tok < 0)
            continue;
        const int32_t slot = s_slot[tok];
        if (slot < 0)
            continue;
        if ((int64_t)slot >= g.num_slots) {
            flags |= PKV_ST_SLOT_OOR;
            continue;
        }
        const int64_t dst = (int64_t)slot * g.chunks_per_row + c;
        nt_store(kv[u], g.k_cache + dst);
        nt_store(vv[u], g.v_cache + dst);
    }
}

// Token phase of a tile, run by the index wavefront: position, input id
// (group 0) and slot of each token, with the same results and flags as
// pkv_prepare_batch and pkv_compute_slot_mapping.  All of a lane's
// block-table and token-table loads are issued together.
__device__ inline void tile_tokens(const StepArgs& a, const StepGroup& g, bool first_group,
                                   const BatchLds<PKV_STEP_MAX_BATCH, 1, true>& lds, int64_t t0,
                                   int tile_len, int32_t* s_slot, uint32_t& flags)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t* s_row = lds.row();
    const int32_t* s_done = lds.done();
    int32_t pos_out[kTokensPerLane];
    int64_t id_src[kTokensPerLane];
    int64_t bt_src[kTokensPerLane];
    int32_t off[kTokensPerLane];
#pragma unroll
    for (int u = 0; u < kTokensPerLane; ++u) {
        const int j = u * kWave + lane;
        const int64_t t = t0 + j;
        pos_out[u] = -1;
        id_src[u] = -1;
        bt_src[u] = -1;
        off[u] = 0;
        if (j >= tile_len)
            continue;
        const int b = owner_of(lds.qsl, a.n, t);
        if (b < 0 || b >= a.n)
            continue;                                   // past the last request
        const int32_t row = s_row[b];
        if (row < 0 || row >= a.R) {
            flags |= PKV_ST_BAD_ROW;
            continue;
        }
        const int64_t p = (int64_t)s_done[b] + (t - lds.qsl[b]);
        pos_out[u] = (int32_t)(uint32_t)(uint64_t)p;
        if (first_group) {
            if (p < 0 || (a.input_ids != nullptr && p >= a.L))
                flags |= PKV_ST_POS_OOR;
            else if (a.input_ids != nullptr)
                id_src[u] = (int64_t)row * a.token_stride + p;
        }
        if (pos_out[u] < 0) {
            flags |= PKV_ST_POS_OOR;
            continue;
        }
        const int32_t lb = g.bs_shift >= 0 ? (pos_out[u] >> g.bs_shift) : pos_out[u] / g.block_size;
        off[u] = pos_out[u] - lb * g.block_size;
        if (lb >= g.MB) {
            flags |= PKV_ST_LB_OOR;
            continue;
        }
        bt_src[u] = (int64_t)row * g.MB + lb;
    }
    // Unconditional loads from clamped in-bounds addresses (see
    // wave_gather), so all of a lane's lookups are in flight together.
    // A valid source exists only when the table is non-empty (uniform test).
    const int parts = (tile_len + kWave - 1) / kWave;      // uniform
    const bool have_bt = a.R > 0 && g.MB > 0;
    const bool have_ids = a.input_ids != nullptr && a.R > 0 && a.L > 0;
    int32_t blk[kTokensPerLane];
    int32_t ids[kTokensPerLane];
#pragma unroll
    for (int u = 0; u < kTokensPerLane; ++u) {
        blk[u] = (u < parts && have_bt) ? g.block_table[bt_src[u] >= 0 ? bt_src[u] : 0] : -1;
        ids[u] = (u < parts && have_ids) ? a.token_ids[id_src[u] >= 0 ? id_src[u] : 0] : -1;
        if (bt_src[u] < 0)
            blk[u] = -1;
        if (id_src[u] < 0)
            ids[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < kTokensPerLane; ++u) {
        const int j = u * kWave + lane;
        if (j >= tile_len)
            continue;
        const int64_t t = t0 + j;
        int32_t slot = -1;
        if (bt_src[u] >= 0) {
            if (blk[u] < 0 || blk[u] >= g.num_blocks)
                flags |= PKV_ST_BLOCK_OOR;
            else
                slot = blk[u] * g.block_size + off[u];
        }
        if (first_group) {
            a.positions[t] = pos_out[u];
            if (a.input_ids != nullptr)
                a.input_ids[t] = ids[u];
        }
        g.slot_mapping[t] = slot;
        s_slot[j] = slot;
    }
}

__device__ inline void copy_pages(const StepArgs& a, const StepGroup& g,
                                  BatchLds<PKV_STEP_MAX_BATCH, 1, true>& lds, int b,
                                  uint32_t& flags)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (b >= a.n)
        return;
    const int32_t row = lds.row()[b];
    if (row < 0 || row >= a.R) {
        flags |= PKV_ST_BAD_ROW;
        return;
    }
    const int32_t sl = (int32_t)(uint32_t)(uint64_t)((int64_t)lds.done()[b] + lds.count[b]);
    int64_t visible = sl <= 0 ? 0 : ((int64_t)sl + g.block_size - 1) / g.block_size;
    if (visible > g.MB) {
        flags |= PKV_ST_LB_OOR;
        visible = g.MB;
    }
    // Pages before the window may be -1 holes (freed blocks).
    const int64_t first_block =
        window_first(sl, (int64_t)lds.qsl[b + 1] - lds.qsl[b], g.window) / g.block_size;
    const int32_t* src = g.block_table + (int64_t)row * g.MB;
    int32_t* dst = g.input_block_tables + (int64_t)b * g.MB;
    for (int64_t i0 = 0; i0 < visible; i0 += kWave * 4) {
        int32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * kWave + lane;
            v[u] = i < visible ? src[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * kWave + lane;
            if (i < visible) {
                const bool hole = i < first_block && v[u] == -1;
                if ((v[u] < 0 || v[u] >= g.num_blocks) && !hole)
                    flags |= PKV_ST_BLOCK_OOR;
                dst[i] = v[u];
            }
        }
    }
}

// Role of the calling wavefront as a scalar (SGPR) value, so that branches on
// it are uniform jumps: each wavefront runs exactly one role's code, and each
// role's code has the same sequence of barriers.  Keeping the roles in
// separate code paths also lets the copy payload and the index temporaries
// share registers.
__device__ inline bool is_index_wave()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)) == PKV_STEP_COPY_WAVES;
}

// kBig: more than 64 requests, ordered by every wavefront (block_sort); the
// two orderings get instantiations of their own.
template <bool kPow2Row, bool kBig>
__global__ __launch_bounds__(kStepThreads) void k_step(const StepArgs a)
{
    __shared__ WaveBatchLds<PKV_STEP_MAX_BATCH> wlds;
    __shared__ int32_t s_slot[2 * kStepMaxTile];
    BatchLds<PKV_STEP_MAX_BATCH, 1, true>& lds = wlds.b;

    const int tid = threadIdx.x;
    const int blk = blockIdx.x;
    const bool index_wave = is_index_wave();
    constexpr bool big = kBig;                   // sort by every wavefront
    uint32_t flags = 0;

    // Which group and which part of it this workgroup serves (uniform).
    int gi = -1;
    bool page = false;
    int local = 0;
    for (int i = 0; i < a.num_groups; ++i) {
        const StepGroup& g = a.g[i];
        const int rel = blk - g.first_block;
        if (rel >= 0 && rel < g.tile_blocks) {
            gi = i;
            local = rel;
        } else if (rel >= g.tile_blocks && rel < g.tile_blocks + g.page_blocks) {
            gi = i;
            page = true;
            local = rel - g.tile_blocks;
        }
    }

    if (gi >= 0 && !page) {
        // Persistent: this workgroup walks tiles local, local + G, ... of its
        // group (G = tile_blocks), so at any moment the workgroups work on
        // neighbouring tiles.  The index wavefront orders the batch once, then
        // computes tile i+1's slots while the copy wavefronts write tile i and
        // fetch tile i+1; the slot buffer is double-buffered across barriers.
        // Barriers per role: [block_sort's when big], then one per tile.
        const StepGroup& g = a.g[gi];
        const int64_t G = g.tile_blocks;
        auto tile_len = [&](int64_t t) {
            const int64_t t0 = t * g.tile_tokens;
            return (int)(a.T - t0 < g.tile_tokens ? a.T - t0 : g.tile_tokens);
        };
        if (!index_wave) {
            u32x4 kv[kStepUnroll];
            u32x4 vv[kStepUnroll];
            int64_t tile = local;
            load_round<kPow2Row>(g, tile * g.tile_tokens, tile_len(tile), 0, kv, vv);
            if (big)
                block_sort<kStepThreads>(wlds, a.n);    // LDS only: the payload stays in flight
            __syncthreads();                             // tile's slots are ready
            int buf = 0;
            for (; tile < g.tiles; tile += G) {
                const int64_t next = tile + G;
                const int32_t* slots = s_slot + buf * kStepMaxTile;
                const int len = tile_len(tile);
                store_round<kPow2Row>(g, slots, len, 0, kv, vv, flags);
                for (int r = 1; r < g.rounds; ++r) {
                    load_round<kPow2Row>(g, tile * g.tile_tokens, len, r, kv, vv);
                    store_round<kPow2Row>(g, slots, len, r, kv, vv, flags);
                }
                if (next < g.tiles)
                    load_round<kPow2Row>(g, next * g.tile_tokens, tile_len(next), 0, kv, vv);
                __syncthreads();
                buf ^= 1;
            }
        } else {
            WaveGather<PKV_STEP_MAX_BATCH> gth;
            wave_gather(wlds, gth, a.n, a.sched_rows, a.num_scheduled, a.completed, a.R, flags);
            if (big)
                block_sort<kStepThreads>(wlds, a.n);
            else
                rank_sort_wave(wlds, a.n);
            wave_finish(wlds, gth, a.n, a.T, a.R, blk == 0, a.index_mapping, a.query_start_loc,
                        a.seq_lens, flags);
            if (blk != 0)
                flags &= ~(uint32_t)PKV_ST_BAD_COUNT;   // per-request flags: workgroup 0 only
            wave_sync();
            int64_t tile = local;
            tile_tokens(a, g, gi == 0, lds, tile * g.tile_tokens, tile_len(tile), s_slot, flags);
            __syncthreads();                             // tile's slots are ready
            int buf = 0;
            for (; tile < g.tiles; tile += G) {
                const int64_t next = tile + G;
                if (next < g.tiles)
                    tile_tokens(a, g, gi == 0, lds, next * g.tile_tokens, tile_len(next),
                                s_slot + (buf ^ 1) * kStepMaxTile, flags);
                __syncthreads();
                buf ^= 1;
            }
        }
    } else {
        // Page workgroups, and the lone workgroup of a step with nothing else.
        // Barriers per role: [block_sort's when big], then one.
        if (!index_wave) {
            if (big)
                block_sort<kStepThreads>(wlds, a.n);
            __syncthreads();
            if (gi >= 0)
                copy_pages(a, a.g[gi], lds, local * kPageRows + tid / kWave, flags);
        } else {
            WaveGather<PKV_STEP_MAX_BATCH> gth;
            wave_gather(wlds, gth, a.n, a.sched_rows, a.num_scheduled, a.completed, a.R, flags);
            if (big)
                block_sort<kStepThreads>(wlds, a.n);
            else
                rank_sort_wave(wlds, a.n);
            wave_finish(wlds, gth, a.n, a.T, a.R, blk == 0, a.index_mapping, a.query_start_loc,
                        a.seq_lens, flags);
            if (blk != 0)
                flags &= ~(uint32_t)PKV_ST_BAD_COUNT;
            __syncthreads();
        }
    }
    report_status(a.status, flags);
}

}  // namespace

hipError_t launch_step(int32_t n, int32_t T, const int32_t* sched_rows,
                       const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                       const int32_t* token_ids, int64_t token_stride, int32_t L,
                       int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                       int32_t* positions, int32_t* input_ids, int32_t num_groups,
                       const pkv_group* groups, uint32_t* status, hipStream_t stream)
{
    StepArgs a = {};
    a.sched_rows = sched_rows;
    a.num_scheduled = num_scheduled;
    a.completed = completed;
    a.token_ids = token_ids;
    a.index_mapping = index_mapping;
    a.query_start_loc = query_start_loc;
    a.seq_lens = seq_lens;
    a.positions = positions;
    a.input_ids = input_ids;
    a.status = status;
    a.token_stride = token_stride;
    a.n = n;
    a.T = T;
    a.R = R;
    a.L = L;
    a.num_groups = num_groups;
    int64_t blocks = 0;
    for (int i = 0; i < num_groups; ++i) {
        const pkv_group& in = groups[i];
        StepGroup& g = a.g[i];
        g.block_table = in.block_table;
        g.slot_mapping = in.slot_mapping;
        g.input_block_tables = in.input_block_tables;
        g.k = static_cast<const u32x4*>(in.k);
        g.v = static_cast<const u32x4*>(in.v);
        g.k_cache = static_cast<u32x4*>(in.k_cache);
        g.v_cache = static_cast<u32x4*>(in.v_cache);
        g.k_stride16 = in.k_stride / 16;
        g.v_stride16 = in.v_stride / 16;
        g.num_slots = in.num_slots;
        g.MB = in.MB;
        g.block_size = in.block_size;
        g.bs_shift = (in.block_size & (in.block_size - 1)) == 0 ? __builtin_ctz(in.block_size) : -1;
        g.num_blocks = in.num_blocks;
        g.window = in.sliding_window;
        const int64_t cpr = in.row_bytes / 16;
        g.chunks_per_row = (int32_t)cpr;
        g.row_shift = (cpr & (cpr - 1)) == 0 ? __builtin_ctzll((unsigned long long)cpr) : -1;
        const int64_t tile = step_tile_tokens(cpr);
        g.tile_tokens = (int32_t)tile;
        g.rounds = (int32_t)((tile * cpr + kStepChunks - 1) / kStepChunks);
        g.first_block = (int32_t)blocks;
        g.tiles = (int32_t)(((int64_t)T + tile - 1) / tile);
        const int64_t wgs = step_tile_workgroups(num_groups);
        g.tile_blocks = (int32_t)(g.tiles < wgs ? g.tiles : wgs);
        g.page_blocks = in.input_block_tables != nullptr ? (n + kPageRows - 1) / kPageRows : 0;
        blocks += (int64_t)g.tile_blocks + g.page_blocks;
    }
    if (blocks == 0)
        blocks = 1;      // still order the batch and write its per-request outputs
    bool pow2 = true;
    for (int i = 0; i < num_groups; ++i)
        pow2 = pow2 && a.g[i].row_shift >= 0;
    const bool big = n > kWave;
    const dim3 grid((unsigned)blocks), block(kStepThreads);
    if (pow2 && !big)
        k_step<true, false><<<grid, block, 0, stream>>>(a);
    else if (pow2)
        k_step<true, true><<<grid, block, 0, stream>>>(a);
    else if (!big)
        k_step<false, false><<<grid, block, 0, stream>>>(a);
    else
        k_step<false, true><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace pkv
