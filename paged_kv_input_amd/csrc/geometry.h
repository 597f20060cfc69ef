// geometry.h -- launch geometry of libpagedkv's fused step, in plain C++ (no
// HIP types), so that the host code choosing between pkv_step's launch plans
// and the kernel that runs the one-launch plan share one definition.  Not part
// of the public ABI.
#pragma once

#include <stdint.h>

#include <initializer_list>

#include "pagedkv.h"

#ifndef PKV_STEP_COPY_WAVES
#define PKV_STEP_COPY_WAVES 3
#endif
#ifndef PKV_STEP_UNROLL
#define PKV_STEP_UNROLL 6
#endif
#ifndef PKV_STEP_TILE_WGS
#define PKV_STEP_TILE_WGS 1536             // persistent tile workgroups per step, over all groups
#endif

namespace pkv {

constexpr int kWave = 64;                  // gfx950 wavefront width

// The fused step's workgroup: PKV_STEP_COPY_WAVES copy wavefronts plus one
// index wavefront.  One round of the copy wavefronts moves kStepChunks 16-byte
// chunks of K and as many of V.
constexpr int kStepCopyThreads = PKV_STEP_COPY_WAVES * kWave;
constexpr int kStepThreads = kStepCopyThreads + kWave;
constexpr int kStepUnroll = PKV_STEP_UNROLL;
constexpr int kStepChunks = kStepCopyThreads * kStepUnroll;
constexpr int kStepMaxTile = 256;                       // tokens per tile, at most
constexpr int kStepPageRows = kStepCopyThreads / kWave; // batch rows per page workgroup

// Tokens per tile: as many whole rows as one round of the copy wavefronts
// moves, rounded down to a power of two, so that tiles never straddle a block
// of a power-of-two block size (each tile writes one contiguous run of slots;
// measured on MI355X: 8 instead of 9 rows of 2 KiB, 52.9 vs 53.9 us at the
// 32k-token prefill), and at most kStepMaxTile.
inline int64_t step_tile_tokens(int64_t chunks_per_row)
{
    int64_t tile = 1;
    while (tile < kStepMaxTile && tile * 2 * chunks_per_row <= kStepChunks)
        tile *= 2;
    return tile;
}

// Persistent tile workgroups of each group: PKV_STEP_TILE_WGS per step, split
// evenly over the groups (measured on MI355X: best for a 16-request prefill;
// for 512 requests in two groups 768 per group beat 512 and 1024; fewer were
// slower for 72 requests).
inline int64_t step_tile_workgroups(int32_t num_groups)
{
    const int64_t per = PKV_STEP_TILE_WGS / (num_groups > 0 ? num_groups : 1);
    return per > 0 ? per : 1;
}

// Workgroups of the one-launch grid: each group's tile workgroups (no more
// than its tiles) and, when it writes visible pages, one page workgroup per
// kStepPageRows batch rows; at least one.
inline int64_t step_grid_blocks(int32_t n, int32_t T, int32_t num_groups, const pkv_group* groups)
{
    int64_t blocks = 0;
    for (int i = 0; i < num_groups; ++i) {
        const int64_t tile = step_tile_tokens(groups[i].row_bytes / 16);
        const int64_t tiles = ((int64_t)T + tile - 1) / tile;
        const int64_t wgs = step_tile_workgroups(num_groups);
        blocks += tiles < wgs ? tiles : wgs;
        if (groups[i].input_block_tables != nullptr)
            blocks += ((int64_t)n + kStepPageRows - 1) / kStepPageRows;
    }
    return blocks > 0 ? blocks : 1;
}

// The one-launch kernel addresses a tile's K and V rows from the tile's first
// row by 32-bit chunk offsets: (tile_tokens - 1) * stride / 16 + row_bytes / 16
// must not exceed 2^32 for either payload.
inline bool step_offsets_fit(const pkv_group& g)
{
    const int64_t cpr = g.row_bytes / 16;
    const int64_t span = step_tile_tokens(cpr) - 1;
    const int64_t lim = (int64_t)1 << 32;
    for (const int64_t stride : {g.k_stride, g.v_stride}) {
        const int64_t s16 = stride / 16;
        if (s16 < 0)
            return false;
        if (span > 0 && s16 > (lim - cpr) / span)
            return false;
        if (span * s16 + cpr > lim)
            return false;
    }
    return true;
}

}  // namespace pkv
