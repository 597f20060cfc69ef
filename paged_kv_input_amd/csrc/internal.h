// internal.h -- device helpers shared by the HIP kernels of libpagedkv
// (gfx950, wave64).  Not part of the public ABI; the host-side launchers are
// declared in launchers.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.h"
#include "pagedkv.h"

namespace pkv {

// One DPP move of a 64-bit value (its two 32-bit halves from the same source
// lane); lanes without a source, or in rows outside kRowMask, get 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp64(uint64_t x)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, kCtrl,
                                                              kRowMask, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), kCtrl,
                                                              kRowMask, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ inline int64_t wave_inclusive_scan(int64_t x)
{
    // Hillis-Steele steps inside each 16-lane row by row shifts of 1, 2, 4 and
    // 8 lanes, then the row totals carried on by row broadcasts: lane 15 into
    // rows 1 and 3, then lane 31 into rows 2 and 3.  All in registers.
    uint64_t v = (uint64_t)x;
    v += dpp64<0x111, 0xF>(v);      // row_shr:1
    v += dpp64<0x112, 0xF>(v);      // row_shr:2
    v += dpp64<0x114, 0xF>(v);      // row_shr:4
    v += dpp64<0x118, 0xF>(v);      // row_shr:8
    v += dpp64<0x142, 0xA>(v);      // row_bcast:15
    v += dpp64<0x143, 0xC>(v);      // row_bcast:31
    return (int64_t)v;
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

// Sliding-window groups: the first position any new token of a request
// attends, when the token at position p attends p-W+1 .. p and the request
// has `count` new tokens ending at seq_len (0 for W == 0: full attention).
__device__ inline int64_t window_first(int64_t seq_len, int64_t count, int32_t window)
{
    if (window <= 0)
        return 0;
    const int64_t first = seq_len - (count > 0 ? count : 0) - window + 1;
    return first > 0 ? first : 0;
}

// Ascending order of (count, row) as unsigned 64-bit keys: the count (>= 0) in
// the high word, the row with its sign bit flipped in the low word so that
// signed row order equals unsigned key order.
__device__ inline uint64_t sort_key(int32_t count, int32_t row)
{
    return ((uint64_t)(uint32_t)count << 32) | (uint32_t)(row ^ INT32_MIN);
}
__device__ inline int32_t key_count(uint64_t key) { return (int32_t)(key >> 32); }
__device__ inline int32_t key_row(uint64_t key) { return (int32_t)((uint32_t)key ^ 0x80000000u); }

__device__ inline int pad_pow2(int n)
{
    int n_pad = 1;
    while (n_pad < n)
        n_pad <<= 1;
    return n_pad;
}

// Value of the same register in lane (lane ^ J) of the wavefront.  Distances
// 1, 2, 4 and 8 stay inside a 16-lane row and use DPP moves (quad
// permutations, the half-row mirror, the row rotation by 8); 16 uses an LDS
// swizzle in bit mode and 32 a backward permute (neither touches LDS memory).
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v)
{
    const int x = (int)v;
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
    } else if constexpr (J == 4) {
        // mirror in the 8-lane half row (i -> 7 - i), then reverse each quad
        // (i -> 3 - i): together i -> i ^ 4
        const int m = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
        return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row rotate by 8
    } else if constexpr (J == 16) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x1F | (16 << 10));   // and 31, xor 16
    } else {
        static_assert(J == 32, "lane distances 1 .. 32");
        const int lane = (int)(threadIdx.x & (kWave - 1));
        return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, x);
    }
}

// Elements of the register bitonic sort: kPer per lane (element s of lane l in
// wavefront w has sort index w * 64 * kPer + s * 64 + l), each a 64-bit key
// and the key's original index.
template <int kPer>
struct SortRegs {
    uint64_t key[kPer];
    int32_t idx[kPer];
};

// Compare-exchange of element s with the partner's (okey, oidx): the lower
// position of an ascending pair keeps the smaller key, and so on.  Strict
// comparisons on both sides, so equal keys never move and the indices stay a
// permutation.
template <int kPer>
__device__ __forceinline__ void keep(SortRegs<kPer>& r, int s, uint64_t okey, int32_t oidx,
                                     bool lower, bool ascending)
{
    const bool take = lower == ascending ? okey < r.key[s] : r.key[s] < okey;
    r.key[s] = take ? okey : r.key[s];
    r.idx[s] = take ? oidx : r.idx[s];
}

template <int J, int kPer>
__device__ __forceinline__ void lane_pass(SortRegs<kPer>& r, int base, int k)
{
    const int lane = (int)(threadIdx.x & (kWave - 1));
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
        const uint32_t lo = lane_xor<J>((uint32_t)r.key[s]);
        const uint32_t hi = lane_xor<J>((uint32_t)(r.key[s] >> 32));
        const int32_t oidx = (int32_t)lane_xor<J>((uint32_t)r.idx[s]);
        const int i = base + s * kWave + lane;
        keep(r, s, ((uint64_t)hi << 32) | lo, oidx, (lane & J) == 0, (i & k) == 0);
    }
}

// Compare-exchange of slots s and s ^ D of each lane (elements 64 * D apart).
template <int D, int kPer>
__device__ __forceinline__ void slot_pass(SortRegs<kPer>& r, int base, int k)
{
    const int lane = (int)(threadIdx.x & (kWave - 1));
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
        const int o = s ^ D;
        if (o > s && o < kPer) {
            const int i = base + s * kWave + lane;
            const bool ascending = (i & k) == 0;
            const bool swap = ascending ? r.key[o] < r.key[s] : r.key[s] < r.key[o];
            const uint64_t tk = r.key[s];
            r.key[s] = swap ? r.key[o] : r.key[s];
            r.key[o] = swap ? tk : r.key[o];
            const int32_t ti = r.idx[s];
            r.idx[s] = swap ? r.idx[o] : r.idx[s];
            r.idx[o] = swap ? ti : r.idx[o];
        }
    }
}

// Ascending bitonic sort of key[0 .. n) with idx[0 .. n), the keys' original
// indices, by every wavefront of a kThreads-thread workgroup; call
// from every thread with the same n <= kPad.  The network spans kPad (a power
// of two, at most kThreads * kPer) positions, padded with ~0 keys, and is
// unrolled whole.  The elements stay in registers: pairs closer than 64 are
// exchanged between lanes, pairs 64 .. 64 * (kPer - 1) apart are swapped
// inside a lane, and only pairs in different wavefronts go through LDS.
// Wavefronts holding only padding skip the work but keep the barriers.  The
// LDS exchanges alternate between two buffers (key / idx and xkey / xidx), so
// each costs one barrier.  LDS traffic only, so the wavefronts' outstanding
// loads stay in flight.  key / idx hold the result on return, after a barrier.
template <int kThreads, int kPer, int kPad>
__device__ __forceinline__ void bitonic_regs(uint64_t* key, int16_t* idx, uint64_t* xkey,
                                             int16_t* xidx, int32_t n)
{
    constexpr int kSpan = kWave * kPer;                  // elements per wavefront
    static_assert(kPad >= 2 && (kPad & (kPad - 1)) == 0 && kPad <= kThreads * kPer,
                  "the network spans a power of two of the workgroup's elements");
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int base = (int)(threadIdx.x / kWave) * kSpan;
    const bool active = base < kPad;                      // uniform per wavefront
    SortRegs<kPer> r;
    __syncthreads();                                      // the keys are in LDS
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
        const int i = base + s * kWave + lane;
        r.key[s] = i < n ? key[i] : ~0ull;                // padding sorts last
        r.idx[s] = i < n ? idx[i] : i;
    }
    int pass = 0;                                         // LDS exchanges so far
#pragma unroll
    for (int k = 2; k <= kPad; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j >= kWave; j >>= 1) {
            if (j >= kSpan) {
                // partner in another wavefront
                const bool second = (pass & 1) == 0;
                uint64_t* bk = second ? xkey : key;
                int16_t* bi = second ? xidx : idx;
                if (active) {
#pragma unroll
                    for (int s = 0; s < kPer; ++s) {
                        const int i = base + s * kWave + lane;
                        bk[i] = r.key[s];
                        bi[i] = (int16_t)r.idx[s];
                    }
                }
                __syncthreads();
                if (active) {
#pragma unroll
                    for (int s = 0; s < kPer; ++s) {
                        const int i = base + s * kWave + lane;
                        const int32_t oidx = bi[i ^ j];
                        keep(r, s, bk[i ^ j], oidx, (i & j) == 0, (i & k) == 0);
                    }
                }
                ++pass;
            } else if (active) {
                // partner in the same lane: slot s ^ (j / 64)
                if (j == kWave)
                    slot_pass<1>(r, base, k);
                else
                    slot_pass<2>(r, base, k);
            }
        }
        if (active) {
            if (k > 32) lane_pass<32>(r, base, k);
            if (k > 16) lane_pass<16>(r, base, k);
            if (k > 8) lane_pass<8>(r, base, k);
            if (k > 4) lane_pass<4>(r, base, k);
            if (k > 2) lane_pass<2>(r, base, k);
            lane_pass<1>(r, base, k);
        }
    }
    // key / idx were read by the initial loads or by an exchange: wait for every
    // wavefront before overwriting them, unless the last exchange used the
    // second buffer (every read of key / idx then came before its barrier).
    if ((pass & 1) == 0)
        __syncthreads();
    if (active) {
#pragma unroll
        for (int s = 0; s < kPer; ++s) {
            const int i = base + s * kWave + lane;
            if (i < n) {
                key[i] = r.key[s];
                idx[i] = (int16_t)r.idx[s];
            }
        }
    }
    __syncthreads();
}

// LDS working set of the batch ordering for up to kMaxN requests.  The keys
// are dead once ordered, so the per-request rows and completed counts reuse
// them.
template <int kMaxN, int kWaves, bool kCounts = false>
struct BatchLds {
    uint64_t key[kMaxN];
    int32_t qsl[kMaxN + 1];
    int32_t count[kCounts ? kMaxN : 1];     // clamped counts in batch order (kCounts only)
    int64_t wave_total[kWaves];
    __device__ int32_t* row() { return reinterpret_cast<int32_t*>(key); }
    __device__ int32_t* done() { return reinterpret_cast<int32_t*>(key) + kMaxN; }
    __device__ const int32_t* row() const { return reinterpret_cast<const int32_t*>(key); }
    __device__ const int32_t* done() const { return reinterpret_cast<const int32_t*>(key) + kMaxN; }
};

// Orders LDS accesses between the lanes of one wavefront (no s_barrier: the
// other wavefronts of the workgroup are not involved).
__device__ inline void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Batch assembly ("Batch Construction and Sequence Flattening" of the
// kongchang.com article) inside a workgroup whose global loads are all made
// by ONE wavefront (the "index" wavefront), so that the workgroup's other
// wavefronts can keep their own memory traffic in flight meanwhile (a
// wavefront's loads complete in issue order): the n scheduled requests as
// (count, row) keys in ascending order, the prefix sums of their counts
// (saturating at INT32_MAX) and their completed counts; the same results and
// flags as pkv_prepare_batch.  Three phases:
//   wave_gather  (index wavefront) loads rows and counts, then at once each
//                row's completed count, and writes the keys and their original
//                indices to LDS; the completed counts stay in registers;
//   sort         the keys put in order with their original indices: by the
//                index wavefront alone for n <= 64 (rank_sort_wave: each key
//                ranked by counting the keys before it, one LDS broadcast per
//                key, no barrier), else by every wavefront of the workgroup
//                (block_sort, a bitonic sort in registers with cross-lane
//                moves and three LDS exchanges; no memory traffic, so the
//                other wavefronts' loads stay in flight);
//   wave_finish  (index wavefront) prefix sums, rows, completed counts and the
//                per-request outputs.
// The fetch of the completed counts thus overlaps the sort instead of adding a
// dependent round trip after it.
template <int kMaxN>
struct WaveBatchLds {
    BatchLds<kMaxN, 1, true> b;
    int16_t idx[kMaxN];          // original index of each key during the sort
    int32_t done_by_i[kMaxN];    // completed count by original index
    uint64_t xkey[kMaxN];        // block_sort's second exchange buffer
    int16_t xidx[kMaxN];
};

template <int kMaxN>
struct WaveGather {
    static constexpr int kPer = kMaxN / kWave;
    int32_t done_i[kPer];        // completed count of request e * 64 + lane
};

template <int kMaxN>
__device__ inline void wave_gather(WaveBatchLds<kMaxN>& w, WaveGather<kMaxN>& gth, int32_t n,
                                   const int32_t* __restrict__ sched_rows,
                                   const int32_t* __restrict__ num_scheduled,
                                   const int32_t* __restrict__ completed, int32_t R,
                                   uint32_t& flags)
{
    constexpr int kPer = WaveGather<kMaxN>::kPer;
    static_assert(kMaxN % kWave == 0, "batch rows split evenly over lanes");
    static_assert(kMaxN <= 32768, "original indices are kept in 16 bits");
    const int lane = threadIdx.x & (kWave - 1);
    const int n_pad = pad_pow2(n);
    // Unconditional loads from a clamped in-bounds address where the value is
    // not needed, so each group of them is issued back to back (a load under a
    // divergent branch is issued only after a full wait).
    int32_t row_i[kPer];
    int32_t cnt_i[kPer];
    const int nparts = (n + kWave - 1) / kWave;          // uniform
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int i = e * kWave + lane;
        const int ic = i < n ? i : n - 1;
        row_i[e] = e < nparts ? sched_rows[ic] : 0;
        cnt_i[e] = e < nparts ? num_scheduled[ic] : 0;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int i = e * kWave + lane;
        const bool ok = i < n && row_i[e] >= 0 && row_i[e] < R;
        gth.done_i[e] = (e < nparts && R > 0) ? completed[ok ? row_i[e] : 0] : 0;
        if (!ok)
            gth.done_i[e] = 0;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int i = e * kWave + lane;
        if (i >= n_pad)
            break;
        uint64_t key = ~0ull;                       // padding sorts last
        if (i < n) {
            int32_t c = cnt_i[e];
            if (c < 0) {
                flags |= PKV_ST_BAD_COUNT;
                c = 0;
            }
            key = sort_key(c, row_i[e]);
        }
        w.b.key[i] = key;
        w.idx[i] = (int16_t)i;
    }
}

// Bitonic sort of 64 < n <= kThreads * 2 keys with their original indices by
// every wavefront of the workgroup (call from every thread): one element per
// lane up to kThreads keys (a network of kThreads / 2 positions when that
// holds them: 28 passes instead of 36), else two.  w.xkey / w.xidx serve as
// the second exchange buffer.
template <int kThreads, int kMaxN>
__device__ __forceinline__ void block_sort(WaveBatchLds<kMaxN>& w, int32_t n)
{
    if (n <= kThreads / 2)
        bitonic_regs<kThreads, 1, kThreads / 2>(w.b.key, w.idx, w.xkey, w.xidx, n);
    else if (n <= kThreads)
        bitonic_regs<kThreads, 1, kThreads>(w.b.key, w.idx, w.xkey, w.xidx, n);
    else
        bitonic_regs<kThreads, 2, 2 * kThreads>(w.b.key, w.idx, w.xkey, w.xidx, n);
}

// Stable rank of each lane's key among run[0 .. len) (an LDS array holding
// lane j's key at j; len <= 64): the number of keys that are smaller, plus the
// equal ones held by lower lanes.  Every lane reads the same element at a
// time (an LDS broadcast), eight reads in flight per batch.
__device__ inline int wave_rank(const uint64_t* run, uint64_t key, int len)
{
    const int lane = threadIdx.x & (kWave - 1);
    int rank = 0;
    for (int j0 = 0; j0 < len; j0 += 8) {            // uniform
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = run[j0 + u < len ? j0 + u : len - 1];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            rank += (j < len && (v[u] < key || (v[u] == key && j < lane))) ? 1 : 0;
        }
    }
    return rank;
}

// Batch order for n <= 64, by the index wavefront alone: each lane ranks its
// key with wave_rank and stores key and original index at that rank.  Same
// order as a stable sort of the keys (equal keys keep their schedule order).
template <int kMaxN>
__device__ inline void rank_sort_wave(WaveBatchLds<kMaxN>& w, int32_t n)
{
    const int lane = threadIdx.x & (kWave - 1);
    wave_sync();                                      // wave_gather's keys are in LDS
    const uint64_t key = lane < n ? w.b.key[lane] : ~0ull;
    const int rank = wave_rank(w.b.key, key, n);
    wave_sync();                                      // every key is read before any is moved
    if (lane < n) {
        w.b.key[rank] = key;
        w.idx[rank] = (int16_t)lane;
    }
    wave_sync();
}

template <int kMaxN>
__device__ inline void wave_finish(WaveBatchLds<kMaxN>& w, const WaveGather<kMaxN>& gth,
                                   int32_t n, int32_t T, int32_t R, bool writer,
                                   int32_t* __restrict__ index_mapping,
                                   int32_t* __restrict__ query_start_loc,
                                   int32_t* __restrict__ seq_lens, uint32_t& flags)
{
    constexpr int kPer = WaveGather<kMaxN>::kPer;
    BatchLds<kMaxN, 1, true>& lds = w.b;
    const int lane = threadIdx.x & (kWave - 1);
    // The completed counts have had the whole sort to arrive.
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int i = e * kWave + lane;
        if (i < n)
            w.done_by_i[i] = gth.done_i[e];
    }
    uint64_t keys[kPer];
    int64_t local = 0;
    const int first = lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int b = first + e;
        keys[e] = b < n ? lds.key[b] : 0ull;
        local += b < n ? key_count(keys[e]) : 0;
    }
    const int64_t incl = wave_inclusive_scan(local);
    const uint32_t total_lo = __shfl((uint32_t)(uint64_t)incl, kWave - 1, kWave);
    const uint32_t total_hi = __shfl((uint32_t)((uint64_t)incl >> 32), kWave - 1, kWave);
    const int64_t total = (int64_t)(((uint64_t)total_hi << 32) | total_lo);
    int64_t run = incl - local;
    wave_sync();          // done_by_i is written; every key is in registers
    int32_t done_v[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int b = first + e;
        done_v[e] = b < n ? w.done_by_i[w.idx[b]] : 0;
    }
    wave_sync();          // lds.key is dead: row() / done() may overwrite it
    int32_t* s_row = lds.row();
    int32_t* s_done = lds.done();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int b = first + e;
        if (b >= n)
            break;
        const int32_t c = key_count(keys[e]);
        const int32_t row = key_row(keys[e]);
        run += c;
        const int32_t end = run > INT32_MAX ? INT32_MAX : (int32_t)run;
        const bool row_ok = row >= 0 && row < R;
        lds.qsl[b + 1] = end;
        s_row[b] = row;
        s_done[b] = row_ok ? done_v[e] : 0;
        lds.count[b] = c;
        if (writer) {
            index_mapping[b] = row;
            query_start_loc[b + 1] = end;
            if (row_ok) {
                seq_lens[b] = (int32_t)(uint32_t)(uint64_t)((int64_t)done_v[e] + c);
            } else {
                seq_lens[b] = -1;
                flags |= PKV_ST_BAD_ROW;
            }
        }
    }
    if (lane == 0) {
        lds.qsl[0] = 0;
        if (writer) {
            query_start_loc[0] = 0;
            if (total != (int64_t)T)
                flags |= PKV_ST_TOKEN_SUM;
        }
    }
}

}  // namespace pkv
