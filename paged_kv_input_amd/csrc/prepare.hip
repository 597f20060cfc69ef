// prepare.hip -- batch assembly and flattening in one launch.
//
// Batch order, prefix sums and seq_lens follow "Batch Construction and Sequence
// Flattening" and "Contiguous Token Sequence Processing" of "Deep Dive into
// vLLM's Scheduling Mechanism: The Complete CPU-to-GPU Mapping Pipeline"
// (kongchang.com/en); seq_lens as in its "Complete Input Preparation for the
// Attention Module".
//
// Design (gfx950): no sort.  A request's batch row is the number of keys
// (count << 32 | biased row, 64 bits) that sort before its own, equal keys
// ordered by schedule index, and its first flat token the sum of their
// counts: n comparisons per request, made by one to sixteen wavefronts and
// added up by a butterfly over the lanes, so a batch's n^2 comparisons spread
// over the chip instead of binding one CU's ALUs to a sort network (measured
// on MI355X against a one-workgroup bitonic sort: 4096 decodes 37.0 -> 8.9 us,
// 512 requests 11.0 -> 6.0 us, a 16-request prefill 7.1 -> 5.3-6.3 us).  Each
// workgroup stages every key in LDS, ranks its own 1 .. 16 requests (fewer
// when their tokens are many), writes their per-request outputs and then
// their flat tokens, which need no search beyond its own requests; when even
// one request has many tokens, several workgroups (the grid's second
// dimension) rank the same requests and split their tokens.  The
// kernel's time is about three memory round trips (schedule, completed
// counts, token table) plus the launch; no grid-wide barrier, second launch
// or device-side counter is needed.
//
// With KV-cache groups attached (pkv_step past its one-launch limits) the same
// pass also writes every group's slots, through the coordinate-conversion
// chain of the article's "Multi-Layer Coordinate Conversion Pipeline" and
// "Address Calculation Example", and each workgroup copies its requests'
// visible pages ("Complete Input Preparation for the Attention Module"), where
// a sliding-window group may hold -1 holes before the window (the blocks
// freed by "allocate_slots()" of the caffein.top scheduler page).
//
// With the K/V write as well (pkv_step's request-ranked plan: batches of at
// least 32 short requests) the launch is the whole step: each workgroup also
// copies its tokens' K and V rows to their slots.  Its tokens go in rounds of
// 1024, one per thread; a round issues the token-table and block-table
// lookups first, then group 0's payload loads (which need only the flat
// tokens), so the lookups come back ahead of the payload and the payload
// arrives while the slots are worked out.  Measured on MI355X: 256 decodes
// 10.1 -> 7.7 us per step against the tile launch of step.hip, 4096 decodes
// 19.7 -> 18.0 us against the batch launch followed by the scatter.
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

constexpr int kPrepThreads = 1024;                          // workgroup size without the K/V write
constexpr int kPrepUnroll = 8;                              // comparisons per lane and step
constexpr int kPrepTok = 4;                                 // tokens per thread and round

template <int J>
__device__ __forceinline__ void xor_add(uint32_t& less, uint64_t& sum)
{
    less += lane_xor<J>(less);
    const uint32_t lo = lane_xor<J>((uint32_t)sum);
    const uint32_t hi = lane_xor<J>((uint32_t)(sum >> 32));
    sum += ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void wave_add(uint32_t& less, uint64_t& sum)
{
    xor_add<1>(less, sum);
    xor_add<2>(less, sum);
    xor_add<4>(less, sum);
    xor_add<8>(less, sum);
    xor_add<16>(less, sum);
    xor_add<32>(less, sum);                  // every lane holds the wavefront's totals
}

// KV-cache groups whose write slots and visible pages k_prepare<K, true>
// produces with the batch (pkv_step past its one-launch limits).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct PrepGroup {
    const int32_t* block_table;
    int32_t* slot_mapping;
    int32_t* input_block_tables;      // or NULL
    int32_t MB;
    int32_t block_size;
    int32_t bs_shift;                 // log2(block_size), or -1
    int32_t num_blocks;
    int32_t window;                   // sliding window, 0 = full attention
    // the K/V write (k_prepare<K, true, true> only)
    int32_t chunks_per_row;           // row_bytes / 16
    int32_t row_shift;                // log2(chunks_per_row), or -1
    const u32x4* k;
    const u32x4* v;
    u32x4* k_cache;
    u32x4* v_cache;
    int64_t k_stride16;
    int64_t v_stride16;
    int64_t num_slots;
};

struct PrepGroups {
    int32_t num_groups;
    PrepGroup g[PKV_STEP_MAX_GROUPS];
};

constexpr int kPagePer = 4;                                 // visible pages per thread and round
struct PageRound {
    int64_t dst[kPagePer];            // input_block_tables index, or -1
    bool maybe_hole[kPagePer];        // before the window: -1 is a hole
    int32_t v[kPagePer];
};

constexpr int kScatThreads = 1024;                          // workgroup size with the K/V write
constexpr int kScatTok = kScatThreads;                      // tokens per round with the K/V write
constexpr int kScatUnroll = 4;                              // 16-byte chunks per thread and round

__device__ inline u32x4 nt_load(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ inline void nt_store(u32x4 x, u32x4* p) { __builtin_nontemporal_store(x, p); }

// One load round of the K/V write: chunk u * kScatThreads + tid of the
// round's chunks [base, base + ...) -- 16-byte chunk c of round token r = idx /
// chunks_per_row, i.e. of list entry f0 + r, whose flat token the list
// offsets s_first / s_start give.  A wavefront whose chunks all lie past the
// round's `chunks` issues no load; single lanes past it load the round's
// first chunk instead (harmless, keeps the loads together).
template <int kKeys>
__device__ inline void scat_load(const PrepGroup& g, const int64_t* s_first,
                                 const int64_t* s_start, int64_t f0, int64_t chunks, int64_t base,
                                 u32x4 (&kv)[kScatUnroll], u32x4 (&vv)[kScatUnroll])
{
    const int64_t wave0 = base + (threadIdx.x & ~(kWave - 1));
#pragma unroll
    for (int u = 0; u < kScatUnroll; ++u) {
        if (wave0 + (int64_t)u * kScatThreads >= chunks)   // uniform per wavefront
            continue;
        const int64_t idx0 = base + (int64_t)u * kScatThreads + threadIdx.x;
        const int64_t idx = idx0 < chunks ? idx0 : 0;
        const int64_t r = g.row_shift >= 0 ? (idx >> g.row_shift) : idx / g.chunks_per_row;
        const int64_t c = idx - r * g.chunks_per_row;
        const int64_t f = f0 + r;
        int w = 0;
#pragma unroll
        for (int step = kKeys / 2; step > 0; step >>= 1)
            if (s_first[w + step] <= f)
                w += step;
        const int64_t t = s_start[w] + (f - s_first[w]);
        kv[u] = nt_load(g.k + t * g.k_stride16 + c);
        vv[u] = nt_load(g.v + t * g.v_stride16 + c);
    }
}

// The matching store round: each chunk to its token's slot (slot < 0: no
// write; slot >= num_slots: SLOT_OOR, no write), as pkv_scatter_kv.
__device__ inline void scat_store(const PrepGroup& g, const int32_t* s_slot, int64_t chunks,
                                  int64_t base, u32x4 (&kv)[kScatUnroll],
                                  u32x4 (&vv)[kScatUnroll], uint32_t& flags)
{
#pragma unroll
    for (int u = 0; u < kScatUnroll; ++u)
        __asm__ volatile("" : "+v"(kv[u]), "+v"(vv[u]));     // the loads stay ahead of the tests
#pragma unroll
    for (int u = 0; u < kScatUnroll; ++u) {
        const int64_t idx = base + (int64_t)u * kScatThreads + threadIdx.x;
        if (idx >= chunks)
            continue;
        const int64_t r = g.row_shift >= 0 ? (idx >> g.row_shift) : idx / g.chunks_per_row;
        const int64_t c = idx - r * g.chunks_per_row;
        const int32_t slot = s_slot[r];
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

template <int kKeys, bool kSlots, bool kScatter>
__global__ __launch_bounds__(kScatter ? kScatThreads : kPrepThreads) void k_prepare(
    int32_t n, int32_t T, const int32_t* __restrict__ sched_rows,
    const int32_t* __restrict__ num_scheduled, const int32_t* __restrict__ completed, int32_t R,
    const int32_t* __restrict__ token_ids, int64_t token_stride, int32_t L,
    int32_t* __restrict__ index_mapping, int32_t* __restrict__ query_start_loc,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ positions,
    int32_t* __restrict__ input_ids, uint32_t* __restrict__ status, const PrepGroups gs)
{
    constexpr int kThr = kScatter ? kScatThreads : kPrepThreads;
    constexpr int kWaves = kThr / kWave;
    constexpr int kLoads = PKV_MAX_BATCH / kThr;           // schedule entries per thread
    static_assert(kKeys <= kWaves, "at least one wavefront per request");
    constexpr int kPerKey = kWaves / kKeys;                // wavefronts per request
    constexpr int kLanes = kPerKey * kWave;                // lanes per request
    __shared__ uint64_t s_key[PKV_MAX_BATCH];
    __shared__ int64_t s_total[kWaves];
    __shared__ uint32_t s_less[kWaves];
    __shared__ uint64_t s_sum[kWaves];
    __shared__ int64_t s_first[kKeys + 1];        // workgroup-local offsets of the token lists
    __shared__ int64_t s_start[kKeys];            // first flat token of each request
    __shared__ int32_t s_row[kKeys];              // its row, or -1 when outside [0, R)
    __shared__ int32_t s_done[kKeys];             // its completed count
    __shared__ int32_t s_b[kKeys];                // its batch row
    __shared__ int32_t s_sl[kKeys];               // its seq_len as written
    __shared__ int32_t s_qcount[kKeys];           // query_start_loc[b + 1] - query_start_loc[b]
    __shared__ int64_t s_pfirst[kKeys + 1];       // offsets of the visible-page lists
    __shared__ int64_t s_pwin[kKeys];             // first page a window may leave as a hole
    __shared__ int32_t s_slot[kScatter ? PKV_STEP_MAX_GROUPS * kScatTok : 1];  // and their slots
    static_assert(!kScatter || kSlots, "the K/V write needs the slots");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    uint32_t flags = 0;

    // The row of this wavefront's own request first (every lane loads the same
    // word), so that its completed count can be fetched as soon as it is in,
    // while the batch is still being staged.
    const int q = wave / kPerKey;                          // request within the workgroup
    const int i = (int)blockIdx.x * kKeys + q;
    const bool have = i < n;                               // uniform per wavefront
    const int32_t own_row = have ? sched_rows[i] : 0;

    // Every key of the batch (a thread's loads all in flight together, from
    // clamped in-bounds addresses) and the sum of every count.
    int32_t rows[kLoads];
    int32_t counts[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int j = u * kThr + tid;
        const bool any = u * kThr < n;                     // uniform: rounds the batch reaches
        rows[u] = any ? sched_rows[j < n ? j : 0] : 0;
        counts[u] = any ? num_scheduled[j < n ? j : 0] : 0;
    }
    const bool mine_ok = have && own_row >= 0 && own_row < R;
    const int32_t mine_done = R > 0 ? completed[mine_ok ? own_row : 0] : 0;
    uint64_t part = 0;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int j = u * kThr + tid;
        if (j < n) {
            int32_t c = counts[u];
            if (c < 0) {
                if (blockIdx.x == 0 && blockIdx.y == 0)
                    flags |= PKV_ST_BAD_COUNT;
                c = 0;
            }
            part += (uint32_t)c;
            s_key[j] = sort_key(c, rows[u]);
        }
    }
    {
        uint32_t unused = 0;
        wave_add(unused, part);
        if (lane == 0)
            s_total[wave] = (int64_t)part;
    }
    __syncthreads();
    int64_t total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        total += s_total[w];

    // The kPerKey wavefronts of request i compare keys l, l + kLanes, ...
    // with its own (l = its lane among them).  Branch-free, all reads of a
    // step first (a short-circuit test would split each comparison into
    // branches with a wait for its LDS read).
    const uint64_t mine = s_key[have ? i : 0];
    uint32_t less = 0;
    uint64_t sum = 0;
    int j = (wave % kPerKey) * kWave + lane;
    for (; j + (kPrepUnroll - 1) * kLanes < n; j += kPrepUnroll * kLanes) {
        uint64_t kj[kPrepUnroll];
#pragma unroll
        for (int u = 0; u < kPrepUnroll; ++u)
            kj[u] = s_key[j + u * kLanes];
#pragma unroll
        for (int u = 0; u < kPrepUnroll; ++u) {
            const bool before = (kj[u] < mine) | ((kj[u] == mine) & (j + u * kLanes < i));
            less += (uint32_t)before;
            sum += before ? (uint64_t)(uint32_t)key_count(kj[u]) : 0ull;
        }
    }
    for (; j < n; j += kLanes) {
        const uint64_t kj = s_key[j];
        const bool before = (kj < mine) | ((kj == mine) & (j < i));
        less += (uint32_t)before;
        sum += before ? (uint64_t)(uint32_t)key_count(kj) : 0ull;
    }
    wave_add(less, sum);
    if (kPerKey > 1) {
        if (lane == 0) {
            s_less[wave] = less;
            s_sum[wave] = sum;
        }
        __syncthreads();
        less = 0;
        sum = 0;
#pragma unroll
        for (int w = 0; w < kPerKey; ++w) {
            less += s_less[q * kPerKey + w];
            sum += s_sum[q * kPerKey + w];
        }
    }

    if (lane == 0 && wave % kPerKey == 0) {
        const int b = (int)less;
        const int32_t c = key_count(mine);
        const int32_t row = key_row(mine);
        const bool row_ok = row >= 0 && row < R;
        const int64_t start = (int64_t)sum;
        const int32_t done = mine_ok ? mine_done : 0;
        const int64_t end = start + c;
        const int32_t q_end = end > INT32_MAX ? INT32_MAX : (int32_t)end;
        const int32_t q_start = start > INT32_MAX ? INT32_MAX : (int32_t)start;
        const int32_t sl = row_ok ? (int32_t)(uint32_t)(uint64_t)((int64_t)done + c) : -1;
        if (have && blockIdx.y == 0) {                  // one split writes them
            index_mapping[b] = row;
            query_start_loc[b + 1] = q_end;
            seq_lens[b] = sl;
            if (!row_ok)
                flags |= PKV_ST_BAD_ROW;
        }
        s_b[q] = b;
        s_sl[q] = sl;
        s_qcount[q] = q_end - q_start;
        // tokens of this request below T (those at T and beyond are dropped)
        const int64_t room = (int64_t)T - start;
        const int64_t own = !have ? 0 : (c < room ? c : (room > 0 ? room : 0));
        s_start[q] = start;
        s_row[q] = have && row_ok ? row : -1;
        s_done[q] = done;
        s_first[q + 1] = own;
        if constexpr (kScatter) {
            // group 0's visible pages of the request, as page_lists lays them out
            const PrepGroup& g = gs.g[0];
            int64_t visible = 0;
            int64_t firstp = 0;
            if (g.input_block_tables != nullptr && have && row_ok) {
                visible = sl <= 0 ? 0 : ((int64_t)sl + g.block_size - 1) / g.block_size;
                if (visible > g.MB) {
                    flags |= PKV_ST_LB_OOR;
                    visible = g.MB;
                }
                firstp = window_first(sl, q_end - q_start, g.window) / g.block_size;
            }
            s_pfirst[q + 1] = visible;
            s_pwin[q] = firstp;
        }
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
        query_start_loc[0] = 0;
        if (total != (int64_t)T)
            flags |= PKV_ST_TOKEN_SUM;
    }
    __syncthreads();
    if (tid == 0) {
        int64_t run = 0;
        s_first[0] = 0;
        for (int w = 0; w < kKeys; ++w) {
            run += s_first[w + 1];
            s_first[w + 1] = run;
        }
        if constexpr (kScatter) {
            run = 0;
            s_pfirst[0] = 0;
            for (int w = 0; w < kKeys; ++w) {
                run += s_pfirst[w + 1];
                s_pfirst[w + 1] = run;
            }
        }
    }
    __syncthreads();

    // The workgroup's token lists, concatenated, kPrepTok tokens per thread
    // and round: resolve each token's request, then issue all token-table
    // loads of the round together.
    // This split's slice [f_lo, f_hi) of the concatenated lists.
    const int64_t F = s_first[kKeys];
    const int64_t per = gridDim.y == 1 ? F : (F + gridDim.y - 1) / gridDim.y;   // uniform
    const int64_t f_lo = (int64_t)blockIdx.y * per;
    const int64_t f_hi = f_lo + per < F ? f_lo + per : F;
    const bool want_ids = input_ids != nullptr;
    const bool have_ids = want_ids && R > 0 && L > 0;

    // Visible pages (kSlots): page_lists lays out a group's lists (this
    // workgroup's requests, their first ceil(seq_len / block_size) entries)
    // in s_pfirst / s_pwin and gives this split's slice; page_load /
    // page_store move one round of kPagePer entries per thread.
    auto page_lists = [&](const PrepGroup& g, int64_t& p_lo, int64_t& p_hi) {
        if (tid < kKeys) {
            const int qq = tid;
            int64_t visible = 0;
            int64_t first = 0;
            if (s_row[qq] >= 0) {
                const int32_t sl = s_sl[qq];
                visible = sl <= 0 ? 0 : ((int64_t)sl + g.block_size - 1) / g.block_size;
                if (visible > g.MB) {
                    flags |= PKV_ST_LB_OOR;
                    visible = g.MB;
                }
                // pages before the window may be -1 holes (freed blocks)
                first = window_first(sl, s_qcount[qq], g.window) / g.block_size;
            }
            s_pfirst[qq + 1] = visible;
            s_pwin[qq] = first;
        }
        __syncthreads();
        if (tid == 0) {
            int64_t run = 0;
            s_pfirst[0] = 0;
            for (int w = 0; w < kKeys; ++w) {
                run += s_pfirst[w + 1];
                s_pfirst[w + 1] = run;
            }
        }
        __syncthreads();
        const int64_t P = s_pfirst[kKeys];
        const int64_t pper = gridDim.y == 1 ? P : (P + gridDim.y - 1) / gridDim.y;
        p_lo = (int64_t)blockIdx.y * pper;
        p_hi = p_lo + pper < P ? p_lo + pper : P;
    };
    auto page_load = [&](const PrepGroup& g, int64_t f0, int64_t p_hi, PageRound& pr) {
        int64_t psrc[kPagePer];
#pragma unroll
        for (int u = 0; u < kPagePer; ++u) {
            const int64_t f = f0 + (int64_t)u * kThr + tid;
            psrc[u] = -1;
            pr.dst[u] = -1;
            pr.maybe_hole[u] = false;
            if (f >= p_hi)
                continue;
            int w = 0;
#pragma unroll
            for (int step = kKeys / 2; step > 0; step >>= 1)
                if (s_pfirst[w + step] <= f)
                    w += step;
            const int64_t i = f - s_pfirst[w];
            psrc[u] = (int64_t)s_row[w] * g.MB + i;
            pr.dst[u] = (int64_t)s_b[w] * g.MB + i;
            pr.maybe_hole[u] = i < s_pwin[w];
        }
#pragma unroll
        for (int u = 0; u < kPagePer; ++u)    // f0 < p_hi: a visible page exists, so a table
            pr.v[u] = g.block_table[psrc[u] >= 0 ? psrc[u] : 0];
    };
    auto page_store = [&](const PrepGroup& g, PageRound& pr) {
#pragma unroll
        for (int u = 0; u < kPagePer; ++u) {
            if (pr.dst[u] < 0)
                continue;
            const bool hole = pr.maybe_hole[u] && pr.v[u] == -1;
            if ((pr.v[u] < 0 || pr.v[u] >= g.num_blocks) && !hole)
                flags |= PKV_ST_BLOCK_OOR;
            g.input_block_tables[pr.dst[u]] = pr.v[u];
        }
    };
    // With the K/V write, group 0's first round of pages is loaded together
    // with the first tokens' lookups (one round trip for both).
    PageRound pr0;
#pragma unroll
    for (int u = 0; u < kPagePer; ++u) {
        pr0.dst[u] = -1;                                    // nothing to store
        pr0.maybe_hole[u] = false;
        pr0.v[u] = -1;
    }
    int64_t p0_lo = 0, p0_hi = 0;
    if constexpr (kScatter) {
        // the lists were laid out with the requests' outputs; no splits
        const PrepGroup& g = gs.g[0];
        p0_hi = s_pfirst[kKeys];
        if (g.input_block_tables != nullptr && p0_lo < p0_hi)   // uniform; no pages: no table read
            page_load(g, p0_lo, p0_hi, pr0);
    }

    if constexpr (!kScatter) {
        constexpr int kTok = kPrepTok;                         // tokens per thread and round
        for (int64_t f0 = f_lo; f0 < f_hi; f0 += (int64_t)kTok * kThr) {
            int64_t t_of[kTok];
            int32_t pos_out[kTok];
            int64_t src[kTok];
            int w_of[kTok];                                     // request within the workgroup
    #pragma unroll
            for (int u = 0; u < kTok; ++u) {
                const int64_t f = f0 + (int64_t)u * kThr + tid;
                t_of[u] = -1;
                pos_out[u] = -1;
                src[u] = -1;
                w_of[u] = 0;
                if (f >= f_hi)
                    continue;
                int w = 0;                                      // last list starting at or before f
    #pragma unroll
                for (int step = kKeys / 2; step > 0; step >>= 1)
                    if (s_first[w + step] <= f)
                        w += step;
                w_of[u] = w;
                const int64_t jj = f - s_first[w];
                t_of[u] = s_start[w] + jj;
                const int32_t row = s_row[w];
                if (row < 0)
                    continue;                                   // flagged above: position -1
                const int64_t p = (int64_t)s_done[w] + jj;
                pos_out[u] = (int32_t)(uint32_t)(uint64_t)p;
                if (p < 0 || (want_ids && p >= L))
                    flags |= PKV_ST_POS_OOR;
                else if (want_ids)
                    src[u] = (int64_t)row * token_stride + p;
            }
            int32_t id_out[kTok];
    #pragma unroll
            for (int u = 0; u < kTok; ++u) {
                id_out[u] = have_ids ? token_ids[src[u] >= 0 ? src[u] : 0] : -1;
                if (src[u] < 0)
                    id_out[u] = -1;
            }
            if constexpr (kSlots) {
                // Each group's slots: position -> (logical block, offset) ->
                // physical block through the row's block table; a lane's lookups
                // of a group are in flight together.
                for (int gi = 0; gi < gs.num_groups; ++gi) {
                    const PrepGroup& g = gs.g[gi];
                    int64_t bsrc[kTok];
                    int32_t boff[kTok];
    #pragma unroll
                    for (int u = 0; u < kTok; ++u) {
                        bsrc[u] = -1;
                        boff[u] = 0;
                        if (t_of[u] < 0 || s_row[w_of[u]] < 0)
                            continue;                           // no request, or a bad row
                        const int32_t p = pos_out[u];
                        if (p < 0) {
                            flags |= PKV_ST_POS_OOR;
                            continue;
                        }
                        const int32_t lb = g.bs_shift >= 0 ? (p >> g.bs_shift) : p / g.block_size;
                        boff[u] = p - lb * g.block_size;
                        if (lb >= g.MB)
                            flags |= PKV_ST_LB_OOR;
                        else
                            bsrc[u] = (int64_t)s_row[w_of[u]] * g.MB + lb;
                    }
                    const bool have_bt = R > 0 && g.MB > 0;     // uniform
                    int32_t blk[kTok];
    #pragma unroll
                    for (int u = 0; u < kTok; ++u) {
                        blk[u] = have_bt ? g.block_table[bsrc[u] >= 0 ? bsrc[u] : 0] : -1;
                        if (bsrc[u] < 0)
                            blk[u] = -1;
                    }
    #pragma unroll
                    for (int u = 0; u < kTok; ++u) {
                        if (t_of[u] < 0)
                            continue;
                        int32_t slot = -1;
                        if (bsrc[u] >= 0) {
                            if (blk[u] < 0 || blk[u] >= g.num_blocks)
                                flags |= PKV_ST_BLOCK_OOR;
                            else
                                slot = blk[u] * g.block_size + boff[u];
                        }
                        g.slot_mapping[t_of[u]] = slot;
                    }
                }
            }
    #pragma unroll
            for (int u = 0; u < kTok; ++u) {
                if (t_of[u] >= 0) {
                    positions[t_of[u]] = pos_out[u];
                    if (want_ids)
                        input_ids[t_of[u]] = id_out[u];
                }
            }
        }
    }
    if constexpr (kScatter) {
        // Rounds of kScatTok tokens, one per thread: the round's flat tokens
        // go to LDS; the token-table and block-table loads are issued first,
        // then group 0's payload loads (they need only the flat tokens), so
        // the lookups come back ahead of the payload; then positions, ids and
        // slots; then, after one barrier, the K and V rows to their slots.
        for (int64_t f0 = f_lo; f0 < f_hi; f0 += kScatTok) {
            const int ntok = (int)(f_hi - f0 < kScatTok ? f_hi - f0 : kScatTok);   // uniform
            const int64_t f = f0 + tid;
            const bool valid = tid < ntok;
            int w = 0;                                      // last list starting at or before f
#pragma unroll
            for (int step = kKeys / 2; step > 0; step >>= 1)
                if (s_first[w + step] <= f)
                    w += step;
            const int64_t jj = f - s_first[w];
            const int64_t t = s_start[w] + jj;
            const int32_t row = valid ? s_row[w] : -1;
            int32_t pos = -1;
            int64_t src = -1;
            if (row >= 0) {
                const int64_t p = (int64_t)s_done[w] + jj;
                pos = (int32_t)(uint32_t)(uint64_t)p;
                if (p < 0 || (want_ids && p >= L))
                    flags |= PKV_ST_POS_OOR;
                else if (want_ids)
                    src = (int64_t)row * token_stride + p;
            }
            int64_t bsrc[PKV_STEP_MAX_GROUPS];
            int32_t boff[PKV_STEP_MAX_GROUPS];
#pragma unroll
            for (int gi = 0; gi < PKV_STEP_MAX_GROUPS; ++gi) {
                bsrc[gi] = -1;
                boff[gi] = 0;
                if (gi >= gs.num_groups || row < 0)
                    continue;
                const PrepGroup& g = gs.g[gi];
                if (pos < 0) {
                    flags |= PKV_ST_POS_OOR;
                    continue;
                }
                const int32_t lb = g.bs_shift >= 0 ? (pos >> g.bs_shift) : pos / g.block_size;
                boff[gi] = pos - lb * g.block_size;
                if (lb >= g.MB)
                    flags |= PKV_ST_LB_OOR;
                else
                    bsrc[gi] = (int64_t)row * g.MB + lb;
            }
            // every lookup of the round in flight together (clamped in-bounds
            // addresses where none is needed)
            const int32_t id = have_ids ? token_ids[src >= 0 ? src : 0] : -1;
            int32_t blk[PKV_STEP_MAX_GROUPS];
#pragma unroll
            for (int gi = 0; gi < PKV_STEP_MAX_GROUPS; ++gi) {
                const PrepGroup& g = gs.g[gi < gs.num_groups ? gi : 0];
                const bool have_bt = gi < gs.num_groups && R > 0 && g.MB > 0;   // uniform
                blk[gi] = have_bt ? g.block_table[bsrc[gi] >= 0 ? bsrc[gi] : 0] : -1;
            }
            u32x4 kv[kScatUnroll];
            u32x4 vv[kScatUnroll];
            const int64_t chunks0 = (int64_t)ntok * gs.g[0].chunks_per_row;
            scat_load<kKeys>(gs.g[0], s_first, s_start, f0, chunks0, 0, kv, vv);
            if (valid) {
                positions[t] = pos;
                if (want_ids)
                    input_ids[t] = src >= 0 ? id : -1;
            }
#pragma unroll
            for (int gi = 0; gi < PKV_STEP_MAX_GROUPS; ++gi) {
                if (gi >= gs.num_groups)
                    break;
                const PrepGroup& g = gs.g[gi];
                int32_t slot = -1;
                if (bsrc[gi] >= 0) {
                    if (blk[gi] < 0 || blk[gi] >= g.num_blocks)
                        flags |= PKV_ST_BLOCK_OOR;
                    else
                        slot = blk[gi] * g.block_size + boff[gi];
                }
                if (valid) {
                    g.slot_mapping[t] = slot;
                    s_slot[gi * kScatTok + tid] = slot;
                }
            }
            __syncthreads();                                // the round's slots are in LDS
            for (int gi = 0; gi < gs.num_groups; ++gi) {
                const PrepGroup& g = gs.g[gi];
                const int64_t chunks = (int64_t)ntok * g.chunks_per_row;
                for (int64_t base = 0; base < chunks; base += kScatUnroll * kThr) {
                    if (gi > 0 || base > 0)
                        scat_load<kKeys>(g, s_first, s_start, f0, chunks, base, kv, vv);
                    scat_store(g, s_slot + gi * kScatTok, chunks, base, kv, vv, flags);
                }
            }
            __syncthreads();                                // before the next round's tokens
        }
    }
    if constexpr (kSlots) {
        if constexpr (kScatter) {
            // group 0's pages: the first round was loaded with the tokens
            const PrepGroup& g = gs.g[0];
            if (g.input_block_tables != nullptr) {
                page_store(g, pr0);
                for (int64_t f0 = p0_lo + (int64_t)kPagePer * kThr; f0 < p0_hi;
                     f0 += (int64_t)kPagePer * kThr) {
                    PageRound pr;
                    page_load(g, f0, p0_hi, pr);
                    page_store(g, pr);
                }
                __syncthreads();                            // the lists are rebuilt per group
            }
        }
        // Each group's visible pages of this workgroup's requests: the first
        // ceil(seq_len / block_size) block-table entries, copied as one list
        // over the workgroup, kPagePer entries per thread and round.
        for (int gi = kScatter ? 1 : 0; gi < gs.num_groups; ++gi) {
            const PrepGroup& g = gs.g[gi];
            if (g.input_block_tables == nullptr)
                continue;                                   // uniform
            int64_t p_lo, p_hi;
            page_lists(g, p_lo, p_hi);
            for (int64_t f0 = p_lo; f0 < p_hi; f0 += (int64_t)kPagePer * kThr) {
                PageRound pr;
                page_load(g, f0, p_hi, pr);
                page_store(g, pr);
            }
            __syncthreads();                                // the lists are rebuilt per group
        }
    }

    // Tokens past the counts' sum belong to no request (TOKEN_SUM).
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t t = total + wg * kThr + tid; t < T;
         t += (int64_t)gridDim.x * gridDim.y * kThr) {
        positions[t] = -1;
        if (want_ids)
            input_ids[t] = -1;
        if constexpr (kSlots) {
            for (int gi = 0; gi < gs.num_groups; ++gi)
                gs.g[gi].slot_mapping[t] = -1;
        }
    }
    report_status(status, flags);
}

// Requests per workgroup of k_prepare: about 2048 tokens per workgroup
// on average (one round of its token loop), at most 256 workgroups (each
// stages all n keys), at most 16.
__host__ inline int prep_keys(int32_t n, int32_t T)
{
    const int64_t by_tokens = T > 0 ? (int64_t)n * 2048 / T : 16;
    const int64_t by_grid = ((int64_t)n + 255) / 256;
    int k = 1;
    while (k < 16 && (k * 2 <= by_tokens || k < by_grid))
        k *= 2;
    return k;
}

// Splits of each workgroup's token and page lists (the grid's second
// dimension): about 8192 tokens per workgroup on average, so that a few long
// requests still spread over the chip; every split ranks its requests again
// (cheap: splits > 1 only when n is small next to T).
__host__ inline int prep_splits(int32_t n, int32_t T, int keys)
{
    const int64_t per_wg = n > 0 ? (int64_t)T * keys / n : (int64_t)T;
    int64_t s = (per_wg + 8191) / 8192;
    if (s < 1)
        s = 1;
    if (s > 1024)
        s = 1024;
    return (int)s;
}

// With the K/V write: at most 16 requests per workgroup, as few as leave
// 256 workgroups (one request each when n <= 256), so that the payload
// spreads over the chip; no splits (the plan takes it for decode-like
// batches, a few tokens per request).
__host__ inline int scat_keys(int32_t n)
{
    int k = 1;
    while (k < 16 && (int64_t)n > 256 * (int64_t)k)
        k *= 2;
    return k;
}

}  // namespace

hipError_t launch_prepare(int32_t n, int32_t T, const int32_t* sched_rows,
                          const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                          const int32_t* token_ids, int64_t token_stride, int32_t L,
                          int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                          int32_t* positions, int32_t* input_ids, int32_t num_groups,
                          const pkv_group* groups, bool with_scatter, uint32_t* status,
                          hipStream_t stream)
{
    PrepGroups gs = {};
    gs.num_groups = num_groups;
    for (int i = 0; i < num_groups; ++i) {
        const pkv_group& in = groups[i];
        PrepGroup& g = gs.g[i];
        g.block_table = in.block_table;
        g.slot_mapping = in.slot_mapping;
        g.input_block_tables = in.input_block_tables;
        g.MB = in.MB;
        g.block_size = in.block_size;
        g.bs_shift = (in.block_size & (in.block_size - 1)) == 0 ? __builtin_ctz(in.block_size) : -1;
        g.num_blocks = in.num_blocks;
        g.window = in.sliding_window;
        const int64_t cpr = in.row_bytes / 16;
        g.chunks_per_row = (int32_t)cpr;
        g.row_shift = (cpr & (cpr - 1)) == 0 ? __builtin_ctzll((unsigned long long)cpr) : -1;
        g.k = static_cast<const u32x4*>(in.k);
        g.v = static_cast<const u32x4*>(in.v);
        g.k_cache = static_cast<u32x4*>(in.k_cache);
        g.v_cache = static_cast<u32x4*>(in.v_cache);
        g.k_stride16 = in.k_stride / 16;
        g.v_stride16 = in.v_stride / 16;
        g.num_slots = in.num_slots;
    }
    const bool scatter = with_scatter && num_groups > 0;
    const int keys = scatter ? scat_keys(n) : prep_keys(n, T);
    const int64_t blocks = n > 0 ? ((int64_t)n + keys - 1) / keys : 1;
    const int splits = scatter ? 1 : prep_splits(n, T, keys);
    const dim3 grid((unsigned)blocks, (unsigned)splits);
    const dim3 block(scatter ? kScatThreads : kPrepThreads);
#define PKV_PREP_LAUNCH(K, S, W)                                                                  \
    k_prepare<K, S, W><<<grid, block, 0, stream>>>(n, T, sched_rows, num_scheduled, completed,   \
                                                   R, token_ids, token_stride, L, index_mapping,  \
                                                   query_start_loc, seq_lens, positions,          \
                                                   input_ids, status, gs)
#define PKV_PREP_KEYS(S, W)                                                                       \
    switch (keys) {                                                                               \
    case 1: PKV_PREP_LAUNCH(1, S, W); break;                                                      \
    case 2: PKV_PREP_LAUNCH(2, S, W); break;                                                      \
    case 4: PKV_PREP_LAUNCH(4, S, W); break;                                                      \
    case 8: PKV_PREP_LAUNCH(8, S, W); break;                                                      \
    default: PKV_PREP_LAUNCH(16, S, W); break;                                                    \
    }
    if (scatter) {
        PKV_PREP_KEYS(true, true)
    } else if (num_groups > 0) {
        PKV_PREP_KEYS(true, false)
    } else {
        PKV_PREP_KEYS(false, false)
    }
#undef PKV_PREP_KEYS
#undef PKV_PREP_LAUNCH
    return hipGetLastError();
}

}  // namespace pkv
