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
#include "internal.h"
#include "launchers.h"

namespace pkv {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / kWave;
constexpr int kPrepLoads = PKV_MAX_BATCH / kPrepThreads;    // schedule entries per thread
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
struct PrepGroup {
    const int32_t* block_table;
    int32_t* slot_mapping;
    int32_t* input_block_tables;      // or NULL
    int32_t MB;
    int32_t block_size;
    int32_t bs_shift;                 // log2(block_size), or -1
    int32_t num_blocks;
    int32_t window;                   // sliding window, 0 = full attention
};

struct PrepGroups {
    int32_t num_groups;
    PrepGroup g[PKV_STEP_MAX_GROUPS];
};

constexpr int kPagePer = 4;                                 // visible pages per thread and round

// A batch of 0 <= n <= PKV_MAX_BATCH requests (n = 0: one workgroup, for
// query_start_loc[0] and the tokens); workgroup w serves the kKeys
// requests kKeys*w .. kKeys*w + kKeys - 1 in schedule order (w = blockIdx.x),
// with 16 / kKeys wavefronts each, and slice blockIdx.y of gridDim.y of their
// token and page lists.  A request's batch row b is the number of keys that sort
// before its own and its first flat token the sum of their counts; the
// workgroup then writes its requests' per-request outputs and flat tokens
// (every token below T that belongs to one of them), and its share of the
// tokens past the counts' sum.  With kSlots it also writes, for every group
// in gs, those tokens' slots and those requests' visible pages, with the
// results and flags of pkv_compute_slot_mapping.
template <int kKeys, bool kSlots>
__global__ __launch_bounds__(kPrepThreads) void k_prepare(
    int32_t n, int32_t T, const int32_t* __restrict__ sched_rows,
    const int32_t* __restrict__ num_scheduled, const int32_t* __restrict__ completed, int32_t R,
    const int32_t* __restrict__ token_ids, int64_t token_stride, int32_t L,
    int32_t* __restrict__ index_mapping, int32_t* __restrict__ query_start_loc,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ positions,
    int32_t* __restrict__ input_ids, uint32_t* __restrict__ status, const PrepGroups gs)
{
    constexpr int kPerKey = kPrepWaves / kKeys;            // wavefronts per request
    constexpr int kLanes = kPerKey * kWave;                // lanes per request
    __shared__ uint64_t s_key[PKV_MAX_BATCH];
    __shared__ int64_t s_total[kPrepWaves];
    __shared__ uint32_t s_less[kPrepWaves];
    __shared__ uint64_t s_sum[kPrepWaves];
    __shared__ int64_t s_first[kKeys + 1];        // workgroup-local offsets of the token lists
    __shared__ int64_t s_start[kKeys];            // first flat token of each request
    __shared__ int32_t s_row[kKeys];              // its row, or -1 when outside [0, R)
    __shared__ int32_t s_done[kKeys];             // its completed count
    __shared__ int32_t s_b[kKeys];                // its batch row
    __shared__ int32_t s_sl[kKeys];               // its seq_len as written
    __shared__ int32_t s_qcount[kKeys];           // query_start_loc[b + 1] - query_start_loc[b]
    __shared__ int64_t s_pfirst[kKeys + 1];       // offsets of the visible-page lists
    __shared__ int64_t s_pwin[kKeys];             // first page a window may leave as a hole
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    uint32_t flags = 0;

    // Every key of the batch (a thread's loads all in flight together, from
    // clamped in-bounds addresses) and the sum of every count.
    int32_t rows[kPrepLoads];
    int32_t counts[kPrepLoads];
#pragma unroll
    for (int u = 0; u < kPrepLoads; ++u) {
        const int i = u * kPrepThreads + tid;
        rows[u] = n > 0 ? sched_rows[i < n ? i : 0] : 0;
        counts[u] = n > 0 ? num_scheduled[i < n ? i : 0] : 0;
    }
    uint64_t part = 0;
#pragma unroll
    for (int u = 0; u < kPrepLoads; ++u) {
        const int i = u * kPrepThreads + tid;
        if (i < n) {
            int32_t c = counts[u];
            if (c < 0) {
                if (blockIdx.x == 0 && blockIdx.y == 0)
                    flags |= PKV_ST_BAD_COUNT;
                c = 0;
            }
            part += (uint32_t)c;
            s_key[i] = sort_key(c, rows[u]);
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
    for (int w = 0; w < kPrepWaves; ++w)
        total += s_total[w];

    // The kPerKey wavefronts of request i compare keys l, l + kLanes, ...
    // with its own (l = its lane among them).  Branch-free, all reads of a
    // step first (a short-circuit test would split each comparison into
    // branches with a wait for its LDS read).
    const int q = wave / kPerKey;                          // request within the workgroup
    const int i = (int)blockIdx.x * kKeys + q;
    const bool have = i < n;                               // uniform per wavefront
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
        const int32_t done = have && row_ok ? completed[row] : 0;
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
    for (int64_t f0 = f_lo; f0 < f_hi; f0 += (int64_t)kPrepTok * kPrepThreads) {
        int64_t t_of[kPrepTok];
        int32_t pos_out[kPrepTok];
        int64_t src[kPrepTok];
        int w_of[kPrepTok];                                 // request within the workgroup
#pragma unroll
        for (int u = 0; u < kPrepTok; ++u) {
            const int64_t f = f0 + (int64_t)u * kPrepThreads + tid;
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
        int32_t id_out[kPrepTok];
#pragma unroll
        for (int u = 0; u < kPrepTok; ++u) {
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
                int64_t bsrc[kPrepTok];
                int32_t boff[kPrepTok];
#pragma unroll
                for (int u = 0; u < kPrepTok; ++u) {
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
                int32_t blk[kPrepTok];
#pragma unroll
                for (int u = 0; u < kPrepTok; ++u) {
                    blk[u] = have_bt ? g.block_table[bsrc[u] >= 0 ? bsrc[u] : 0] : -1;
                    if (bsrc[u] < 0)
                        blk[u] = -1;
                }
#pragma unroll
                for (int u = 0; u < kPrepTok; ++u) {
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
        for (int u = 0; u < kPrepTok; ++u) {
            if (t_of[u] >= 0) {
                positions[t_of[u]] = pos_out[u];
                if (want_ids)
                    input_ids[t_of[u]] = id_out[u];
            }
        }
    }

    if constexpr (kSlots) {
        // Each group's visible pages of this workgroup's requests: the first
        // ceil(seq_len / block_size) block-table entries, copied as one list
        // over the workgroup, kPagePer entries per thread and round.
        for (int gi = 0; gi < gs.num_groups; ++gi) {
            const PrepGroup& g = gs.g[gi];
            if (g.input_block_tables == nullptr)
                continue;                                   // uniform
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
            const int64_t p_lo = (int64_t)blockIdx.y * pper;
            const int64_t p_hi = p_lo + pper < P ? p_lo + pper : P;
            for (int64_t f0 = p_lo; f0 < p_hi; f0 += (int64_t)kPagePer * kPrepThreads) {
                int64_t psrc[kPagePer];
                int64_t pdst[kPagePer];
                bool maybe_hole[kPagePer];
#pragma unroll
                for (int u = 0; u < kPagePer; ++u) {
                    const int64_t f = f0 + (int64_t)u * kPrepThreads + tid;
                    psrc[u] = -1;
                    pdst[u] = -1;
                    maybe_hole[u] = false;
                    if (f >= p_hi)
                        continue;
                    int w = 0;
#pragma unroll
                    for (int step = kKeys / 2; step > 0; step >>= 1)
                        if (s_pfirst[w + step] <= f)
                            w += step;
                    const int64_t i = f - s_pfirst[w];
                    psrc[u] = (int64_t)s_row[w] * g.MB + i;
                    pdst[u] = (int64_t)s_b[w] * g.MB + i;
                    maybe_hole[u] = i < s_pwin[w];
                }
                int32_t v[kPagePer];
#pragma unroll
                for (int u = 0; u < kPagePer; ++u)
                    v[u] = g.block_table[psrc[u] >= 0 ? psrc[u] : 0];   // P > 0: a table exists
#pragma unroll
                for (int u = 0; u < kPagePer; ++u) {
                    if (pdst[u] < 0)
                        continue;
                    const bool hole = maybe_hole[u] && v[u] == -1;
                    if ((v[u] < 0 || v[u] >= g.num_blocks) && !hole)
                        flags |= PKV_ST_BLOCK_OOR;
                    g.input_block_tables[pdst[u]] = v[u];
                }
            }
            __syncthreads();                                // the lists are rebuilt per group
        }
    }

    // Tokens past the counts' sum belong to no request (TOKEN_SUM).
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t t = total + wg * kPrepThreads + tid; t < T;
         t += (int64_t)gridDim.x * gridDim.y * kPrepThreads) {
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

}  // namespace

hipError_t launch_prepare(int32_t n, int32_t T, const int32_t* sched_rows,
                          const int32_t* num_scheduled, const int32_t* completed, int32_t R,
                          const int32_t* token_ids, int64_t token_stride, int32_t L,
                          int32_t* index_mapping, int32_t* query_start_loc, int32_t* seq_lens,
                          int32_t* positions, int32_t* input_ids, int32_t num_groups,
                          const pkv_group* groups, uint32_t* status, hipStream_t stream)
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
    }
    const int keys = prep_keys(n, T);
    const int64_t blocks = n > 0 ? ((int64_t)n + keys - 1) / keys : 1;
    const dim3 grid((unsigned)blocks, (unsigned)prep_splits(n, T, keys)), block(kPrepThreads);
#define PKV_PREP_LAUNCH(K, S)                                                                     \
    k_prepare<K, S><<<grid, block, 0, stream>>>(n, T, sched_rows, num_scheduled, completed, R,   \
                                                token_ids, token_stride, L, index_mapping,        \
                                                query_start_loc, seq_lens, positions, input_ids,  \
                                                status, gs)
#define PKV_PREP_KEYS(S)                                                                          \
    switch (keys) {                                                                               \
    case 1: PKV_PREP_LAUNCH(1, S); break;                                                         \
    case 2: PKV_PREP_LAUNCH(2, S); break;                                                         \
    case 4: PKV_PREP_LAUNCH(4, S); break;                                                         \
    case 8: PKV_PREP_LAUNCH(8, S); break;                                                         \
    default: PKV_PREP_LAUNCH(16, S); break;                                                       \
    }
    if (num_groups > 0) {
        PKV_PREP_KEYS(true)
    } else {
        PKV_PREP_KEYS(false)
    }
#undef PKV_PREP_KEYS
#undef PKV_PREP_LAUNCH
    return hipGetLastError();
}

}  // namespace pkv
