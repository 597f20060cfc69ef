// A C-ABI caller with no Python and no torch: the worked example of "Deep Dive
// into vLLM's Scheduling Mechanism: The Complete CPU-to-GPU Mapping Pipeline"
// (kongchang.com/en) run through pkv_step with device buffers from the HIP
// runtime, checked against the values the article prints ("Contiguous Token
// Sequence Processing": query_start_loc [0, 1, 9], positions 31 and 16..23;
// "Address Calculation Example": request B's token lands in slot 207) and
// against the definitions for the rest (request A's slots 704..711 from its
// block 44, the visible pages, input ids, the K/V rows at their slots).
// Request A: state row 6, 16 tokens computed, 8 new; request B: row 7, 31
// computed, 1 new; block size 16; block tables [81, 44] and [37, 12].
// Exit status 0 when every check passes.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pagedkv.h"

#define HIP_OK(x)                                                                 \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));          \
            return 2;                                                             \
        }                                                                         \
    } while (0)

static int failures = 0;

static void expect(const char* what, const int32_t* got, const int32_t* want, int count)
{
    for (int i = 0; i < count; ++i)
        if (got[i] != want[i]) {
            std::fprintf(stderr, "%s[%d] = %d, expected %d\n", what, i, got[i], want[i]);
            ++failures;
            return;
        }
}

int main()
{
    const int32_t R = 8, L = 32, n = 2, T = 9, bs = 16, MB = 2, NB = 128;
    const int32_t H = 8, D = 128;
    const int64_t row_bytes = (int64_t)H * D * 2, num_slots = (int64_t)NB * bs;
    const int32_t row_words = H * D;

    // schedule order: A, then B
    const int32_t sched_rows[n] = {6, 7}, num_scheduled[n] = {8, 1};
    std::vector<int32_t> completed(R, 0), token_ids((size_t)R * L), block_table((size_t)R * MB, -1);
    completed[6] = 16;
    completed[7] = 31;
    for (int r = 0; r < R; ++r)
        for (int p = 0; p < L; ++p)
            token_ids[(size_t)r * L + p] = 1000 * r + p;
    block_table[6 * MB + 0] = 81;
    block_table[6 * MB + 1] = 44;
    block_table[7 * MB + 0] = 37;
    block_table[7 * MB + 1] = 12;
    std::vector<uint16_t> k((size_t)T * row_words), v(k.size());
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < row_words; ++j) {
            k[(size_t)t * row_words + j] = (uint16_t)(t * 997 + j);
            v[(size_t)t * row_words + j] = (uint16_t)(40000 + t * 991 + j);
        }

    int32_t *d_rows, *d_counts, *d_completed, *d_tokens, *d_bt, *d_im, *d_qsl, *d_sl, *d_pos,
        *d_ids, *d_slots, *d_ibt;
    uint32_t* d_status;
    void *d_k, *d_v, *d_kc, *d_vc;
    HIP_OK(hipMalloc((void**)&d_rows, n * 4));
    HIP_OK(hipMalloc((void**)&d_counts, n * 4));
    HIP_OK(hipMalloc((void**)&d_completed, R * 4));
    HIP_OK(hipMalloc((void**)&d_tokens, (size_t)R * L * 4));
    HIP_OK(hipMalloc((void**)&d_bt, (size_t)R * MB * 4));
    HIP_OK(hipMalloc((void**)&d_im, n * 4));
    HIP_OK(hipMalloc((void**)&d_qsl, (n + 1) * 4));
    HIP_OK(hipMalloc((void**)&d_sl, n * 4));
    HIP_OK(hipMalloc((void**)&d_pos, T * 4));
    HIP_OK(hipMalloc((void**)&d_ids, T * 4));
    HIP_OK(hipMalloc((void**)&d_slots, T * 4));
    HIP_OK(hipMalloc((void**)&d_ibt, n * MB * 4));
    HIP_OK(hipMalloc((void**)&d_status, 4));
    HIP_OK(hipMalloc(&d_k, (size_t)T * row_bytes));
    HIP_OK(hipMalloc(&d_v, (size_t)T * row_bytes));
    HIP_OK(hipMalloc(&d_kc, (size_t)num_slots * row_bytes));
    HIP_OK(hipMalloc(&d_vc, (size_t)num_slots * row_bytes));
    HIP_OK(hipMemcpy(d_rows, sched_rows, n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_counts, num_scheduled, n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_completed, completed.data(), R * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_tokens, token_ids.data(), token_ids.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_bt, block_table.data(), block_table.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_k, k.data(), k.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, v.data(), v.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_kc, 0xFF, (size_t)num_slots * row_bytes));      // sentinel rows
    HIP_OK(hipMemset(d_vc, 0xFF, (size_t)num_slots * row_bytes));
    HIP_OK(hipMemset(d_ibt, 0xFF, n * MB * 4));
    HIP_OK(hipMemset(d_status, 0, 4));

    pkv_group g;
    std::memset(&g, 0, sizeof g);
    g.block_table = d_bt;
    g.slot_mapping = d_slots;
    g.input_block_tables = d_ibt;
    g.k = d_k;
    g.v = d_v;
    g.k_cache = d_kc;
    g.v_cache = d_vc;
    g.k_stride = row_bytes;
    g.v_stride = row_bytes;
    g.num_slots = num_slots;
    g.row_bytes = row_bytes;
    g.MB = MB;
    g.block_size = bs;
    g.num_blocks = NB;
    g.sliding_window = 0;
    const int rc = pkv_step(n, T, d_rows, d_counts, d_completed, R, d_tokens, L, L, d_im, d_qsl,
                            d_sl, d_pos, d_ids, 1, &g, d_status, nullptr);
    if (rc != PKV_OK) {
        std::fprintf(stderr, "pkv_step: %s\n", pkv_error_string(rc));
        return 2;
    }
    HIP_OK(hipDeviceSynchronize());

    int32_t im[n], qsl[n + 1], sl[n], pos[T], ids[T], slots[T], ibt[n * MB];
    uint32_t status = 0;
    HIP_OK(hipMemcpy(im, d_im, sizeof im, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(qsl, d_qsl, sizeof qsl, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sl, d_sl, sizeof sl, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(pos, d_pos, sizeof pos, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ids, d_ids, sizeof ids, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(slots, d_slots, sizeof slots, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ibt, d_ibt, sizeof ibt, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));

    // B (one token) before A (eight): batch rows 0 and 1
    const int32_t want_im[n] = {7, 6}, want_qsl[n + 1] = {0, 1, 9}, want_sl[n] = {32, 24};
    const int32_t want_pos[T] = {31, 16, 17, 18, 19, 20, 21, 22, 23};
    const int32_t want_slots[T] = {207, 704, 705, 706, 707, 708, 709, 710, 711};
    const int32_t want_ibt[n * MB] = {37, 12, 81, 44};
    int32_t want_ids[T];
    for (int t = 0; t < T; ++t)
        want_ids[t] = 1000 * want_im[t == 0 ? 0 : 1] + want_pos[t];
    expect("index_mapping", im, want_im, n);
    expect("query_start_loc", qsl, want_qsl, n + 1);
    expect("seq_lens", sl, want_sl, n);
    expect("positions", pos, want_pos, T);
    expect("input_ids", ids, want_ids, T);
    expect("slot_mapping", slots, want_slots, T);
    expect("input_block_tables", ibt, want_ibt, n * MB);
    if (status != 0) {
        std::fprintf(stderr, "status bits %#x\n", status);
        ++failures;
    }

    // Each token's K and V rows at its slot; every other cache row untouched.
    std::vector<uint16_t> kc((size_t)num_slots * row_words), vc(kc.size());
    HIP_OK(hipMemcpy(kc.data(), d_kc, kc.size() * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(vc.data(), d_vc, vc.size() * 2, hipMemcpyDeviceToHost));
    int64_t written = 0;
    for (int64_t s = 0; s < num_slots; ++s) {
        int t = -1;
        for (int u = 0; u < T; ++u)
            if (want_slots[u] == s)
                t = u;
        bool touched = false;
        for (int j = 0; j < row_words; ++j) {
            const uint16_t gk = kc[(size_t)s * row_words + j], gv = vc[(size_t)s * row_words + j];
            const uint16_t ek = t >= 0 ? k[(size_t)t * row_words + j] : 0xFFFF;
            const uint16_t ev = t >= 0 ? v[(size_t)t * row_words + j] : 0xFFFF;
            touched = touched || gk != 0xFFFF || gv != 0xFFFF;
            if (gk != ek || gv != ev) {
                std::fprintf(stderr, "cache slot %lld word %d: K %u V %u, expected %u %u\n",
                             (long long)s, j, gk, gv, ek, ev);
                ++failures;
                break;
            }
        }
        written += touched ? 1 : 0;
    }
    if (written != T) {
        std::fprintf(stderr, "%lld cache rows written, expected %d\n", (long long)written, T);
        ++failures;
    }

    void* const allocations[] = {d_rows, d_counts, d_completed, d_tokens, d_bt, d_im, d_qsl,
                                 d_sl, d_pos, d_ids, d_slots, d_ibt, d_status, d_k, d_v,
                                 d_kc, d_vc};
    for (void* ptr : allocations)
        HIP_OK(hipFree(ptr));
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("pages example through the C ABI: bit-exact (abi %d)\n", pkv_abi_version());
    return 0;
}
