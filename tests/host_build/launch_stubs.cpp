// launch_stubs.cpp -- test infrastructure: stand-ins for every launcher of
// launchers.h, so that the library's host code (the C entry points with their
// argument checks and launch plans, and the row pool) builds and runs with
// g++ alone, on a machine without a GPU, e.g. under the address and
// undefined-behaviour sanitizers.  A stub enqueues nothing: it appends the
// launcher's name (and, for the batch launch, how many groups ride along) to
// a log that the tests read through pkv_stub_log(), and reports success.
#include <string>

#include "launchers.h"

namespace {
std::string g_log;
hipError_t logged(const char* name)
{
    g_log += name;
    g_log += ';';
    return hipSuccess;
}
}  // namespace

extern "C" {
const char* pkv_stub_log(void) { return g_log.c_str(); }
void pkv_stub_log_clear(void) { g_log.clear(); }
}

namespace pkv {

hipError_t launch_prepare(int32_t, int32_t, const int32_t*, const int32_t*, const int32_t*,
                          int32_t, const int32_t*, int64_t, int32_t, int32_t*, int32_t*, int32_t*,
                          int32_t*, int32_t*, int32_t num_groups, const pkv_group*,
                          bool with_scatter, uint32_t*, hipStream_t)
{
    return logged(("prepare+" + std::to_string(num_groups) + (with_scatter ? "+kv" : "")).c_str());
}

hipError_t launch_slots(int32_t, int32_t, const int32_t*, const int32_t*, const int32_t*,
                        const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                        int32_t, int32_t*, int32_t*, uint32_t*, hipStream_t)
{
    return logged("slots");
}

hipError_t launch_step(int32_t, int32_t, const int32_t*, const int32_t*, const int32_t*, int32_t,
                       const int32_t*, int64_t, int32_t, int32_t*, int32_t*, int32_t*, int32_t*,
                       int32_t*, int32_t, const pkv_group*, uint32_t*, hipStream_t)
{
    return logged("step");
}

hipError_t launch_gather(int32_t, const int32_t*, const int32_t*, int32_t, const int32_t*,
                         int32_t, int32_t, int32_t, int64_t, const void*, const void*, int32_t,
                         void*, int64_t, void*, int64_t, int32_t*, uint32_t*, hipStream_t)
{
    return logged("gather");
}

hipError_t launch_add_requests(int32_t, const int32_t*, const int32_t*, const int32_t*,
                               const int32_t*, int32_t, const int32_t*, const int32_t*, int32_t,
                               int32_t, int32_t*, int32_t*, int64_t, int32_t, int32_t*, int32_t,
                               int32_t*, uint32_t*, hipStream_t)
{
    return logged("add_requests");
}

hipError_t launch_append_blocks(int32_t, const int32_t*, const int32_t*, const int32_t*, int32_t,
                                int32_t, int32_t*, int32_t, int32_t*, uint32_t*, hipStream_t)
{
    return logged("append_blocks");
}

hipError_t launch_advance_state(int32_t, const int32_t*, const int32_t*, const int32_t*, int32_t,
                                int32_t*, int32_t*, int64_t, int32_t, uint32_t*, hipStream_t)
{
    return logged("advance_state");
}

hipError_t launch_scatter(int32_t, int64_t, const void*, int64_t, const void*, int64_t, void*,
                          void*, int64_t, const int32_t*, uint32_t*, hipStream_t)
{
    return logged("scatter");
}

hipError_t launch_window_free(int32_t, const int32_t*, const int32_t*, int32_t*, int32_t, int32_t,
                              int32_t, int32_t, int32_t*, int32_t*, uint32_t*, hipStream_t)
{
    return logged("window_free");
}

hipError_t launch_lookahead_slots(int32_t, const int32_t*, const int32_t*, const int32_t*,
                                  int32_t, int32_t, int32_t, int32_t, int32_t, int32_t*,
                                  uint32_t*, hipStream_t)
{
    return logged("lookahead_slots");
}

hipError_t launch_blocks_needed(int32_t, const int32_t*, const int32_t*, int32_t, int32_t,
                                const int32_t*, const int32_t*, int32_t, int32_t*, uint32_t*,
                                hipStream_t)
{
    return logged("blocks_needed");
}

hipError_t launch_hash_blocks(int32_t, const int32_t*, int64_t, const int64_t*, const int32_t*,
                              int32_t, int32_t, uint64_t*, int32_t*, uint32_t*, hipStream_t)
{
    return logged("hash_blocks");
}

hipError_t launch_prefix_lookup(int32_t, const uint64_t*, int32_t, const int32_t*, int32_t,
                                const uint64_t*, const int32_t*, int64_t, int32_t*, int32_t*,
                                uint32_t*, hipStream_t)
{
    return logged("prefix_lookup");
}

hipError_t launch_prefix_insert(int32_t, const uint64_t*, int32_t, const int32_t*,
                                const int32_t*, const int32_t*, const int32_t*, int32_t,
                                uint64_t*, int32_t*, int64_t, uint32_t*, hipStream_t)
{
    return logged("prefix_insert");
}

hipError_t launch_prefix_evict(int32_t, const uint64_t*, const int32_t*, uint64_t*, int32_t*,
                               int64_t, hipStream_t)
{
    return logged("prefix_evict");
}

hipError_t launch_prefix_clear(uint64_t*, int32_t*, int64_t, hipStream_t)
{
    return logged("prefix_clear");
}

}  // namespace pkv
