// rowpool.cpp -- the pool of request_state_index rows (host code only).
//
// A new request is handed a row of the persistent state and a completed one
// gives it back to be handed out again, so rows are pooled rather than
// allocated ("Design Logic Behind the Dual-Index System" of "Deep Dive into
// vLLM's Scheduling Mechanism: The Complete CPU-to-GPU Mapping Pipeline",
// kongchang.com/en).  Which row a request gets is decided where the schedule
// is built -- the host needs the row to name the request in sched_rows -- so
// the pool lives on the host; the state behind the rows lives on the device.
//
// The free rows are a stack: rows 0, 1, 2, ... come out first, and the row
// released last is handed out next (its state is the most likely to still be
// in the GPU's caches).  acquire and release are all-or-nothing.
#include <algorithm>
#include <new>
#include <vector>

#include "pagedkv.h"

struct pkv_row_pool {
    std::vector<int32_t> free_rows;     // stack; top = back()
    std::vector<uint8_t> in_use;        // 1 while handed out
    std::vector<uint32_t> mark;         // release's duplicate check (per-call epoch)
    uint32_t epoch = 0;
};

extern "C" {

int pkv_row_pool_create(int32_t R, pkv_row_pool** out)
{
    if (R < 0 || out == nullptr)
        return PKV_EINVAL;
    *out = nullptr;
    pkv_row_pool* p = new (std::nothrow) pkv_row_pool;
    if (p == nullptr)
        return PKV_ENOMEM;
    try {
        p->free_rows.resize((size_t)R);
        p->in_use.assign((size_t)R, 0);
        p->mark.assign((size_t)R, 0);
    } catch (...) {
        delete p;
        return PKV_ENOMEM;
    }
    for (int32_t i = 0; i < R; ++i)
        p->free_rows[(size_t)i] = R - 1 - i;
    *out = p;
    return PKV_OK;
}

void pkv_row_pool_destroy(pkv_row_pool* pool) { delete pool; }

int32_t pkv_row_pool_num_free(const pkv_row_pool* pool)
{
    return pool == nullptr ? -1 : (int32_t)pool->free_rows.size();
}

int pkv_row_pool_acquire(pkv_row_pool* pool, int32_t m, int32_t* rows)
{
    if (pool == nullptr || m < 0 || (m > 0 && rows == nullptr))
        return PKV_EINVAL;
    if ((size_t)m > pool->free_rows.size())
        return PKV_ENOROWS;
    for (int32_t i = 0; i < m; ++i) {
        const int32_t r = pool->free_rows.back();
        pool->free_rows.pop_back();
        pool->in_use[(size_t)r] = 1;
        rows[i] = r;
    }
    return PKV_OK;
}

int pkv_row_pool_release(pkv_row_pool* pool, int32_t m, const int32_t* rows)
{
    if (pool == nullptr || m < 0 || (m > 0 && rows == nullptr))
        return PKV_EINVAL;
    const int32_t R = (int32_t)pool->in_use.size();
    if (++pool->epoch == 0) {                 // epoch wrapped: clear the marks once
        std::fill(pool->mark.begin(), pool->mark.end(), 0u);
        pool->epoch = 1;
    }
    for (int32_t i = 0; i < m; ++i) {
        const int32_t r = rows[i];
        if (r < 0 || r >= R || !pool->in_use[(size_t)r] || pool->mark[(size_t)r] == pool->epoch)
            return PKV_EINVAL;
        pool->mark[(size_t)r] = pool->epoch;
    }
    for (int32_t i = 0; i < m; ++i) {
        pool->in_use[(size_t)rows[i]] = 0;
        pool->free_rows.push_back(rows[i]);
    }
    return PKV_OK;
}

}  // extern "C"
