// Host-side block pool of include/spec_verify_attn.h: a stack of free
// physical KV-block ids; reserve pops blocks onto a request's table row, trim
// pushes the row's trailing blocks back (the rollback of rejected positions).
#include <stdint.h>

#include <new>
#include <vector>

#include "host.hpp"
#include "spec_verify.h"
#include "spec_verify_attn.h"

struct sv_kv_pool {
    std::vector<int32_t> free;   // top of the stack = back
};

using sv::fail;

extern "C" {

int sv_kv_pool_create(int32_t num_blocks, sv_kv_pool** out) {
    if (!out) return fail(SV_ERR_INVALID_ARG, "kv_pool_create: null output");
    *out = nullptr;
    if (num_blocks < 1) return fail(SV_ERR_INVALID_ARG, "kv_pool_create: num_blocks < 1");
    sv_kv_pool* p = new (std::nothrow) sv_kv_pool;
    if (!p) return fail(SV_ERR_INVALID_ARG, "kv_pool_create: out of host memory");
    try {
        p->free.resize(num_blocks);
    } catch (...) {
        delete p;
        return fail(SV_ERR_INVALID_ARG, "kv_pool_create: out of host memory");
    }
    for (int32_t i = 0; i < num_blocks; ++i) p->free[i] = num_blocks - 1 - i;   // hands out 0, 1, ...
    *out = p;
    return SV_OK;
}

void sv_kv_pool_destroy(sv_kv_pool* pool) { delete pool; }

int32_t sv_kv_pool_free_blocks(const sv_kv_pool* pool) {
    return pool ? (int32_t)pool->free.size() : 0;
}

int sv_kv_pool_reserve(sv_kv_pool* pool, int32_t* table_row, int32_t* n_blocks,
                       int32_t max_blocks, int32_t tokens) {
    if (!pool || !table_row || !n_blocks) return fail(SV_ERR_INVALID_ARG, "kv_pool_reserve: null pointer");
    if (tokens < 0 || max_blocks < 0 || *n_blocks < 0 || *n_blocks > max_blocks)
        return fail(SV_ERR_INVALID_ARG, "kv_pool_reserve: bad sizes");
    const int64_t need = ((int64_t)tokens + SV_KV_BLOCK - 1) / SV_KV_BLOCK;
    if (need > max_blocks)
        return fail(SV_ERR_WORKSPACE, "kv_pool_reserve: %d tokens need %lld blocks, the row holds %d",
                    tokens, (long long)need, max_blocks);
    const int64_t add = need - *n_blocks;
    if (add > (int64_t)pool->free.size())
        return fail(SV_ERR_WORKSPACE, "kv_pool_reserve: %lld blocks needed, %zu free",
                    (long long)add, pool->free.size());
    while (*n_blocks < need) {
        table_row[(*n_blocks)++] = pool->free.back();
        pool->free.pop_back();
    }
    return SV_OK;
}

int sv_kv_pool_trim(sv_kv_pool* pool, int32_t* table_row, int32_t* n_blocks, int32_t tokens) {
    if (!pool || !table_row || !n_blocks) return fail(SV_ERR_INVALID_ARG, "kv_pool_trim: null pointer");
    if (tokens < 0 || *n_blocks < 0) return fail(SV_ERR_INVALID_ARG, "kv_pool_trim: bad sizes");
    const int64_t keep = ((int64_t)tokens + SV_KV_BLOCK - 1) / SV_KV_BLOCK;
    while (*n_blocks > keep) pool->free.push_back(table_row[--(*n_blocks)]);
    return SV_OK;
}

}  // extern "C"
