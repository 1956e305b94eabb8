/* Causal attention of the verified positions over a paged KV cache.
 *
 * The target scores all drafted slots of a request in one pass (NVIDIA
 * co-design post, "What is speculative decoding?"): the T = K + 1 positions
 * verified in a step sit at sequence positions ctx_len[b] .. ctx_len[b] + K,
 * and position t attends to every earlier position and to itself.  The KV
 * cache is paged (publishertech, section 4 "Segmented Block Allocation
 * (PagedAttention)"): fixed-size physical blocks named by a per-request
 * block table, so rolling back rejected positions moves the committed
 * length and returns trailing blocks to a free list without copying cached
 * data (same section; mohashari, "Serving Architecture and KV Cache
 * Syncing").
 *
 * Companion of spec_verify.h: same status codes (SV_OK = 0, negative on
 * error; spec_verify_last_error() describes the last failure on the calling
 * thread), same rules: device pointers, stream-ordered, no allocation, no
 * synchronisation, no host reads of device data, all argument checks on the
 * host before anything is enqueued.
 *
 * Layouts (bf16 = IEEE bfloat16 bits in uint16):
 *   q        [B, T, Hq, Dh] bf16, T = K + 1 query positions per request
 *   k_cache  [num_blocks, Hkv, SV_KV_BLOCK, Dh] bf16
 *   v_cache  [num_blocks, Hkv, Dh, SV_KV_BLOCK] bf16 (V transposed inside a
 *            block: the layout the matrix cores read P V from)
 *   block_table [B, max_blocks] int32: physical block of positions
 *            SV_KV_BLOCK*i .. SV_KV_BLOCK*i + SV_KV_BLOCK - 1 of request b
 *   ctx_len  [B] int32: committed positions of request b before the step
 *   query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 * Device data are not validated (that would need a host read): block ids
 * are clamped to [0, num_blocks) and lengths to [0, max_blocks *
 * SV_KV_BLOCK], so a bad table gives wrong values but never an access
 * outside the buffers.
 */
#ifndef SPEC_VERIFY_ATTN_H
#define SPEC_VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_KV_BLOCK 32 /* tokens per KV block */

/* Workspace for spec_verify_attention: partial results when the context is
 * split across workgroups (0 when it is not).  Depends on the sizes only. */
size_t spec_verify_attention_workspace_bytes(int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                                             int32_t head_dim, int32_t max_blocks);

/* Write the T new positions' keys and values (k_new, v_new [B, T, Hkv, Dh]
 * bf16) of every request at positions ctx_len[b] + t.  The caller has
 * reserved blocks for them (sv_kv_pool_reserve); positions beyond
 * max_blocks * SV_KV_BLOCK are skipped.  head_dim in {64, 128}. */
int spec_verify_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          const int32_t* block_table, const int32_t* ctx_len, int32_t B, int32_t T,
                          int32_t Hkv, int32_t head_dim, int32_t max_blocks, int32_t num_blocks,
                          hipStream_t stream);

/* out[b, t, h, :] (fp32 [B, T, Hq, Dh]) = softmax(scale * K q) V over
 * positions 0 .. ctx_len[b] + t of request b (the step's own positions must
 * have been appended).  head_dim in {64, 128}; Hq a multiple of Hkv.
 * ws / ws_bytes: device workspace of spec_verify_attention_workspace_bytes
 * (ws may be NULL when that is 0).  The context is split across
 * workgroups by max_blocks, so size the table to the batch's longest
 * request. */
int spec_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* ctx_len, int32_t B, int32_t T,
                          int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t max_blocks,
                          int32_t num_blocks, float scale, float* out, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* After verification: ctx_len[b] += accept_len[b] on the device (the step's
 * input position and the AL - 1 accepted drafts stay committed; the
 * rejected slots are simply overwritten by the next step).  Requests with
 * accept_len < 1 (rejected as invalid) keep their length. */
int spec_verify_kv_commit(int32_t* ctx_len, const int32_t* accept_len, int32_t B,
                          hipStream_t stream);

/* Host-side free list of physical blocks (publishertech section 4: the block
 * allocator hands out block pointers for speculative positions and takes
 * back those of rejected ones).  A stack: the block freed last is reused
 * first; a new pool hands out 0, 1, 2, ...  Not thread-safe. */
typedef struct sv_kv_pool sv_kv_pool;

int sv_kv_pool_create(int32_t num_blocks, sv_kv_pool** out);
void sv_kv_pool_destroy(sv_kv_pool* pool);
int32_t sv_kv_pool_free_blocks(const sv_kv_pool* pool);

/* Append blocks to a request's host table row (n_blocks in use, at most
 * max_blocks) until it covers `tokens` positions.  O(blocks added).
 * SV_ERR_WORKSPACE (nothing changed) when the pool or the row is too small. */
int sv_kv_pool_reserve(sv_kv_pool* pool, int32_t* table_row, int32_t* n_blocks,
                       int32_t max_blocks, int32_t tokens);

/* The rollback: return the blocks past the first `tokens` positions of the
 * row to the pool.  O(blocks returned); no cached data moves. */
int sv_kv_pool_trim(sv_kv_pool* pool, int32_t* table_row, int32_t* n_blocks, int32_t tokens);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_ATTN_H */
