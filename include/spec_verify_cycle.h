/* The speculative cycle around the verification step: a draft loop that
 * proposes K tokens one after another, the verification of the K + 1
 * positions in one target pass, and the next input token (publishertech,
 * section 1 "The Speculative Cycle: Draft, Verify, and Accept": the drafter
 * runs gamma steps autoregressively, the target scores all of them in one
 * pass; section 2 "Theoretical Speedup Equation": T_cycle = gamma t_draft +
 * t_target; section 3 "Eliminating CPU-GPU Launch Latency with CUDA Graphs":
 * the draft loop is captured once and replayed with one launch).  With K = 0
 * a cycle is one step of plain decoding: the target alone samples the next
 * token.
 *
 * Tokens enter a model through an embedding table: the input row of a
 * position holding token x is table[x] (fp32 [V, d]).  The drafter is any
 * sv_model over the same d and vocabulary, for instance the target's first
 * blocks with its final norm and its own head (an early exit that shares the
 * target's weights).
 *
 * Uniforms (Philox4x32-10, key = seed): the token drawn for draft slot j
 * (1..K) of request b uses counter (b, j, 2, step); the verification uses
 * (b, j, 0, step) and (b, j, 1, step) as spec_verify_accept documents.  A
 * draw picks the smallest token id whose running sum of softmax(z / T)
 * exceeds u * (the row's total), u = (w >> 8) * 2^-24 from Philox word 0 w;
 * at T = 0 the argmax (lowest id on ties).
 *
 * Companion of spec_verify.h: the same status codes and rules (device
 * pointers, stream-ordered, no allocation, no synchronisation, no host reads
 * of device data, every argument check on the host before anything is
 * enqueued), so a whole cycle can be captured in one graph.  Workspaces are
 * device buffers of at least the stated size, 256-byte aligned.
 */
#ifndef SPEC_VERIFY_CYCLE_H
#define SPEC_VERIFY_CYCLE_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* hidden[i] (fp32 [n, d]) = table[tokens[i]] (fp32 [V, d]); a token outside
 * [0, V) gives a zero row.  d a multiple of 4. */
int spec_verify_embed(const float* table, int32_t V, int32_t d, const int32_t* tokens, int32_t n,
                      float* hidden, void* stream);

/* One token per row of logits [B, V] fp32: tokens[b * out_stride] is drawn
 * from softmax(logits[b] / T) with the counter (b, slot, 2, step), slot >= 1
 * (argmax at T = 0). */
size_t spec_verify_sample_workspace_bytes(int32_t B, int32_t V);
int spec_verify_sample(const float* logits, int32_t B, int32_t V, float temperature,
                       uint64_t seed, uint32_t step, int32_t slot, int32_t* tokens,
                       int32_t out_stride, void* ws, size_t ws_bytes, void* stream);

/* The draft loop: from the current token cur[b] of every request, K steps of
 * the drafter, each on the token drawn by the step before:
 *   z = drafter(table[x_{j-1}]),  draft_logits[b, j-1, :] = z,
 *   x_j = draw from softmax(z / T) with counter (b, j, 2, step),
 *   draft_tokens[b, j-1] = x_j,            j = 1..K, x_0 = cur[b].
 * draft_tokens [B, K] int32, draft_logits [B, K, V] fp32: the inputs of
 * spec_verify_accept / spec_verify_step. */
size_t spec_verify_draft_workspace_bytes(const sv_model* drafter, int32_t B);
int spec_verify_draft(const sv_model* drafter, const float* table, const int32_t* cur, int32_t B,
                      int32_t K, float temperature, uint64_t seed, uint32_t step,
                      int32_t* draft_tokens, float* draft_logits, void* ws, size_t ws_bytes,
                      void* stream);

/* One speculative cycle: the draft loop above, then the verification of the
 * positions cur[b], x_1 .. x_K by the target (spec_verify_step), then
 * cur[b] <- the last token emitted for b (unchanged if the request was
 * rejected as invalid).  out_tokens [B, K+1], accept_len [B] as in
 * spec_verify_accept.  drafter may be NULL when K = 0. */
size_t spec_verify_cycle_workspace_bytes(const sv_model* target, const sv_model* drafter, int32_t B,
                                         int32_t K);
int spec_verify_cycle(const sv_model* target, const sv_model* drafter, const float* table,
                      int32_t* cur, int32_t B, int32_t K, float temperature, uint64_t seed,
                      uint32_t step, int32_t* out_tokens, int32_t* accept_len, void* ws,
                      size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_CYCLE_H */
