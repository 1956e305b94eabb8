/* Verification forward of a mixture-of-experts target.
 *
 * Every block is a pre-norm MoE block: a router scores the n_experts
 * experts for each of the M = B (K + 1) verified positions, the top_k are
 * kept (ties to the lower expert id) and weighted by the softmax of their
 * scores, each chosen expert is a SiLU MLP (up [ffn, d], down [d, ffn]),
 * and the weighted expert outputs are added to the residual stream in rank
 * order; a final RMSNorm and the LM head follow.  Verifying more positions
 * touches more experts, so the weight bytes of a step grow with M until
 * every expert is loaded (Cohere, "Hardware-Aware, Dynamic Speculative
 * Decoding", section "Dynamic speculative decoding"; NVIDIA co-design post,
 * "Draft length and performance of linear layers": grouped expert GEMMs).
 * Only the experts a step uses are read: the grouped kernels skip experts
 * with no positions before touching their weights.
 *
 * Companion of spec_verify.h (same status codes, same stream / workspace /
 * no-allocation rules; logits feed spec_verify_accept unchanged).  Weights
 * are bf16 in the tiled layout of spec_verify_pack_weights:
 *   w_router  n_layers packed [n_experts, d] matrices
 *   w_up      n_layers * n_experts packed [ffn, d] matrices (layer-major)
 *   w_down    n_layers * n_experts packed [d, ffn] matrices
 *   gain      [n_layers + 1, d] fp32 (the last row is the final norm)
 *   w_head    one packed [vocab, d] matrix
 * Limits: d a multiple of 64 (<= 32768), ffn a multiple of 32,
 * 1 <= top_k <= min(8, n_experts), n_experts <= 256, M <= 1024.
 */
#ifndef SPEC_VERIFY_MOE_H
#define SPEC_VERIFY_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t d, ffn, n_experts, top_k, n_layers, vocab;
    float rms_eps;
    const void* w_router;
    const void* w_up;
    const void* w_down;
    const float* gain;
    const void* w_head;
} sv_moe_desc;

typedef struct sv_moe sv_moe; /* opaque; borrows the weight pointers */

int sv_moe_create(const sv_moe_desc* desc, sv_moe** out);
void sv_moe_destroy(sv_moe* model);

size_t spec_verify_moe_workspace_bytes(const sv_moe* model, int32_t M);

/* logits [M, vocab] fp32 of hidden [M, d] fp32.  active_experts: NULL or a
 * device int32 [n_layers] that receives, per block, the number of distinct
 * experts the M positions used.  Returns SV_OK or a negative status
 * (nothing enqueued on argument errors). */
int spec_verify_moe_forward(const sv_moe* model, const float* hidden, int32_t M, float* logits,
                            int32_t* active_experts, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_MOE_H */
