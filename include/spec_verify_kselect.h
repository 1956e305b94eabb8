/* Hardware-aware choice of the draft length K for the verification step.
 *
 * Host-side companions of spec_verify.h: they read host arrays only, launch
 * nothing and never touch device memory.  Status codes are those of
 * spec_verify.h (SV_OK = 0, negative on error; spec_verify_last_error()
 * describes the last failure on the calling thread).
 */
#ifndef SPEC_VERIFY_KSELECT_H
#define SPEC_VERIFY_KSELECT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Goodput-optimal draft length for each batch size.
 *
 * Cohere, "Hardware-Aware, Dynamic Speculative Decoding (DSD)", section
 * "Dynamic speculative decoding": the draft length is chosen per batch size
 * from offline profiles of acceptance length and inter-token latency, by
 * the goodput AL / ITL, with ITL the sum of the draft and verification
 * times; the result is a lookup table used at run time.  The same ratio,
 * taken against K = 0, is the speedup of the NVIDIA co-design post
 * ("What is speculative decoding?"): T_verif(B) * AL / (T_verif(B (1+D)) +
 * T_draft(B, D)).
 *
 *   m_rows[n_m]   ascending row counts M = B * (K + 1) at which the
 *                 verification step was timed (int32, >= 1, strictly
 *                 increasing)
 *   t_verif[n_m]  the step times there (any unit, finite, > 0); between two
 *                 measured counts the time is linear in M, outside the
 *                 table it is unknown
 *   al[n_k]       expected tokens emitted per request at K = 0 .. n_k - 1
 *                 (finite, 1 <= al[K] <= K + 1)
 *   batch[n_b]    batch sizes B (>= 1)
 *   t_draft       NULL (no draft cost) or [n_b][n_k] row-major draft times
 *                 for (batch[i], K), same unit as t_verif (finite, >= 0)
 *   out_k[n_b]    (output) for batch[i], the K in 0 .. n_k - 1 with
 *                 B * (K + 1) inside the table that maximises
 *                 goodput = al[K] / (T_verif(B * (K + 1)) + t_draft[i][K]);
 *                 the smallest such K on ties
 *   out_goodput   NULL or (output) [n_b] that goodput (tokens per request
 *                 per unit of time)
 *
 * All arrays are host memory owned by the caller.  Returns SV_OK, or
 * SV_ERR_INVALID_ARG (nothing written) for a null pointer, a size < 1, a
 * value outside the ranges above, or a batch size for which no K lands
 * inside the measured range. */
int spec_verify_choose_k(const int32_t* m_rows, const double* t_verif, int32_t n_m,
                         const double* al, int32_t n_k, const int32_t* batch, int32_t n_b,
                         const double* t_draft, int32_t* out_k, double* out_goodput);

/* Speculation window from recent acceptance lengths.
 *
 * mohashari, "Speculative Decoding in Production", section "Production
 * Failure Modes and Mitigation Strategies", item 1 "Draft Acceptance Rate
 * Collapse (Entropy Shift)" (dynamic window sizing): when the running
 * average of accepted tokens per request over the last few requests falls
 * below a threshold (the page: 1.5 over the last 10), the window K drops
 * from its normal value (the page: 5) to a small one (1 or 2).  "Accepted
 * tokens" is read as the acceptance length AL (tokens emitted per request
 * per step, the page's E[N]), so a low window recovers once AL does.
 *
 *   accept_len[n]  host array of recent acceptance lengths, oldest first;
 *                  entries < 1 (requests rejected as invalid) are skipped
 *   window         how many of the most recent valid entries to average (>= 1)
 *   threshold      the running-average threshold (finite)
 *   k_high, k_low  the normal and the reduced window (0 <= k_low <= k_high)
 *
 * Returns k_low when at least `window` valid entries exist and their mean is
 * below `threshold`, else k_high; SV_ERR_INVALID_ARG (< 0) on bad arguments
 * (accept_len may be NULL only when n == 0). */
int32_t spec_verify_window_k(const int32_t* accept_len, int32_t n, int32_t window,
                             float threshold, int32_t k_high, int32_t k_low);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_KSELECT_H */
