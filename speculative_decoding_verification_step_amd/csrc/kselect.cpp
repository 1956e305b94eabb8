// Host side of include/spec_verify_kselect.h: goodput-optimal draft length
// per batch size, and the running-average window rule.  Pure host code.
#include <math.h>
#include <stdint.h>

#include "host.hpp"
#include "spec_verify.h"
#include "spec_verify_kselect.h"

namespace sv {
namespace {

// Step time at M rows: the measured value at a measured count, linear
// between the two neighbouring counts, unknown (false) outside the table.
bool verif_time(const int32_t* m, const double* t, int n, double M, double* out) {
    if (M < m[0] || M > m[n - 1]) return false;
    for (int j = 0; j < n; ++j) {
        if (M == (double)m[j]) {
            *out = t[j];
            return true;
        }
        if (j + 1 < n && M < (double)m[j + 1]) {
            const double frac = (M - m[j]) / (double)(m[j + 1] - m[j]);
            *out = t[j] + frac * (t[j + 1] - t[j]);
            return true;
        }
    }
    return false;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

int spec_verify_choose_k(const int32_t* m_rows, const double* t_verif, int32_t n_m,
                         const double* al, int32_t n_k, const int32_t* batch, int32_t n_b,
                         const double* t_draft, int32_t* out_k, double* out_goodput) {
    if (!m_rows || !t_verif || !al || !batch || !out_k)
        return fail(SV_ERR_INVALID_ARG, "choose_k: null array");
    if (n_m < 1 || n_k < 1 || n_b < 1)
        return fail(SV_ERR_INVALID_ARG, "choose_k: sizes must be >= 1 (n_m=%d n_k=%d n_b=%d)",
                    n_m, n_k, n_b);
    for (int j = 0; j < n_m; ++j) {
        if (m_rows[j] < 1 || (j && m_rows[j] <= m_rows[j - 1]))
            return fail(SV_ERR_INVALID_ARG, "choose_k: m_rows must be >= 1 and strictly increasing");
        if (!isfinite(t_verif[j]) || !(t_verif[j] > 0.0))
            return fail(SV_ERR_INVALID_ARG, "choose_k: t_verif[%d] must be finite and > 0", j);
    }
    for (int k = 0; k < n_k; ++k)
        if (!isfinite(al[k]) || al[k] < 1.0 || al[k] > k + 1.0)
            return fail(SV_ERR_INVALID_ARG, "choose_k: al[%d] = %g outside [1, %d]", k, al[k], k + 1);
    for (int i = 0; i < n_b; ++i) {
        if (batch[i] < 1) return fail(SV_ERR_INVALID_ARG, "choose_k: batch[%d] < 1", i);
        if (t_draft)
            for (int k = 0; k < n_k; ++k) {
                const double c = t_draft[(int64_t)i * n_k + k];
                if (!isfinite(c) || c < 0.0)
                    return fail(SV_ERR_INVALID_ARG, "choose_k: t_draft[%d][%d] must be finite and >= 0",
                                i, k);
            }
    }
    // every batch size needs at least one K inside the table before anything is written
    for (int i = 0; i < n_b; ++i) {
        bool any = false;
        double t;
        for (int k = 0; k < n_k && !any; ++k)
            any = verif_time(m_rows, t_verif, n_m, (double)batch[i] * (k + 1), &t);
        if (!any)
            return fail(SV_ERR_INVALID_ARG,
                        "choose_k: no draft length puts batch %d inside the measured rows", batch[i]);
    }
    for (int i = 0; i < n_b; ++i) {
        int best_k = -1;
        double best = 0.0;
        for (int k = 0; k < n_k; ++k) {
            double t;
            if (!verif_time(m_rows, t_verif, n_m, (double)batch[i] * (k + 1), &t)) continue;
            const double itl = t + (t_draft ? t_draft[(int64_t)i * n_k + k] : 0.0);
            const double g = al[k] / itl;
            if (best_k < 0 || g > best) {
                best_k = k;
                best = g;
            }
        }
        out_k[i] = best_k;
        if (out_goodput) out_goodput[i] = best;
    }
    return SV_OK;
}

int32_t spec_verify_window_k(const int32_t* accept_len, int32_t n, int32_t window,
                             float threshold, int32_t k_high, int32_t k_low) {
    if (n < 0 || (n > 0 && !accept_len))
        return fail(SV_ERR_INVALID_ARG, "window_k: need n >= 0 and accept_len for n > 0");
    if (window < 1) return fail(SV_ERR_INVALID_ARG, "window_k: window must be >= 1");
    if (!isfinite(threshold)) return fail(SV_ERR_INVALID_ARG, "window_k: threshold must be finite");
    if (k_low < 0 || k_high < k_low)
        return fail(SV_ERR_INVALID_ARG, "window_k: need 0 <= k_low <= k_high");
    // the most recent `window` valid entries, newest first
    int64_t sum = 0;
    int used = 0;
    for (int j = n - 1; j >= 0 && used < window; --j) {
        if (accept_len[j] < 1) continue;
        sum += accept_len[j];
        ++used;
    }
    if (used < window) return k_high;
    return (double)sum / used < (double)threshold ? k_low : k_high;
}

}  // extern "C"
