// The speculative cycle around the verification step (C ABI in
// include/spec_verify_cycle.h): token embedding, the draft loop, the
// verification of the K + 1 positions, and the next input token.
//
// Per draft step (publishertech section 1, "The Speculative Cycle: Draft,
// Verify, and Accept": the drafter runs autoregressively, one token per
// step): gather the input rows of the previous tokens, the drafter's forward
// (the same kernels as the target's), and a draw from each row.  The draw's
// statistics pass also copies the row into the [B, K, V] draft-logit array
// the verification reads, so a draft step adds no copy.  The cycle then
// gathers the K + 1 positions' rows, runs the target forward and the
// vocabulary stage, and moves every request's current token to the last one
// it emitted, all on the caller's stream (section 3, "Eliminating CPU-GPU
// Launch Latency with CUDA Graphs": nothing here needs the host, so the
// whole cycle can be captured once and replayed).
#include <math.h>

#include "common.hpp"
#include "host.hpp"
#include "kernels.hpp"
#include "model.hpp"
#include "spec_verify.h"
#include "spec_verify_cycle.h"

namespace sv {
namespace {

constexpr int kEmbedThreads = 256;

// hidden[r] = table[token(r)]: for a flat token list token(r) = flat[r];
// otherwise r = b * npos + t holds position j = j0 + t of request b, whose
// token is cur[b] (j = 0) or drafts[b * K + j - 1].  A token outside [0, V)
// gives a zero row.
__global__ __launch_bounds__(kEmbedThreads) void embed_kernel(
    const float* __restrict__ table, int V, int d, const int32_t* __restrict__ flat,
    const int32_t* __restrict__ cur, const int32_t* __restrict__ drafts, int K, int j0, int npos,
    float* __restrict__ hidden) {
    const int r = blockIdx.x;
    int tok;
    if (flat) {
        tok = flat[r];
    } else {
        const int b = r / npos, j = j0 + (r - b * npos);
        tok = j == 0 ? cur[b] : drafts[(size_t)b * K + j - 1];
    }
    const bool ok = tok >= 0 && tok < V;
    const f32x4* src = reinterpret_cast<const f32x4*>(table + (size_t)(ok ? tok : 0) * d);
    f32x4* dst = reinterpret_cast<f32x4*>(hidden + (size_t)r * d);
    for (int c = threadIdx.x; c < d / 4; c += kEmbedThreads)
        dst[c] = ok ? src[c] : f32x4{0.f, 0.f, 0.f, 0.f};
}

// cur[b] <- out[b, accept_len[b] - 1], the last token emitted for request b.
__global__ __launch_bounds__(256) void next_input_kernel(const int32_t* __restrict__ out,
                                                         const int32_t* __restrict__ al, int B,
                                                         int K, int32_t* __restrict__ cur) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= B) return;
    const int n = al[b];
    if (n >= 1 && n <= K + 1) cur[b] = out[(size_t)b * (K + 1) + n - 1];
}

hipError_t launch_embed(const float* table, int V, int d, const int32_t* flat, const int32_t* cur,
                        const int32_t* drafts, int K, int j0, int npos, int rows, float* hidden,
                        hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    ProfScope prof("embed", s, (double)rows * d * 8.0, 0.0);
    SV_LAUNCH(prof, embed_kernel, rows, kEmbedThreads, s, table, V, d, flat, cur, drafts, K, j0,
              npos, hidden);
    return hipGetLastError();
}

// Statistics of the B rows (optionally copying each row to copy + b *
// copy_stride), then one draw per row into tokens[b * out_stride].
int run_sample(const float* logits, int B, int V, float T, uint64_t seed, uint32_t step, int slot,
               int32_t* tokens, int out_stride, float* copy, size_t copy_stride, char* ws,
               hipStream_t s) {
    const int greedy = T == 0.0f;
    const float inv_t = greedy ? 0.0f : 1.0f / T;
    const size_t nc = (size_t)stats_chunks(V);
    float* pv = reinterpret_cast<float*>(ws);
    float* ps = reinterpret_cast<float*>(ws + align_up((size_t)B * nc * 4));
    int* pi = reinterpret_cast<int*>(ws + 2 * align_up((size_t)B * nc * 4));
    float* scratch = reinterpret_cast<float*>(ws + 3 * align_up((size_t)B * nc * 4));
    hipError_t e = launch_row_stats(logits, nullptr, B, 0, V, inv_t, greedy, pv, ps, pi, s, copy,
                                    copy_stride);
    if (e != hipSuccess) return hip_fail(e, "row-stats launch");
    e = launch_sample(logits, B, V, inv_t, greedy, seed, step, slot, pv, ps, pi, scratch, tokens,
                      out_stride, s);
    if (e != hipSuccess) return hip_fail(e, "draw launch");
    return SV_OK;
}

size_t sample_bytes(int B, int V) { return accept_bytes(B, 0, V); }

struct DraftPlan {
    size_t off_hidden, off_logits, off_fwd, off_sample, bytes;
};

DraftPlan plan_draft(const sv_model_desc& d, int B) {
    DraftPlan p{};
    size_t o = 0;
    p.off_hidden = o; o = align_up(o + (size_t)B * d.d * 4);
    p.off_logits = o; o = align_up(o + (size_t)B * d.vocab * 4);
    p.off_fwd = o; o = align_up(o + forward_bytes(d, B));
    p.off_sample = o; o = align_up(o + sample_bytes(B, d.vocab));
    p.bytes = o;
    return p;
}

int run_draft(const sv_model_desc& d, const float* table, const int32_t* cur, int B, int K,
              float T, uint64_t seed, uint32_t step, int32_t* drafts, float* dlogits, char* ws,
              hipStream_t s) {
    const DraftPlan p = plan_draft(d, B);
    float* hidden = reinterpret_cast<float*>(ws + p.off_hidden);
    float* logits = reinterpret_cast<float*>(ws + p.off_logits);
    const size_t V = (size_t)d.vocab;
    for (int j = 1; j <= K; ++j) {
        hipError_t e = launch_embed(table, d.vocab, d.d, nullptr, cur, drafts, K, j - 1, 1, B,
                                    hidden, s);
        if (e != hipSuccess) return hip_fail(e, "embed launch");
        int rc = run_forward(d, hidden, B, logits, ws + p.off_fwd, s);
        if (rc != SV_OK) return rc;
        rc = run_sample(logits, B, d.vocab, T, seed, step, j, drafts + (j - 1), K,
                        dlogits + (size_t)(j - 1) * V, (size_t)K * V, ws + p.off_sample, s);
        if (rc != SV_OK) return rc;
    }
    return SV_OK;
}

struct CyclePlan {
    DraftPlan draft;
    size_t off_draft, off_hidden, off_tlogits, off_dtok, off_dlogits, off_fwd, off_acc, bytes;
};

CyclePlan plan_cycle(const sv_model_desc& t, const sv_model_desc* dr, int B, int K) {
    CyclePlan p{};
    const int M = B * (K + 1);
    const size_t V = (size_t)t.vocab;
    size_t o = 0;
    if (K > 0) p.draft = plan_draft(*dr, B);
    p.off_draft = o; o = align_up(o + (K > 0 ? p.draft.bytes : 0));
    p.off_hidden = o; o = align_up(o + (size_t)M * t.d * 4);
    p.off_tlogits = o; o = align_up(o + (size_t)M * V * 4);
    p.off_dtok = o; o = align_up(o + (size_t)B * K * 4);
    p.off_dlogits = o; o = align_up(o + (size_t)B * K * V * 4);
    p.off_fwd = o; o = align_up(o + forward_bytes(t, M));
    p.off_acc = o; o = align_up(o + accept_bytes(B, K, t.vocab));
    p.bytes = o;
    return p;
}

bool rows_ok(int B, int K, int V, int d) {
    const int64_t M = (int64_t)B * (K + 1);
    return M <= (1 << 24) && M * V <= ((int64_t)1 << 40) && M * d <= ((int64_t)1 << 40);
}

int check_ws(void* ws, size_t ws_bytes, size_t need, const char* what) {
    if (!ws || ws_bytes < need || (uintptr_t)ws % kAlign)
        return fail(SV_ERR_WORKSPACE, "%s: workspace must be %zu bytes, %d-byte aligned (got %zu)",
                    what, need, (int)kAlign, ws_bytes);
    return SV_OK;
}

int check_draft_args(const sv_model* drafter, const float* table, const int32_t* cur, int B,
                     int K, float T, const char* what) {
    if (!drafter) return fail(SV_ERR_INVALID_ARG, "%s: null drafter", what);
    if (B < 0 || K < 0) return fail(SV_ERR_INVALID_ARG, "%s: need B >= 0, K >= 0", what);
    if (!temp_ok(T))
        return fail(SV_ERR_INVALID_ARG, "%s: temperature must be finite and 0 or >= FLT_MIN", what);
    if (!rows_ok(B, K, drafter->desc.vocab, drafter->desc.d))
        return fail(SV_ERR_UNSUPPORTED, "%s: B*(K+1) too large", what);
    if (B > 0 && (!table || !cur)) return fail(SV_ERR_INVALID_ARG, "%s: null table or cur", what);
    if ((uintptr_t)table % 16) return fail(SV_ERR_INVALID_ARG, "%s: table must be 16-byte aligned", what);
    return SV_OK;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

int spec_verify_embed(const float* table, int32_t V, int32_t d, const int32_t* tokens, int32_t n,
                      float* hidden, void* stream) {
    if (V < 1 || d < 4 || d % 4 || n < 0)
        return fail(SV_ERR_INVALID_ARG, "embed: need V >= 1, d a positive multiple of 4, n >= 0");
    if (n == 0) return SV_OK;
    if (!table || !tokens || !hidden) return fail(SV_ERR_INVALID_ARG, "embed: null pointer");
    if (((uintptr_t)table | (uintptr_t)hidden) % 16)
        return fail(SV_ERR_INVALID_ARG, "embed: table and hidden must be 16-byte aligned");
    const hipError_t e = launch_embed(table, V, d, tokens, nullptr, nullptr, 0, 0, 1, n, hidden,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SV_OK : hip_fail(e, "embed launch");
}

size_t spec_verify_sample_workspace_bytes(int32_t B, int32_t V) {
    if (B < 0 || V < 1) return 0;
    return B == 0 ? kAlign : sample_bytes(B, V);
}

int spec_verify_sample(const float* logits, int32_t B, int32_t V, float temperature,
                       uint64_t seed, uint32_t step, int32_t slot, int32_t* tokens,
                       int32_t out_stride, void* ws, size_t ws_bytes, void* stream) {
    if (B < 0 || V < 1 || slot < 1 || out_stride < 1)
        return fail(SV_ERR_INVALID_ARG, "sample: need B >= 0, V >= 1, slot >= 1, out_stride >= 1");
    if (!temp_ok(temperature))
        return fail(SV_ERR_INVALID_ARG, "sample: temperature must be finite and 0 or >= FLT_MIN");
    if ((int64_t)B * V > ((int64_t)1 << 40)) return fail(SV_ERR_UNSUPPORTED, "sample: B*V too large");
    if (B == 0) return SV_OK;
    if (!logits || !tokens) return fail(SV_ERR_INVALID_ARG, "sample: null logits or tokens");
    int rc = check_ws(ws, ws_bytes, sample_bytes(B, V), "sample");
    if (rc != SV_OK) return rc;
    return run_sample(logits, B, V, temperature, seed, step, slot, tokens, out_stride, nullptr, 0,
                      static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

size_t spec_verify_draft_workspace_bytes(const sv_model* drafter, int32_t B) {
    if (!drafter || B < 0) return 0;
    return B == 0 ? kAlign : plan_draft(drafter->desc, B).bytes;
}

int spec_verify_draft(const sv_model* drafter, const float* table, const int32_t* cur, int32_t B,
                      int32_t K, float temperature, uint64_t seed, uint32_t step,
                      int32_t* draft_tokens, float* draft_logits, void* ws, size_t ws_bytes,
                      void* stream) {
    int rc = check_draft_args(drafter, table, cur, B, K, temperature, "draft");
    if (rc != SV_OK || B == 0 || K == 0) return rc;
    if (!draft_tokens || !draft_logits)
        return fail(SV_ERR_INVALID_ARG, "draft: null draft_tokens or draft_logits");
    rc = check_ws(ws, ws_bytes, plan_draft(drafter->desc, B).bytes, "draft");
    if (rc != SV_OK) return rc;
    return run_draft(drafter->desc, table, cur, B, K, temperature, seed, step, draft_tokens,
                     draft_logits, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

size_t spec_verify_cycle_workspace_bytes(const sv_model* target, const sv_model* drafter, int32_t B,
                                         int32_t K) {
    if (!target || B < 0 || K < 0 || (K > 0 && !drafter)) return 0;
    if (B == 0) return kAlign;
    return plan_cycle(target->desc, drafter ? &drafter->desc : nullptr, B, K).bytes;
}

int spec_verify_cycle(const sv_model* target, const sv_model* drafter, const float* table,
                      int32_t* cur, int32_t B, int32_t K, float temperature, uint64_t seed,
                      uint32_t step, int32_t* out_tokens, int32_t* accept_len, void* ws,
                      size_t ws_bytes, void* stream) {
    if (!target) return fail(SV_ERR_INVALID_ARG, "cycle: null target");
    const sv_model_desc& t = target->desc;
    int rc;
    if (K > 0) {
        rc = check_draft_args(drafter, table, cur, B, K, temperature, "cycle");
        if (rc != SV_OK) return rc;
        if (drafter->desc.d != t.d || drafter->desc.vocab != t.vocab)
            return fail(SV_ERR_INVALID_ARG, "cycle: drafter and target differ in d or vocabulary");
    } else {
        if (B < 0) return fail(SV_ERR_INVALID_ARG, "cycle: need B >= 0");
        if (!temp_ok(temperature))
            return fail(SV_ERR_INVALID_ARG, "cycle: temperature must be finite and 0 or >= FLT_MIN");
        if (B > 0 && (!table || !cur)) return fail(SV_ERR_INVALID_ARG, "cycle: null table or cur");
        if ((uintptr_t)table % 16)
            return fail(SV_ERR_INVALID_ARG, "cycle: table must be 16-byte aligned");
    }
    if (K < 0) return fail(SV_ERR_INVALID_ARG, "cycle: need K >= 0");
    if (!rows_ok(B, K, t.vocab, t.d)) return fail(SV_ERR_UNSUPPORTED, "cycle: B*(K+1) too large");
    if (B == 0) return SV_OK;
    if (!out_tokens || !accept_len) return fail(SV_ERR_INVALID_ARG, "cycle: null out_tokens or accept_len");
    const CyclePlan p = plan_cycle(t, K > 0 ? &drafter->desc : nullptr, B, K);
    rc = check_ws(ws, ws_bytes, p.bytes, "cycle");
    if (rc != SV_OK) return rc;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    const int M = B * (K + 1);
    float* hidden = reinterpret_cast<float*>(w + p.off_hidden);
    float* tlogits = reinterpret_cast<float*>(w + p.off_tlogits);
    int32_t* dtok = reinterpret_cast<int32_t*>(w + p.off_dtok);
    float* dlogits = reinterpret_cast<float*>(w + p.off_dlogits);
    if (K > 0) {
        rc = run_draft(drafter->desc, table, cur, B, K, temperature, seed, step, dtok, dlogits,
                       w + p.off_draft, s);
        if (rc != SV_OK) return rc;
    }
    hipError_t e = launch_embed(table, t.vocab, t.d, nullptr, cur, dtok, K, 0, K + 1, M, hidden, s);
    if (e != hipSuccess) return hip_fail(e, "embed launch");
    rc = run_forward(t, hidden, M, tlogits, w + p.off_fwd, s);
    if (rc != SV_OK) return rc;
    rc = run_accept(tlogits, K > 0 ? dlogits : nullptr, K > 0 ? dtok : nullptr, B, K, t.vocab,
                    temperature, seed, step, out_tokens, accept_len, nullptr, nullptr,
                    w + p.off_acc, s);
    if (rc != SV_OK) return rc;
    {
        ProfScope prof("next_input", s, (double)B * 12.0, 0.0);
        SV_LAUNCH(prof, next_input_kernel, (unsigned)((B + 255) / 256), 256, s, out_tokens,
                  accept_len, B, K, cur);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "next-input launch");
    }
    return SV_OK;
}

}  // extern "C"
