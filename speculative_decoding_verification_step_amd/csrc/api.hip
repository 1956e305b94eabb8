// Host side of the C ABI declared in include/spec_verify.h: argument checks,
// workspace carving, the forward's launch sequence and kernel choice, and
// per-launch timing.  Nothing here allocates device memory, synchronises a
// stream, or reads device data.
#include <float.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "host.hpp"
#include "kernels.hpp"
#include "model.hpp"
#include "spec_verify.h"

namespace sv {

namespace {
thread_local std::string g_err;
}  // namespace

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

namespace {

// ---- kernel choice ---------------------------------------------------------
// bf16 weights: matrix cores with the weights streamed straight to registers
// (measured faster than the vector-ALU dot products already at 5 rows);
// fp32 weights: the vector-ALU GEMV.  For measurement, SPEC_VERIFY_MATMUL =
// gemv | skinny overrides the choice for row-major bf16 weights.
int forced_kind() {
    static int k = [] {
        const char* e = getenv("SPEC_VERIFY_MATMUL");
        if (!e) return -1;
        if (!strcmp(e, "gemv")) return (int)kGemvValu;
        if (!strcmp(e, "skinny")) return (int)kMfmaSkinny;
        return -1;
    }();
    return k;
}

// Kernel family per row count: kTiledMinRows, kHeadTiledMinRows and
// kActTiledMinRows (kernels.hpp).

int matmul_kind(const sv_model_desc& d, int M, bool head = false) {
    if (d.wdtype != SV_BF16) return kGemvValu;
    if (d.layout == SV_LAYOUT_TILED) {
        const char* e = getenv("SPEC_VERIFY_MATMUL");
        if (e && !strcmp(e, "skinny")) return kMfmaSkinny;
        if (e && !strcmp(e, "tiled")) return kMfmaTiled;
        return M >= (head ? kHeadTiledMinRows : kTiledMinRows) ? kMfmaTiled : kMfmaSkinny;
    }
    const int f = forced_kind();
    if (f >= 0) return f;
    return kMfmaSkinny;
}

struct ForwardPlan {
    int M = 0;
    int kind = kGemvValu;    // up and down projections
    int head_kind = kGemvValu;
    int splits = 0;          // K splits (partial planes) of the down projection
    int act_tiled = 0;       // bf16 activations in the operand layout (LDS-staged GEMM,
                             // and the streaming kernel from kActTiledMinRows rows)
    size_t off_h = 0, off_a = 0, off_s = 0, off_part = 0, bytes = 0;
};

ForwardPlan plan_forward(const sv_model_desc& d, int M) {
    ForwardPlan p;
    p.M = M;
    p.kind = matmul_kind(d, M);
    p.head_kind = matmul_kind(d, M, true);
    const int tiled = d.layout == SV_LAYOUT_TILED;
    p.act_tiled = p.kind == kMfmaTiled || (p.kind == kMfmaSkinny && tiled && M >= kActTiledMinRows);
    p.splits = p.kind == kMfmaTiled    ? tiled_splits(M, d.d, d.ffn)
               : p.kind == kMfmaSkinny ? skinny_splits(M, d.d, d.ffn, tiled, p.act_tiled)
                                       : 0;
    const int es = d.wdtype == SV_BF16 ? 2 : 4;
    const size_t arows = p.act_tiled ? (size_t)(M + 15) / 16 * 16 : (size_t)M;
    size_t off = 0;
    p.off_h = off; off = align_up(off + (size_t)M * d.d * 4);
    p.off_a = off; off = align_up(off + arows * d.d * es);
    p.off_s = off; off = align_up(off + arows * d.ffn * es);
    p.off_part = off; off = align_up(off + (size_t)p.splits * M * d.d * 4);
    p.bytes = off;
    return p;
}

}  // namespace

size_t forward_bytes(const sv_model_desc& d, int M) { return plan_forward(d, M).bytes; }

// Per-chunk softmax statistics: (max, sum) for every target and draft row,
// argmax for every target row.
size_t accept_bytes(int B, int K, int V) {
    const size_t nc = (size_t)stats_chunks(V);
    const size_t rows = (size_t)B * (K + 1) + (size_t)B * K;
    return align_up(rows * nc * 4) * 2 + align_up((size_t)B * (K + 1) * nc * 4) +
           align_up(accept_meta_floats(B, V) * 4);
}

bool temp_ok(float T) { return isfinite(T) && (T == 0.0f || T >= FLT_MIN); }

int run_forward(const sv_model_desc& d, const float* hidden, int M, float* logits, char* ws,
                hipStream_t s) {
    const ForwardPlan p = plan_forward(d, M);
    const int bf16 = d.wdtype == SV_BF16;
    const int tiled = d.layout == SV_LAYOUT_TILED;
    const size_t es = bf16 ? 2 : 4;
    float* h = reinterpret_cast<float*>(ws + p.off_h);
    void* a = ws + p.off_a;
    void* act_s = ws + p.off_s;
    float* part = reinterpret_cast<float*>(ws + p.off_part);
    hipError_t e;

    // h <- hidden (the residual stream), a <- norm(h)
    e = launch_rmsnorm(hidden, h, nullptr, 0, d.gain, a, M, d.d, d.rms_eps, bf16, p.act_tiled, s);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
    for (int l = 0; l < d.n_layers; ++l) {
        // (ffn and d are multiples of 64, so the tiled matrices have the
        // same element counts as the row-major ones)
        MatmulArgs up{};
        up.W = static_cast<const char*>(d.w_up) + (size_t)l * d.ffn * d.d * es;
        up.act = a;
        up.M = M; up.N = d.ffn; up.K = d.d;
        up.epi = kEpiSilu; up.out = act_s; up.bf16 = bf16; up.tiled = tiled;
        up.act_tiled = p.act_tiled;
        e = launch_matmul(up, p.kind, s);
        if (e != hipSuccess) return hip_fail(e, "up-projection launch");

        MatmulArgs dn{};
        dn.W = static_cast<const char*>(d.w_down) + (size_t)l * d.d * d.ffn * es;
        dn.act = act_s;
        dn.M = M; dn.N = d.d; dn.K = d.ffn;
        dn.epi = kEpiResidual; dn.bf16 = bf16; dn.tiled = tiled;
        dn.act_tiled = p.act_tiled;
        // with a K split the down projection leaves partial planes that the
        // next norm folds in; otherwise it adds into h directly
        dn.out = p.splits ? static_cast<void*>(part) : static_cast<void*>(h);
        dn.splits = p.splits;
        e = launch_matmul(dn, p.kind, s);
        if (e != hipSuccess) return hip_fail(e, "down-projection launch");

        e = launch_rmsnorm(h, h, part, p.splits, d.gain + (size_t)(l + 1) * d.d, a, M, d.d,
                           d.rms_eps, bf16, p.act_tiled, s);
        if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
    }
    MatmulArgs hd{};
    hd.W = d.w_head;
    hd.act = a;
    hd.M = M; hd.N = d.vocab; hd.K = d.d;
    hd.epi = kEpiStore; hd.out = logits; hd.bf16 = bf16; hd.tiled = tiled;
    hd.act_tiled = p.act_tiled;
    e = launch_matmul(hd, p.head_kind, s);
    if (e != hipSuccess) return hip_fail(e, "LM-head launch");
    return SV_OK;
}

int run_accept(const float* tl, const float* dl, const int32_t* x, int B, int K, int V, float T,
               uint64_t seed, uint32_t step, int32_t* out, int32_t* al, float* p_at, float* q_at,
               char* ws, hipStream_t s) {
    const int greedy = T == 0.0f;
    const float inv_t = greedy ? 0.0f : 1.0f / T;
    const size_t n_t = (size_t)B * (K + 1), n_d = (size_t)B * K;
    const size_t nc = (size_t)stats_chunks(V);
    const size_t rows = n_t + n_d;
    float* pv = reinterpret_cast<float*>(ws);
    float* ps = reinterpret_cast<float*>(ws + align_up(rows * nc * 4));
    int* pi = reinterpret_cast<int*>(ws + 2 * align_up(rows * nc * 4));
    float* scratch = reinterpret_cast<float*>(ws + 2 * align_up(rows * nc * 4) +
                                              align_up(n_t * nc * 4));
    hipError_t e = launch_row_stats(tl, dl, (int)n_t, greedy ? 0 : (int)n_d, V, inv_t, greedy,
                                    pv, ps, pi, s);
    if (e != hipSuccess) return hip_fail(e, "row-stats launch");
    e = launch_accept(tl, dl, x, B, K, V, inv_t, greedy, seed, step, pv, ps, pi, scratch, out, al,
                      p_at, q_at, s);
    if (e != hipSuccess) return hip_fail(e, "accept launch");
    return SV_OK;
}

int check_accept_args(const float* tl, const float* dl, const int32_t* x, int B, int K, int V,
                      float T, const int32_t* out, const int32_t* al) {
    if (B < 0 || K < 0 || V < 1)
        return fail(SV_ERR_INVALID_ARG, "need B >= 0, K >= 0, V >= 1 (got B=%d K=%d V=%d)", B, K, V);
    if ((int64_t)B * (K + 1) > INT32_MAX / 2 || (int64_t)B * (K + 1) * V > ((int64_t)1 << 40))
        return fail(SV_ERR_UNSUPPORTED, "B*(K+1)*V too large");
    if (!temp_ok(T))
        return fail(SV_ERR_INVALID_ARG, "temperature must be finite and 0 or >= FLT_MIN (got %g)", (double)T);
    if (B == 0) return SV_OK;
    if (!tl || !out || !al) return fail(SV_ERR_INVALID_ARG, "null target_logits / out_tokens / accept_len");
    if (K > 0 && !x) return fail(SV_ERR_INVALID_ARG, "null draft_tokens with K > 0");
    if (K > 0 && T > 0.0f && !dl) return fail(SV_ERR_INVALID_ARG, "null draft_logits with K > 0 and T > 0");
    return SV_OK;
}

namespace {

// ---- per-launch timing -------------------------------------------------------
struct ProfRec {
    const char* name;
    double bytes, flops;
};

struct ProfState {
    std::mutex mu;
    std::atomic<bool> on{false};
    bool paused = false;
    int cap = 0;
    std::vector<hipEvent_t> ev;
    std::vector<ProfRec> recs;
};

ProfState& prof() {
    static ProfState p;
    return p;
}

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s, double bytes, double flops) {
    (void)s;
    ProfState& p = prof();
    if (!p.on) return;
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.on || p.paused || (int)p.recs.size() >= p.cap) return;
    const size_t slot = p.recs.size();
    p.recs.push_back({name, bytes, flops});
    ev0 = p.ev[2 * slot];
    ev1 = p.ev[2 * slot + 1];
}

}  // namespace sv

using namespace sv;

extern "C" {

int32_t spec_verify_abi_version(void) { return SV_ABI_VERSION; }

const char* spec_verify_last_error(void) { return g_err.c_str(); }

size_t spec_verify_packed_elems(int32_t rows, int32_t cols) {
    if (rows < 1 || cols < 32 || cols % 32) return 0;
    return tiled_elems(rows, cols);
}

int spec_verify_pack_weights(const void* src, void* dst, int32_t rows, int32_t cols,
                             int32_t count, void* stream) {
    if (rows < 1 || cols < 32 || cols % 32 || count < 0 || count > 65535)
        return fail(SV_ERR_INVALID_ARG, "need rows >= 1, cols a positive multiple of 32, 0 <= count <= 65535");
    if (count == 0) return SV_OK;
    if (!src || !dst) return fail(SV_ERR_INVALID_ARG, "null src or dst");
    if (((uintptr_t)src | (uintptr_t)dst) % 16)
        return fail(SV_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    const size_t in_bytes = (size_t)count * rows * cols * 2;
    const size_t out_bytes = (size_t)count * tiled_elems(rows, cols) * 2;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + out_bytes && d0 < s0 + in_bytes)
        return fail(SV_ERR_INVALID_ARG, "src and dst overlap");
    hipError_t e = launch_pack(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst),
                               rows, cols, count, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pack launch");
    return SV_OK;
}

int sv_model_create(const sv_model_desc* desc, sv_model** out) {
    if (!desc || !out) return fail(SV_ERR_INVALID_ARG, "null desc or out");
    *out = nullptr;
    const sv_model_desc& d = *desc;
    if (d.d <= 0 || d.ffn <= 0 || d.vocab <= 0 || d.n_layers < 0)
        return fail(SV_ERR_INVALID_ARG, "need d, ffn, vocab > 0 and n_layers >= 0");
    if (d.d % 64 || d.ffn % 64 || d.d > 32768)
        return fail(SV_ERR_UNSUPPORTED, "d and ffn must be multiples of 64, d <= 32768 (got %d, %d)", d.d, d.ffn);
    if (d.wdtype != SV_F32 && d.wdtype != SV_BF16)
        return fail(SV_ERR_UNSUPPORTED, "weight dtype %d not supported", d.wdtype);
    if (d.layout != SV_LAYOUT_ROW_MAJOR && d.layout != SV_LAYOUT_TILED)
        return fail(SV_ERR_UNSUPPORTED, "layout %d not supported", d.layout);
    if (d.layout == SV_LAYOUT_TILED && d.wdtype != SV_BF16)
        return fail(SV_ERR_UNSUPPORTED, "the tiled layout holds bf16 weights only");
    if (!(d.rms_eps >= 0.0f) || !isfinite(d.rms_eps))
        return fail(SV_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
    if (!d.gain || !d.w_head || (d.n_layers > 0 && (!d.w_up || !d.w_down)))
        return fail(SV_ERR_INVALID_ARG, "null weight pointer");
    const uintptr_t al = (uintptr_t)d.gain | (uintptr_t)d.w_head | (uintptr_t)d.w_up |
                         (uintptr_t)d.w_down;
    if (al % 16) return fail(SV_ERR_INVALID_ARG, "weight pointers must be 16-byte aligned");
    if ((int64_t)d.vocab * d.d > ((int64_t)1 << 40) ||
        (int64_t)d.ffn * d.d > ((int64_t)1 << 40))
        return fail(SV_ERR_UNSUPPORTED, "weight matrix too large");
    sv_model* m = new (std::nothrow) sv_model;
    if (!m) return fail(SV_ERR_INVALID_ARG, "out of host memory");
    m->desc = d;
    *out = m;
    return SV_OK;
}

void sv_model_destroy(sv_model* m) { delete m; }

size_t spec_verify_forward_workspace_bytes(const sv_model* m, int32_t M) {
    if (!m || M < 0) return 0;
    if (M == 0) return kAlign;
    return plan_forward(m->desc, M).bytes;
}

size_t spec_verify_accept_workspace_bytes(int32_t B, int32_t K, int32_t V) {
    if (B < 0 || K < 0 || V < 1) return 0;
    if (B == 0) return kAlign;
    return accept_bytes(B, K, V);
}

size_t spec_verify_workspace_bytes(const sv_model* m, int32_t B, int32_t K) {
    if (!m || B < 0 || K < 0) return 0;
    if (B == 0) return kAlign;
    return plan_forward(m->desc, B * (K + 1)).bytes + accept_bytes(B, K, m->desc.vocab);
}

int spec_verify_forward(const sv_model* m, const float* hidden, int32_t M, float* logits,
                        void* ws, size_t ws_bytes, void* stream) {
    if (!m) return fail(SV_ERR_INVALID_ARG, "null model");
    if (M < 0) return fail(SV_ERR_INVALID_ARG, "M must be >= 0 (got %d)", M);
    if (M == 0) return SV_OK;
    if ((int64_t)M * m->desc.vocab > ((int64_t)1 << 40) || M > (1 << 24))
        return fail(SV_ERR_UNSUPPORTED, "M too large");
    if (!hidden || !logits) return fail(SV_ERR_INVALID_ARG, "null hidden or logits");
    if (((uintptr_t)hidden | (uintptr_t)logits) % 16)
        return fail(SV_ERR_INVALID_ARG, "hidden and logits must be 16-byte aligned");
    const size_t need = plan_forward(m->desc, M).bytes;
    if (!ws || ws_bytes < need || (uintptr_t)ws % kAlign)
        return fail(SV_ERR_WORKSPACE, "workspace must be %zu bytes, %d-byte aligned (got %zu)", need,
                    (int)kAlign, ws_bytes);
    return run_forward(m->desc, hidden, M, logits, static_cast<char*>(ws),
                       static_cast<hipStream_t>(stream));
}

int spec_verify_accept(const float* target_logits, const float* draft_logits,
                       const int32_t* draft_tokens, int32_t B, int32_t K, int32_t V,
                       float temperature, uint64_t seed, uint32_t step, int32_t* out_tokens,
                       int32_t* accept_len, float* p_at_draft, float* q_at_draft, void* ws,
                       size_t ws_bytes, void* stream) {
    int rc = check_accept_args(target_logits, draft_logits, draft_tokens, B, K, V, temperature,
                               out_tokens, accept_len);
    if (rc != SV_OK || B == 0) return rc;
    const size_t need = accept_bytes(B, K, V);
    if (!ws || ws_bytes < need || (uintptr_t)ws % kAlign)
        return fail(SV_ERR_WORKSPACE, "workspace must be %zu bytes, %d-byte aligned (got %zu)", need,
                    (int)kAlign, ws_bytes);
    return run_accept(target_logits, draft_logits, draft_tokens, B, K, V, temperature, seed, step,
                      out_tokens, accept_len, p_at_draft, q_at_draft, static_cast<char*>(ws),
                      static_cast<hipStream_t>(stream));
}

int spec_verify_step(const sv_model* m, const float* hidden, const float* draft_logits,
                     const int32_t* draft_tokens, int32_t B, int32_t K, float temperature,
                     uint64_t seed, uint32_t step, float* logits_out, int32_t* out_tokens,
                     int32_t* accept_len, float* p_at_draft, float* q_at_draft, void* ws,
                     size_t ws_bytes, void* stream) {
    if (!m) return fail(SV_ERR_INVALID_ARG, "null model");
    int rc = check_accept_args(logits_out, draft_logits, draft_tokens, B, K, m->desc.vocab,
                               temperature, out_tokens, accept_len);
    if (rc != SV_OK || B == 0) return rc;
    const int64_t M64 = (int64_t)B * (K + 1);
    if (M64 > (1 << 24) || M64 * m->desc.vocab > ((int64_t)1 << 40))
        return fail(SV_ERR_UNSUPPORTED, "B*(K+1) too large");
    const int M = (int)M64;
    if (!hidden) return fail(SV_ERR_INVALID_ARG, "null hidden");
    if (((uintptr_t)hidden | (uintptr_t)logits_out) % 16)
        return fail(SV_ERR_INVALID_ARG, "hidden and logits_out must be 16-byte aligned");
    const size_t fwd = plan_forward(m->desc, M).bytes;
    const size_t need = fwd + accept_bytes(B, K, m->desc.vocab);
    if (!ws || ws_bytes < need || (uintptr_t)ws % kAlign)
        return fail(SV_ERR_WORKSPACE, "workspace must be %zu bytes, %d-byte aligned (got %zu)", need,
                    (int)kAlign, ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = run_forward(m->desc, hidden, M, logits_out, static_cast<char*>(ws), s);
    if (rc != SV_OK) return rc;
    return run_accept(logits_out, draft_logits, draft_tokens, B, K, m->desc.vocab, temperature,
                      seed, step, out_tokens, accept_len, p_at_draft, q_at_draft,
                      static_cast<char*>(ws) + fwd, s);
}

int spec_verify_profile_begin(int32_t max_launches) {
    if (max_launches < 1 || max_launches > (1 << 20))
        return fail(SV_ERR_INVALID_ARG, "max_launches must be in [1, 2^20]");
    ProfState& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (p.on) return fail(SV_ERR_INVALID_ARG, "profiling already on");
    p.ev.assign(2 * (size_t)max_launches, nullptr);
    for (auto& e : p.ev) {
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            for (auto& f : p.ev)
                if (f) (void)hipEventDestroy(f);
            p.ev.clear();
            return hip_fail(r, "hipEventCreate");
        }
    }
    p.recs.clear();
    p.recs.reserve(max_launches);
    p.cap = max_launches;
    p.paused = false;
    p.on = true;
    return SV_OK;
}

int spec_verify_profile_pause(int32_t paused) {
    ProfState& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.on) return fail(SV_ERR_INVALID_ARG, "profiling not on");
    p.paused = paused != 0;
    return SV_OK;
}

int spec_verify_profile_end(sv_kernel_time* out, int32_t cap, int32_t* n_out) {
    ProfState& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.on) return fail(SV_ERR_INVALID_ARG, "profiling not on");
    p.on = false;
    int rc = SV_OK;
    std::vector<sv_kernel_time> agg;
    for (size_t i = 0; i < p.recs.size(); ++i) {
        hipError_t r = hipEventSynchronize(p.ev[2 * i + 1]);
        float ms = 0.f;
        if (r == hipSuccess) r = hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]);
        if (r != hipSuccess) {
            rc = hip_fail(r, "profile event");
            break;
        }
        sv_kernel_time* t = nullptr;
        for (auto& a : agg)
            if (strncmp(a.name, p.recs[i].name, sizeof a.name) == 0) t = &a;
        if (!t) {
            agg.push_back(sv_kernel_time{});
            t = &agg.back();
            snprintf(t->name, sizeof t->name, "%s", p.recs[i].name);
        }
        t->launches += 1;
        t->total_ms += ms;
        t->bytes += p.recs[i].bytes;
        t->flops += p.recs[i].flops;
    }
    for (auto& e : p.ev) (void)hipEventDestroy(e);
    p.ev.clear();
    p.recs.clear();
    if (rc != SV_OK) return rc;
    const int n = (int)agg.size();
    if (n_out) *n_out = n;
    if (out)
        for (int i = 0; i < n && i < cap; ++i) out[i] = agg[i];
    return SV_OK;
}

}  // extern "C"
