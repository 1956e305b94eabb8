// Verification forward of a mixture-of-experts target (C ABI in
// include/spec_verify_moe.h).
//
// Per block: RMSNorm -> router (streaming MFMA matmul, [M, E] scores) ->
// routing (one workgroup: top_k per position, softmax weights, and a
// counting sort of the M * top_k (position, slot) pairs by expert, in
// position order, so every expert's rows are one contiguous range) ->
// grouped up projection (+ SiLU) -> grouped down projection -> combine
// (h += sum over slots, in rank order, of weight * expert output).  The
// grouped kernels give every (expert, 16-row weight fragment) a workgroup
// that returns before touching memory when the expert has no rows, so a step
// streams the weights of the experts it uses and nothing else - the effect
// the pages attribute to MoE verification (Cohere, "Dynamic speculative
// decoding"): more verified positions, more experts loaded.  The matmul core
// is the streaming one of the dense path: weight fragments from HBM straight
// into registers as the A operand of v_mfma_f32_16x16x32_bf16, eight waves
// splitting the reduction, a fixed-order LDS sum.
#include <float.h>
#include <math.h>
#include <string.h>

#include <new>

#include "common.hpp"
#include "host.hpp"
#include "kernels.hpp"
#include "spec_verify.h"
#include "spec_verify_moe.h"

struct sv_moe {
    sv_moe_desc desc;
};

namespace sv {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kMoeMaxRows = 1024;     // positions per call (routing in one workgroup)
constexpr int kMoeMaxExperts = 256;
constexpr int kMoeMaxTopK = 8;
constexpr int kRouteThreads = 1024;
constexpr int kRouteChunk = 32;       // positions per counting chunk
constexpr int kGroupWaves = 8;        // k slices of a grouped workgroup
constexpr int kGroupSteps = 2;        // 32-wide k steps per buffer

// ---- routing ------------------------------------------------------------------
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const float* __restrict__ z, int M, int E, int k, int32_t* __restrict__ sel_out,
    float* __restrict__ wts, int32_t* __restrict__ offs, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ active) {
    __shared__ int32_t lsel[kMoeMaxRows * kMoeMaxTopK];
    __shared__ int32_t cnt[kMoeMaxRows / kRouteChunk][kMoeMaxExperts];
    __shared__ int32_t loff[kMoeMaxExperts + 1];
    const int tid = threadIdx.x;
    const int nchunk = (M + kRouteChunk - 1) / kRouteChunk;

    // top_k of each position: k passes of an argmax over the unchosen experts
    // (strict >: the lower id wins ties), then softmax over the chosen scores
    for (int t = tid; t < M; t += kRouteThreads) {
        const float* zr = z + (size_t)t * E;
        uint32_t taken[kMoeMaxExperts / 32];
#pragma unroll
        for (int w = 0; w < kMoeMaxExperts / 32; ++w) taken[w] = 0u;
        float zs[kMoeMaxTopK];
        int es[kMoeMaxTopK];
        for (int j = 0; j < k; ++j) {
            float best = -INFINITY;
            int bi = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e >> 5] & (1u << (e & 31))) continue;
                const float v = zr[e] == zr[e] ? zr[e] : -INFINITY;   // NaN ranks last
                if (bi < 0 || v > best) {
                    best = v;
                    bi = e;
                }
            }
            taken[bi >> 5] |= 1u << (bi & 31);
            es[j] = bi;
            zs[j] = best;
        }
        float sum = 0.f, ex[kMoeMaxTopK];
        for (int j = 0; j < k; ++j) {
            ex[j] = zs[0] == -INFINITY ? 1.f : expf(zs[j] - zs[0]);   // no finite score: equal
            sum += ex[j];
        }
        for (int j = 0; j < k; ++j) {
            sel_out[t * k + j] = es[j];
            wts[t * k + j] = ex[j] / sum;
            lsel[t * k + j] = es[j];
        }
    }
    for (int i = tid; i < nchunk * E; i += kRouteThreads) cnt[i / E][i % E] = 0;
    __syncthreads();
    // per-chunk counts (one thread per chunk, so no atomics)
    if (tid < nchunk) {
        const int t1 = min(M, (tid + 1) * kRouteChunk);
        for (int t = tid * kRouteChunk; t < t1; ++t)
            for (int j = 0; j < k; ++j) cnt[tid][lsel[t * k + j]] += 1;
    }
    __syncthreads();
    if (tid < E) {
        int tot = 0;
        for (int c = 0; c < nchunk; ++c) tot += cnt[c][tid];
        loff[tid + 1] = tot;
    }
    __syncthreads();
    if (tid == 0) {
        loff[0] = 0;
        int used = 0;
        for (int e = 0; e < E; ++e) {
            used += loff[e + 1] > 0;
            loff[e + 1] += loff[e];
        }
        if (active) *active = used;
    }
    __syncthreads();
    // chunk counts -> chunk start positions inside each expert's range
    if (tid < E) {
        int base = loff[tid];
        for (int c = 0; c < nchunk; ++c) {
            const int n = cnt[c][tid];
            cnt[c][tid] = base;
            base += n;
        }
    }
    if (tid <= E) offs[tid] = loff[tid];
    __syncthreads();
    if (tid < nchunk) {
        const int t1 = min(M, (tid + 1) * kRouteChunk);
        for (int t = tid * kRouteChunk; t < t1; ++t)
            for (int j = 0; j < k; ++j) {
                const int pos = cnt[tid][lsel[t * k + j]]++;
                perm[pos] = t * k + j;
                inv[t * k + j] = pos;
            }
    }
}

// ---- grouped matmul -------------------------------------------------------------
// out[row, n] = sum_c act[src(row), c] * W_e[n, c] for the rows row of expert
// e (offs[e] .. offs[e+1]); src(row) = perm[row] / top_k (gather of the
// positions' activations) when `gather`, else row.  W_e = W + e * wstride, in
// the tiled layout.  Epilogue: SiLU + bf16 (up) or fp32 store (down).
template <int EPI>
__global__ __launch_bounds__(kGroupWaves * kWave) void moe_grouped_kernel(
    const uint16_t* __restrict__ W, size_t wstride, int N, int K, const uint16_t* __restrict__ act,
    const int32_t* __restrict__ perm, int gather, int top_k, const int32_t* __restrict__ offs,
    void* __restrict__ out) {
    constexpr int MF = 4, U = kGroupSteps;
    const int nfrag = (N + 15) / 16;
    const int e = blockIdx.x / nfrag;
    const int frag = blockIdx.x % nfrag;
    const int row0 = offs[e];
    const int rows = offs[e + 1] - row0;
    if (rows <= 0) return;                 // an idle expert reads nothing

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15, g = lane >> 4;
    const int S = K / 32;
    const int s0 = S * wave / kGroupWaves, s1 = S * (wave + 1) / kGroupWaves;
    const uint16_t* wrow = W + (size_t)e * wstride + ((size_t)frag * S) * 512 + lane * 8;
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    __shared__ float red[kGroupWaves][MF][4][kWave];

    for (int pass = 0; pass < rows; pass += 16 * MF) {
        const uint16_t* arow[MF];
        bool aval[MF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
            const int j = pass + mf * 16 + r16;
            aval[mf] = j < rows;
            const int rr = row0 + (aval[mf] ? j : 0);
            const int src = gather ? perm[rr] / top_k : rr;
            arow[mf] = act + (size_t)src * K + 8 * g;
        }
        f32x4v acc[MF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) acc[mf] = f32x4v{0.f, 0.f, 0.f, 0.f};
        bf16x8 wa[U], wb[U], xa[U][MF], xb[U][MF];
        auto load = [&](bf16x8 (&w)[U], bf16x8 (&x)[U][MF], int s) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ss = s + u;
                const bool in = ss < s1;
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    x[u][mf] = (in && aval[mf]) ? *reinterpret_cast<const bf16x8*>(arow[mf] + 32 * ss)
                                                : zero8;
                w[u] = in ? __builtin_nontemporal_load(
                                reinterpret_cast<const bf16x8*>(wrow + (size_t)512 * ss))
                          : zero8;
            }
        };
        auto compute = [&](const bf16x8 (&w)[U], const bf16x8 (&x)[U][MF]) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[u], x[u][mf], acc[mf], 0, 0, 0);
        };
        load(wa, xa, s0);
        for (int s = s0; s < s1; s += 2 * U) {
            load(wb, xb, s + U);
            compute(wa, xa);
            load(wa, xa, s + 2 * U);
            compute(wb, xb);
        }
        if (pass) __syncthreads();         // the previous pass's readers are done
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][mf][r][lane] = acc[mf][r];
        __syncthreads();
        for (int i = threadIdx.x; i < 256 * MF; i += kGroupWaves * kWave) {
            const int ii = i & 15, jj = (i >> 4) & 15, mf = i >> 8;
            const int n = frag * 16 + ii;
            const int j = pass + mf * 16 + jj;
            if (n >= N || j >= rows) continue;
            const int r = ii & 3, l = ((ii >> 2) << 4) + jj;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < kGroupWaves; ++w) v += red[w][mf][r][l];
            const size_t o = (size_t)(row0 + j) * N + n;
            if constexpr (EPI == kEpiSilu)
                static_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(silu(v));
            else
                static_cast<float*>(out)[o] = v;
        }
    }
}

// h[t] += sum_j wts[t, j] * Y[inv[t * k + j]]   (slots in rank order)
__global__ __launch_bounds__(256) void moe_combine_kernel(
    float* __restrict__ h, const float* __restrict__ Y, const float* __restrict__ wts,
    const int32_t* __restrict__ inv, int M, int d, int k) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;   // (t, 4-column group)
    const int d4 = d / 4;
    if (i >= (long long)M * d4) return;
    const int t = (int)(i / d4), c = (int)(i % d4);
    f32x4v acc = *reinterpret_cast<const f32x4v*>(h + (size_t)t * d + 4 * c);
    f32x4v y = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j)
        y += wts[t * k + j] * *reinterpret_cast<const f32x4v*>(Y + (size_t)inv[t * k + j] * d + 4 * c);
    *reinterpret_cast<f32x4v*>(h + (size_t)t * d + 4 * c) = acc + y;
}

// ---- host plan --------------------------------------------------------------
constexpr size_t kAlign = 256;
size_t aup(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct MoePlan {
    int head_kind = kMfmaSkinny;
    size_t off_h, off_a, off_z, off_sel, off_w, off_offs, off_perm, off_inv, off_s, off_y, bytes;
};

MoePlan plan_moe(const sv_moe_desc& d, int M) {
    MoePlan p{};
    const size_t Mk = (size_t)M * d.top_k;
    p.head_kind = M >= 65 ? kMfmaTiled : kMfmaSkinny;
    const size_t arows = (size_t)(M + 15) / 16 * 16;
    size_t o = 0;
    p.off_h = o; o = aup(o + (size_t)M * d.d * 4);
    p.off_a = o; o = aup(o + arows * d.d * 2);
    p.off_z = o; o = aup(o + (size_t)M * d.n_experts * 4);
    p.off_sel = o; o = aup(o + Mk * 4);
    p.off_w = o; o = aup(o + Mk * 4);
    p.off_offs = o; o = aup(o + (size_t)(d.n_experts + 1) * 4);
    p.off_perm = o; o = aup(o + Mk * 4);
    p.off_inv = o; o = aup(o + Mk * 4);
    p.off_s = o; o = aup(o + Mk * d.ffn * 2);
    p.off_y = o; o = aup(o + Mk * d.d * 4);
    p.bytes = o;
    return p;
}

int moe_hip_fail(hipError_t e, const char* what) {
    return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

int sv_moe_create(const sv_moe_desc* desc, sv_moe** out) {
    if (!out) return fail(SV_ERR_INVALID_ARG, "moe_create: null output");
    *out = nullptr;
    if (!desc) return fail(SV_ERR_INVALID_ARG, "moe_create: null description");
    const sv_moe_desc& d = *desc;
    if (d.d < 64 || d.d % 64 || d.d > 32768 || d.ffn < 32 || d.ffn % 32 || d.vocab < 1 ||
        d.n_layers < 0)
        return fail(SV_ERR_INVALID_ARG,
                    "moe_create: need d a multiple of 64 (<= 32768), ffn a multiple of 32, vocab >= 1");
    if (d.n_experts < 1 || d.n_experts > kMoeMaxExperts || d.top_k < 1 || d.top_k > kMoeMaxTopK ||
        d.top_k > d.n_experts)
        return fail(SV_ERR_UNSUPPORTED, "moe_create: need 1 <= top_k <= min(8, n_experts) <= 256");
    if (!isfinite(d.rms_eps) || d.rms_eps < 0.f)
        return fail(SV_ERR_INVALID_ARG, "moe_create: rms_eps must be finite and >= 0");
    if (!d.gain || !d.w_head || (d.n_layers > 0 && (!d.w_router || !d.w_up || !d.w_down)))
        return fail(SV_ERR_INVALID_ARG, "moe_create: null weight pointer");
    sv_moe* m = new (std::nothrow) sv_moe;
    if (!m) return fail(SV_ERR_INVALID_ARG, "moe_create: out of host memory");
    m->desc = d;
    *out = m;
    return SV_OK;
}

void sv_moe_destroy(sv_moe* model) { delete model; }

size_t spec_verify_moe_workspace_bytes(const sv_moe* model, int32_t M) {
    if (!model || M < 0 || M > kMoeMaxRows) return 0;
    return plan_moe(model->desc, M).bytes;
}

int spec_verify_moe_forward(const sv_moe* model, const float* hidden, int32_t M, float* logits,
                            int32_t* active_experts, void* ws, size_t ws_bytes, hipStream_t s) {
    if (!model) return fail(SV_ERR_INVALID_ARG, "moe_forward: null model");
    if (M < 0 || M > kMoeMaxRows)
        return fail(SV_ERR_UNSUPPORTED, "moe_forward: M = %d outside 0 .. %d", M, kMoeMaxRows);
    if (M == 0) return SV_OK;
    if (!hidden || !logits) return fail(SV_ERR_INVALID_ARG, "moe_forward: null input or output");
    const sv_moe_desc& d = model->desc;
    const MoePlan p = plan_moe(d, M);
    if (!ws || ws_bytes < p.bytes)
        return fail(SV_ERR_WORKSPACE, "moe_forward: workspace of %zu bytes needed, %zu given",
                    p.bytes, ws_bytes);
    char* w = static_cast<char*>(ws);
    float* h = reinterpret_cast<float*>(w + p.off_h);
    void* a = w + p.off_a;
    float* z = reinterpret_cast<float*>(w + p.off_z);
    int32_t* sel = reinterpret_cast<int32_t*>(w + p.off_sel);
    float* wts = reinterpret_cast<float*>(w + p.off_w);
    int32_t* offs = reinterpret_cast<int32_t*>(w + p.off_offs);
    int32_t* perm = reinterpret_cast<int32_t*>(w + p.off_perm);
    int32_t* inv = reinterpret_cast<int32_t*>(w + p.off_inv);
    void* S = w + p.off_s;
    float* Y = reinterpret_cast<float*>(w + p.off_y);
    const int E = d.n_experts, k = d.top_k;
    const size_t router_stride = tiled_elems(E, d.d);
    const size_t up_stride = tiled_elems(d.ffn, d.d);
    const size_t down_stride = tiled_elems(d.d, d.ffn);
    hipError_t e;

    e = launch_rmsnorm(hidden, h, nullptr, 0, d.gain, a, M, d.d, d.rms_eps, 1, 0, s);
    if (e != hipSuccess) return moe_hip_fail(e, "rmsnorm launch");
    for (int l = 0; l < d.n_layers; ++l) {
        MatmulArgs r{};
        r.W = static_cast<const uint16_t*>(d.w_router) + (size_t)l * router_stride;
        r.act = a;
        r.M = M; r.N = E; r.K = d.d;
        r.epi = kEpiStore; r.out = z; r.bf16 = 1; r.tiled = 1;
        r.name = "moe_router";
        e = launch_matmul(r, kMfmaSkinny, s);
        if (e != hipSuccess) return moe_hip_fail(e, "router launch");
        {
            ProfScope prof("moe_route", s, (double)M * E * 4, 0.0);
            SV_LAUNCH(prof, moe_route_kernel, 1, kRouteThreads, s, z, M, E, k, sel, wts, offs, perm,
                      inv, active_experts ? active_experts + l : nullptr);
            e = hipGetLastError();
            if (e != hipSuccess) return moe_hip_fail(e, "route launch");
        }
        {
            // bytes depend on the experts the device picks: counted by the caller
            ProfScope prof("moe_up_silu", s, 0.0, 2.0 * M * k * (double)d.ffn * d.d);
            const unsigned grid = (unsigned)(E * ((d.ffn + 15) / 16));
            SV_LAUNCH(prof, moe_grouped_kernel<kEpiSilu>, grid, kGroupWaves * kWave, s,
                      static_cast<const uint16_t*>(d.w_up) + (size_t)l * E * up_stride, up_stride,
                      d.ffn, d.d, static_cast<const uint16_t*>(a), perm, 1, k, offs, S);
            e = hipGetLastError();
            if (e != hipSuccess) return moe_hip_fail(e, "grouped up launch");
        }
        {
            ProfScope prof("moe_down", s, 0.0, 2.0 * M * k * (double)d.ffn * d.d);
            const unsigned grid = (unsigned)(E * ((d.d + 15) / 16));
            SV_LAUNCH(prof, moe_grouped_kernel<kEpiStore>, grid, kGroupWaves * kWave, s,
                      static_cast<const uint16_t*>(d.w_down) + (size_t)l * E * down_stride,
                      down_stride, d.d, d.ffn, static_cast<const uint16_t*>(S), perm, 0, k, offs, Y);
            e = hipGetLastError();
            if (e != hipSuccess) return moe_hip_fail(e, "grouped down launch");
        }
        {
            ProfScope prof("moe_combine", s, (double)M * d.d * (8.0 + 4.0 * k), 0.0);
            const long long n = (long long)M * (d.d / 4);
            SV_LAUNCH(prof, moe_combine_kernel, (unsigned)((n + 255) / 256), 256, s, h, Y, wts, inv,
                      M, d.d, k);
            e = hipGetLastError();
            if (e != hipSuccess) return moe_hip_fail(e, "combine launch");
        }
        e = launch_rmsnorm(h, h, nullptr, 0, d.gain + (size_t)(l + 1) * d.d, a, M, d.d, d.rms_eps, 1,
                           l + 1 == d.n_layers && p.head_kind == kMfmaTiled, s);
        if (e != hipSuccess) return moe_hip_fail(e, "rmsnorm launch");
    }
    if (d.n_layers == 0 && p.head_kind == kMfmaTiled) {
        e = launch_rmsnorm(h, h, nullptr, 0, d.gain, a, M, d.d, d.rms_eps, 1, 1, s);
        if (e != hipSuccess) return moe_hip_fail(e, "rmsnorm launch");
    }
    MatmulArgs hd{};
    hd.W = d.w_head;
    hd.act = a;
    hd.M = M; hd.N = d.vocab; hd.K = d.d;
    hd.epi = kEpiStore; hd.out = logits; hd.bf16 = 1; hd.tiled = 1;
    hd.act_tiled = p.head_kind == kMfmaTiled;
    e = launch_matmul(hd, p.head_kind, s);
    if (e != hipSuccess) return moe_hip_fail(e, "LM-head launch");
    return SV_OK;
}

}  // extern "C"
