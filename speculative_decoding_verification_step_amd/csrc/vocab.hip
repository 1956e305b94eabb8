// Vocabulary stage of the verification step: softmax statistics, the accept
// scan, and the replacement / bonus draw.
//
// Rule (publishertech section 2 "Modified Rejection Sampling"; mohashari
// "Speculative Decoding Mechanics"; klu.ai "Mathematical Guarantee"): for
// draft positions j = 1..K in order accept x_j iff u_j <= p_j(x_j) / q_j(x_j);
// at the first rejection j* emit one token from max(0, p_j* - q_j*)
// (normalised); if all K are accepted emit one token from p_{K+1}.  At
// temperature 0 the draft is accepted iff it equals the target's argmax and
// the target's argmax is emitted (NVIDIA co-design post, "What is
// speculative decoding?").
//
// Probabilities are fp32: p(y) = exp((z_y - max z) / T) * (1 / sum), computed
// by the same code for target and draft rows, so identical rows give
// bit-identical p and q.  A draw over weights w (ascending token ids) picks
// the smallest y whose running sum exceeds u' * sum(w).
//
// Three launches, all parallel over (request, chunk of kChunk logits):
//   row_stats     per (row, chunk): (max, sum of exp) or (max, argmax), all of
//                 a thread's loads in flight at once;
//   decide_chunk  per (request, chunk): folds the chunk pairs of the rows it
//                 needs (in chunk order), takes the request's accept decisions
//                 (every chunk block of a request reaches the same ones), and
//                 sums the weights of the draw row over its chunk;
//   draw          per request: prefix over the chunk sums, then rescans only
//                 the chunk that holds u' * R.
// Within a chunk a draw scan takes kPasses passes of kPassIds ids; in each,
// thread t owns the run of 4 consecutive ids at 4t.  The running sum C_y is
// prefix(chunk) + (earlier passes' totals + (exclusive(thread) + running sum
// within the run)), and the chunk total is its value at the chunk's last id,
// computed by the same code in both kernels, so the chunk that holds the
// threshold always contains the drawn token.
#include <float.h>
#include <limits.h>
#include <stdlib.h>

#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

constexpr int kStatsThreads = 256;
constexpr int kChunk = 8192;                       // logits per chunk workgroup
constexpr int kPerThread = kChunk / kStatsThreads; // 32 = 8 float4
constexpr int kDrawThreads = kStatsThreads;
constexpr int kPassIds = 4 * kDrawThreads;         // ids per pass of a draw scan: a float4 per thread
constexpr int kPasses = kChunk / kPassIds;         // 8 passes per chunk
constexpr int kScanShared = kPasses * (kDrawThreads / kWave + 1);   // floats of LDS per scan
constexpr int kMeta = 8;                           // per-request words passed to the draw
// chunk workgroups from which the decisions are taken once per request: the
// stage at B = 256, V = 128256 (4096 chunk workgroups) 199-201 -> 192-193 us;
// at 128 (B = 8) and 4 (B = 1) workgroups the extra launch costs 1.4-1.7 us
constexpr long long kSplitMinGroups = 1024;
// statistics reads above the last-level cache's size take non-temporal loads
constexpr double kStreamStatsBytes = 256.0 * 1024 * 1024;

// exp(x) on the transcendental unit: v_exp_f32(x * log2(e)).  Relative error
// about 2^-24 * |x * log2(e)| + 1 ulp, far inside the 1e-5 decision band for
// the exponents a softmax sees; the same function serves target and draft rows.
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ float prob(float z, float m, float inv_t, float inv_s) {
    return fast_exp((z - m) * inv_t) * inv_s;
}

// (max, sum of exp((z - max) / T)) pairs, combined in a fixed order.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2, float inv_t) {
    if (m2 == -INFINITY) return;
    if (m == -INFINITY) {
        m = m2;
        s = s2;
        return;
    }
    const float mx = fmaxf(m, m2);
    s = s * fast_exp((m - mx) * inv_t) + s2 * fast_exp((m2 - mx) * inv_t);
    m = mx;
}

// Better (value, index): larger value, then smaller index.
__device__ __forceinline__ void arg_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// `copy` (optional): the target rows are also written to copy + row *
// copy_stride (a row of a larger array), from the registers they were read into.
// kStream: non-temporal loads, for rows too large to stay in the last-level
// cache (the draw's later re-read of a few rows then misses it anyway).
template <bool kStream>
__global__ __launch_bounds__(kStatsThreads) void row_stats_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int n_t, int V,
    int nchunk, float inv_t, int greedy, int vec4, float* __restrict__ pv,
    float* __restrict__ ps, int* __restrict__ pi, float* __restrict__ copy, size_t copy_stride) {
    const int row = blockIdx.x / nchunk;
    const int chunk = blockIdx.x - row * nchunk;
    const int tid = threadIdx.x;
    const float* z = row < n_t ? target + (size_t)row * V : draft + (size_t)(row - n_t) * V;
    const int base = chunk * kChunk;

    float x[kPerThread];
    int idx0[kPerThread / 4];
    if (vec4) {
#pragma unroll
        for (int v = 0; v < kPerThread / 4; ++v) {
            const int e = base + 4 * (tid + v * kStatsThreads);
            idx0[v] = e;
            f32x4 q = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (e < V) {                                             // V % 4 == 0 here
                const f32x4* a = reinterpret_cast<const f32x4*>(z + e);
                q = kStream ? __builtin_nontemporal_load(a) : *a;
            }
            x[4 * v] = q.x;
            x[4 * v + 1] = q.y;
            x[4 * v + 2] = q.z;
            x[4 * v + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int v = 0; v < kPerThread / 4; ++v) {
            const int e = base + 4 * (tid + v * kStatsThreads);
            idx0[v] = e;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * v + i] = (e + i < V) ? z[e + i] : -INFINITY;
        }
    }

    if (copy && row < n_t) {
        float* dst = copy + (size_t)row * copy_stride;
#pragma unroll
        for (int v = 0; v < kPerThread / 4; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (idx0[v] + i < V) dst[idx0[v] + i] = x[4 * v + i];
    }

    __shared__ float sh_v[kStatsThreads / kWave];
    __shared__ float sh_s[kStatsThreads / kWave];
    __shared__ int sh_i[kStatsThreads / kWave];
    if (greedy) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int v = 0; v < kPerThread / 4; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (idx0[v] + i < V) arg_merge(bv, bi, x[4 * v + i], idx0[v] + i);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            arg_merge(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
        if ((tid & (kWave - 1)) == 0) {
            sh_v[tid / kWave] = bv;
            sh_i[tid / kWave] = bi;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kStatsThreads / kWave; ++w) arg_merge(bv, bi, sh_v[w], sh_i[w]);
            pv[blockIdx.x] = bv;
            pi[blockIdx.x] = bi;
        }
        return;
    }

    // the thread's pair: its maximum, then the sum of exp((x - m) / T) in
    // element order -- no data-dependent branch per element, half the exps of
    // an online update (large batch: stage 194 -> 188 us; 70B share: this
    // kernel 12.4 -> 8.5 us; 8B shape 4.7 -> 3.9 us)
    float m = x[0], s = 0.f;
#pragma unroll
    for (int i = 1; i < kPerThread; ++i) m = fmaxf(m, x[i]);
    if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) s += fast_exp((x[i] - m) * inv_t);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave);
        const float s2 = __shfl_xor(s, o, kWave);
        lse_merge(m, s, m2, s2, inv_t);
    }
    if ((tid & (kWave - 1)) == 0) {
        sh_v[tid / kWave] = m;
        sh_s[tid / kWave] = s;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kStatsThreads / kWave; ++w) lse_merge(m, s, sh_v[w], sh_s[w], inv_t);
        pv[blockIdx.x] = m;
        ps[blockIdx.x] = s;
    }
}

// Row statistics folded from the per-chunk pairs by one whole wave: lane l
// folds chunks l, l+64, ... in order (all loads in flight together), then the
// lanes are combined by a butterfly.  Both combinations are symmetric, so every
// lane ends with the same bits, and every caller of a row gets the same ones.
__device__ __forceinline__ void wave_row_lse(const float* pv, const float* ps, size_t row,
                                             int nchunk, float inv_t, float& m, float& s) {
    const int lane = threadIdx.x & (kWave - 1);
    m = -INFINITY;
    s = 0.f;
    for (int c = lane; c < nchunk; c += kWave)
        lse_merge(m, s, pv[row * nchunk + c], ps[row * nchunk + c], inv_t);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float m2 = __shfl_xor(m, o, kWave);
        const float s2 = __shfl_xor(s, o, kWave);
        lse_merge(m, s, m2, s2, inv_t);
    }
}

__device__ __forceinline__ int wave_row_argmax(const float* pv, const int* pi, size_t row,
                                               int nchunk) {
    const int lane = threadIdx.x & (kWave - 1);
    float v = -INFINITY;
    int i = INT_MAX;
    for (int c = lane; c < nchunk; c += kWave) arg_merge(v, i, pv[row * nchunk + c], pi[row * nchunk + c]);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1)
        arg_merge(v, i, __shfl_xor(v, o, kWave), __shfl_xor(i, o, kWave));
    return i == INT_MAX ? 0 : i;
}

// Weights of a draw: the residual max(0, p - q), or p alone (zd == nullptr).
struct DrawRows {
    const float* zt;
    const float* zd;
    float mt, it_s, md, id_s, inv_t;
};

__device__ __forceinline__ float weight(const DrawRows& dr, int y) {
    const float p = prob(dr.zt[y], dr.mt, dr.inv_t, dr.it_s);
    if (!dr.zd) return p;
    return fmaxf(0.f, p - prob(dr.zd[y], dr.md, dr.inv_t, dr.id_s));
}

// Draw weights of chunk c in kPasses passes of kPassIds ids.  In pass p,
// thread t owns the run of 4 ids c * kChunk + p * kPassIds + 4t .. +3 (zero
// past V), so the lanes of a load are 16 B apart and every line a wave
// touches is read once.  run[p][i] holds the running sum over the run.
// kStream: non-temporal loads (rows that no later kernel re-reads soon).
template <bool kStream = false>
__device__ __forceinline__ void pass_runs(const DrawRows& dr, int c, int V,
                                          float run[kPasses][4]) {
    auto ld = [](const float* a) {
        const f32x4* p4 = reinterpret_cast<const f32x4*>(a);
        return kStream ? __builtin_nontemporal_load(p4) : *p4;
    };
    const int y0 = c * kChunk + 4 * (int)threadIdx.x;
    float w[kPasses][4];
    const bool vec = (V % 4 == 0) && ((uintptr_t)dr.zt % 16 == 0) &&
                     (!dr.zd || (uintptr_t)dr.zd % 16 == 0);
    if (vec) {
        // V % 4 == 0: a run is wholly inside the row or wholly past it.  Runs
        // past it load the row's last four values (no branch around the
        // loads) and weigh zero.
        f32x4 zt[kPasses], zd4[kPasses];
        if (dr.zd) {
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int y = min(y0 + p * kPassIds, V - 4);
                zt[p] = ld(dr.zt + y);
                zd4[p] = ld(dr.zd + y);
            }
        } else {
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                zt[p] = ld(dr.zt + min(y0 + p * kPassIds, V - 4));
                zd4[p] = zt[p];
            }
        }
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const bool in = y0 + p * kPassIds < V;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pt = prob(zt[p][i], dr.mt, dr.inv_t, dr.it_s);
                const float wi = dr.zd ? fmaxf(0.f, pt - prob(zd4[p][i], dr.md, dr.inv_t, dr.id_s)) : pt;
                w[p][i] = in ? wi : 0.f;
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int y = y0 + p * kPassIds + i;
                w[p][i] = y < V ? weight(dr, y) : 0.f;
            }
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s += w[p][i];
            run[p][i] = s;
        }
    }
}

// Per pass: the exclusive prefix ex[p] of the run totals over the
// workgroup's threads (inclusive scan in lane order within a wave, then the
// totals of the earlier waves added in wave order) and the pass total tot[p],
// defined as the last thread's exclusive prefix plus its own run total.
// `sh` holds kScanShared floats: the wave totals of pass p at 4p..4p+3, the
// pass totals after them.
__device__ __forceinline__ void pass_scan(const float run[kPasses][4], float* sh,
                                          float ex[kPasses], float tot[kPasses]) {
    static_assert(kDrawThreads / kWave == 4, "four wave totals per pass");
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    float incl[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) incl[p] = run[p][3];
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1)
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const float t = __shfl_up(incl[p], o, kWave);
            if (lane >= o) incl[p] += t;
        }
    float excl[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        excl[p] = __shfl_up(incl[p], 1, kWave);
        if (lane == 0) excl[p] = 0.f;
        if (lane == kWave - 1) sh[4 * p + wave] = incl[p];
    }
    __syncthreads();
    f32x4 wt[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) wt[p] = *reinterpret_cast<const f32x4*>(sh + 4 * p);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float base = 0.f;
        if (wave > 0) base += wt[p][0];
        if (wave > 1) base += wt[p][1];
        if (wave > 2) base += wt[p][2];
        ex[p] = base + excl[p];
        if (tid == kDrawThreads - 1) sh[4 * kPasses + p] = ex[p] + run[p][3];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kPasses; ++p) tot[p] = sh[4 * kPasses + p];
    __syncthreads();
}

// Chunk total of the draw weights: the pass totals added in pass order from
// zero (the same arithmetic as the draw's rescan, whose last prefix it is).
template <bool kStream = false>
__device__ __forceinline__ float chunk_total(const DrawRows& dr, int c, int V, float* sh) {
    float run[kPasses][4], ex[kPasses], tot[kPasses];
    pass_runs<kStream>(dr, c, V, run);
    pass_scan(run, sh, ex, tot);
    float total = 0.f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) total += tot[p];
    return total;
}

// Decisions of request b, taken by every workgroup that works on b.  Returns
// the first rejected position (1..K) or K + 1; -1 if a draft token is out of
// range.  The wave of position j0 also reports p(x), q(x) when `report`.
__device__ int decide(const float* target, const float* draft, const int32_t* tokens, int b, int K,
                      int V, int nchunk, float inv_t, int greedy, uint32_t k0, uint32_t k1,
                      uint32_t step, size_t n_t, const float* pv, const float* ps, const int* pi,
                      bool report, float* p_at, float* q_at, int* sh_first, int* sh_bad) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        *sh_first = K + 1;
        *sh_bad = 0;
    }
    __syncthreads();
    const size_t trow0 = (size_t)b * (K + 1);
    const int lane = tid & (kWave - 1);
    // one wave per draft position (the whole wave folds the row statistics)
    for (int j0 = tid / kWave; j0 < K; j0 += kDrawThreads / kWave) {
        const int x = tokens[(size_t)b * K + j0];
        if (x < 0 || x >= V) {
            if (lane == 0) atomicOr(sh_bad, 1);
            continue;
        }
        const size_t rt = trow0 + j0;
        bool ok;
        float p, q;
        if (greedy) {
            ok = (x == wave_row_argmax(pv, pi, rt, nchunk));
            p = ok ? 1.f : 0.f;
            q = 1.f;
        } else {
            const size_t rd = (size_t)b * K + j0;
            float mt, st, md, sd;
            wave_row_lse(pv, ps, rt, nchunk, inv_t, mt, st);
            wave_row_lse(pv, ps, n_t + rd, nchunk, inv_t, md, sd);
            p = prob(target[rt * V + x], mt, inv_t, 1.0f / st);
            q = prob(draft[rd * V + x], md, inv_t, 1.0f / sd);
            const float u = u_accept(philox_word0((uint32_t)b, (uint32_t)(j0 + 1), 0u, step, k0, k1));
            ok = (u <= p / q);      // q == 0: +inf (accept) or NaN (p == 0: reject)
        }
        if (lane == 0) {
            if (report) {
                if (p_at) p_at[(size_t)b * K + j0] = p;
                if (q_at) q_at[(size_t)b * K + j0] = q;
            }
            if (!ok) atomicMin(sh_first, j0 + 1);
        }
    }
    __syncthreads();
    const int r = *sh_bad ? -1 : *sh_first;
    __syncthreads();
    return r;
}

__device__ __forceinline__ void write_outputs(int32_t* out, int32_t* accept_len,
                                              const int32_t* tokens, int b, int K, int js,
                                              int tok, int out_stride) {
    int32_t* ob = out + (size_t)b * out_stride;
    for (int y = threadIdx.x; y <= K; y += kDrawThreads) {
        int32_t v = -1;
        if (js > 0) {
            if (y < js - 1) v = tokens[(size_t)b * K + y];
            else if (y == js - 1) v = tok;
        }
        ob[y] = v;
    }
    if (threadIdx.x == 0 && accept_len) accept_len[b] = js > 0 ? js : 0;
}

__global__ __launch_bounds__(kDrawThreads) void decide_chunk_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, int K, int V, int nchunk, float inv_t, int greedy,
    uint32_t k0, uint32_t k1, uint32_t step, const float* __restrict__ pv,
    const float* __restrict__ ps, const int* __restrict__ pi, float* __restrict__ ctot,
    float* __restrict__ meta, int32_t* __restrict__ out, int32_t* __restrict__ accept_len,
    float* __restrict__ p_at, float* __restrict__ q_at, int B, int out_stride) {
    const int b = blockIdx.x / nchunk;
    const int c = blockIdx.x - b * nchunk;
    __shared__ int sh_first, sh_bad;
    __shared__ __align__(16) float sh[kScanShared];
    __shared__ float sh_stat[4];
    const size_t n_t = (size_t)B * (K + 1);
    const int js = decide(target, draft, tokens, b, K, V, nchunk, inv_t, greedy, k0, k1, step, n_t,
                          pv, ps, pi, c == 0, p_at, q_at, &sh_first, &sh_bad);
    if (js < 0 || greedy) {
        // nothing to draw: the first chunk's workgroup writes the request
        if (c == 0) {
            const int tok = js < 0 ? -1 : wave_row_argmax(pv, pi, (size_t)b * (K + 1) + js - 1, nchunk);
            write_outputs(out, accept_len, tokens, b, K, js, tok, out_stride);
            if (threadIdx.x == 0) meta[(size_t)b * kMeta] = __int_as_float(0);
        }
        return;
    }
    const size_t rt = (size_t)b * (K + 1) + js - 1;
    const bool resid = js <= K;
    const size_t rd = (size_t)b * K + js - 1;
    if (threadIdx.x < kWave) {
        float m, s;
        wave_row_lse(pv, ps, rt, nchunk, inv_t, m, s);
        float m2 = 0.f, s2 = 1.f;
        if (resid) wave_row_lse(pv, ps, n_t + rd, nchunk, inv_t, m2, s2);
        if (threadIdx.x == 0) {
            sh_stat[0] = m;
            sh_stat[1] = 1.0f / s;
            sh_stat[2] = resid ? m2 : 0.f;
            sh_stat[3] = resid ? 1.0f / s2 : 0.f;
        }
    }
    __syncthreads();
    DrawRows dr;
    dr.zt = target + rt * V;
    dr.zd = resid ? draft + rd * V : nullptr;
    dr.mt = sh_stat[0];
    dr.it_s = sh_stat[1];
    dr.md = sh_stat[2];
    dr.id_s = sh_stat[3];
    dr.inv_t = inv_t;
    const float tot = chunk_total(dr, c, V, sh);
    if (threadIdx.x == 0) {
        ctot[(size_t)b * nchunk + c] = tot;
        if (c == 0) {
            float* mb = meta + (size_t)b * kMeta;
            mb[0] = __int_as_float(js);
            mb[1] = dr.mt;
            mb[2] = dr.it_s;
            mb[3] = dr.md;
            mb[4] = dr.id_s;
        }
    }
}

// The same stage in two launches, for batches with many chunk workgroups
// and for T = 0 (nothing to draw): decide_kernel takes each request's
// decisions once (one workgroup per request) and leaves the draw parameters
// in `meta`; chunk_total_kernel then only reads them and its chunk, where
// decide_chunk_kernel repeats the decisions in every chunk workgroup.  Both
// forms run the same functions on the same values, so their outputs are
// bit-identical.
__global__ __launch_bounds__(kDrawThreads) void decide_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, int K, int V, int nchunk, float inv_t, int greedy,
    uint32_t k0, uint32_t k1, uint32_t step, const float* __restrict__ pv,
    const float* __restrict__ ps, const int* __restrict__ pi, float* __restrict__ meta,
    int32_t* __restrict__ out, int32_t* __restrict__ accept_len, float* __restrict__ p_at,
    float* __restrict__ q_at, int B, int out_stride) {
    const int b = blockIdx.x;
    __shared__ int sh_first, sh_bad;
    const size_t n_t = (size_t)B * (K + 1);
    const int js = decide(target, draft, tokens, b, K, V, nchunk, inv_t, greedy, k0, k1, step, n_t,
                          pv, ps, pi, true, p_at, q_at, &sh_first, &sh_bad);
    float* mb = meta + (size_t)b * kMeta;
    if (js < 0 || greedy) {
        const int tok = js < 0 ? -1 : wave_row_argmax(pv, pi, (size_t)b * (K + 1) + js - 1, nchunk);
        write_outputs(out, accept_len, tokens, b, K, js, tok, out_stride);
        if (threadIdx.x == 0) mb[0] = __int_as_float(0);
        return;
    }
    if (threadIdx.x < kWave) {
        const size_t rt = (size_t)b * (K + 1) + js - 1;
        const bool resid = js <= K;
        const size_t rd = (size_t)b * K + js - 1;
        float m, s;
        wave_row_lse(pv, ps, rt, nchunk, inv_t, m, s);
        float m2 = 0.f, s2 = 1.f;
        if (resid) wave_row_lse(pv, ps, n_t + rd, nchunk, inv_t, m2, s2);
        if (threadIdx.x == 0) {
            mb[0] = __int_as_float(js);
            mb[1] = m;
            mb[2] = 1.0f / s;
            mb[3] = resid ? m2 : 0.f;
            mb[4] = resid ? 1.0f / s2 : 0.f;
        }
    }
}

__global__ __launch_bounds__(kDrawThreads) void chunk_total_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int K, int V, int nchunk,
    float inv_t, const float* __restrict__ meta, float* __restrict__ ctot) {
    const int b = blockIdx.x / nchunk;
    const int c = blockIdx.x - b * nchunk;
    const float* mb = meta + (size_t)b * kMeta;
    const int js = __float_as_int(mb[0]);
    if (js <= 0) return;                       // no draw for this request
    __shared__ __align__(16) float sh[kScanShared];
    const bool resid = js <= K;
    DrawRows dr;
    dr.zt = target + ((size_t)b * (K + 1) + js - 1) * V;
    dr.zd = resid ? draft + ((size_t)b * K + js - 1) * V : nullptr;
    dr.mt = mb[1];
    dr.it_s = mb[2];
    dr.md = mb[3];
    dr.id_s = mb[4];
    dr.inv_t = inv_t;
    // the split form runs at large batches, whose rows the draw mostly does not
    // re-read: chunk totals 37.3 -> 34.5 us on the 768-row workload
    const float tot = chunk_total<true>(dr, c, V, sh);
    if (threadIdx.x == 0) ctot[(size_t)b * nchunk + c] = tot;
}

// Smallest y of chunk c with prefix + C_y > t, -1 if none.  C_y, the
// cumulative weight of the chunk's ids up to y, is P_p + (ex[p] + run[p][i])
// for id y in pass p: P_p is the sum of the earlier passes' totals in pass
// order, ex and run as in pass_scan / pass_runs.  At the chunk's last id it
// is the chunk total.
__device__ int find_in_chunk(const DrawRows& dr, int c, int V, float prefix, float t, float* sh,
                             int* sh_hit) {
    float run[kPasses][4], ex[kPasses], tot[kPasses];
    pass_runs(dr, c, V, run);
    pass_scan(run, sh, ex, tot);
    if (threadIdx.x == 0) *sh_hit = INT_MAX;
    __syncthreads();
    const int y0 = c * kChunk + 4 * (int)threadIdx.x;
    int hit = INT_MAX;
    float P = 0.f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int y = y0 + p * kPassIds + i;
            if (y < V && prefix + (P + (ex[p] + run[p][i])) > t) hit = min(hit, y);
        }
        P += tot[p];
    }
    if (hit != INT_MAX) atomicMin(sh_hit, hit);
    __syncthreads();
    const int r = *sh_hit;
    __syncthreads();
    return r == INT_MAX ? -1 : r;
}

// The draw's uniform is word 0 of Philox at counter (b, js + pos_base,
// draw_id, step): (b, js, 1, step) for the replacement or bonus token of a
// verification, (b, slot, 2, step) for a token drawn from a draft row.
__global__ __launch_bounds__(kDrawThreads) void draw_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, int K, int V, int nchunk, float inv_t, uint32_t k0,
    uint32_t k1, uint32_t step, uint32_t draw_id, int pos_base, const float* __restrict__ ctot,
    const float* __restrict__ meta, int32_t* __restrict__ out, int32_t* __restrict__ accept_len,
    int out_stride) {
    const int b = blockIdx.x;
    const float* mb = meta + (size_t)b * kMeta;
    const int js = __float_as_int(mb[0]);
    if (js <= 0) return;                       // written by decide_chunk_kernel
    __shared__ __align__(16) float sh[kScanShared];
    __shared__ float sh_c[2];
    __shared__ int sh_i[2];
    const bool resid = js <= K;
    DrawRows dr;
    dr.zt = target + ((size_t)b * (K + 1) + js - 1) * V;
    dr.zd = resid ? draft + ((size_t)b * K + js - 1) * V : nullptr;
    dr.mt = mb[1];
    dr.it_s = mb[2];
    dr.md = mb[3];
    dr.id_s = mb[4];
    dr.inv_t = inv_t;
    const float u =
        u_resample(philox_word0((uint32_t)b, (uint32_t)(js + pos_base), draw_id, step, k0, k1));
    const float* ct = ctot + (size_t)b * nchunk;

    // R, the threshold and its chunk (thread 0, chunk order).  R == 0 after a
    // rejection (the residual mass rounded away) falls back to p; its chunk
    // sums are recomputed here.
    float R = 0.f;
    if (threadIdx.x == 0)
        for (int c = 0; c < nchunk; ++c) R += ct[c];
    if (threadIdx.x == 0) sh_c[0] = R;
    __syncthreads();
    R = sh_c[0];
    const bool fallback = !(R > 0.f);
    if (fallback) dr.zd = nullptr;

    int tok = -1;
    float pre = 0.f;
    int cstar = -1;
    if (threadIdx.x == 0) {
        sh_i[0] = -1;
        sh_c[1] = 0.f;
    }
    if (!fallback) {
        if (threadIdx.x == 0) {
            const float t = u * R;
            float p = 0.f;
            for (int c = 0; c < nchunk; ++c) {
                const float nxt = p + ct[c];
                if (nxt > t) {
                    sh_i[0] = c;
                    sh_c[1] = p;
                    break;
                }
                p = nxt;
            }
        }
        __syncthreads();
        cstar = sh_i[0];
        pre = sh_c[1];
        if (cstar >= 0) tok = find_in_chunk(dr, cstar, V, pre, u * R, sh, &sh_i[1]);
    } else {
        // draw from p: chunk totals of p, then the same search
        float p = 0.f, t = 0.f;
        float tots = 0.f;
        for (int c = 0; c < nchunk; ++c) tots += chunk_total(dr, c, V, sh);
        t = u * tots;
        for (int c = 0; c < nchunk && tok < 0; ++c) {
            const float ctc = chunk_total(dr, c, V, sh);
            if (p + ctc > t) tok = find_in_chunk(dr, c, V, p, t, sh, &sh_i[1]);
            p += ctc;
        }
    }
    if (tok < 0) {
        // u * R rounded up to R: the last token with positive weight
        int last = -1;
        for (int y = threadIdx.x; y < V; y += kDrawThreads)
            if (weight(dr, y) > 0.f) last = y;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
        if (threadIdx.x == 0) sh_i[1] = -1;
        __syncthreads();
        if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(&sh_i[1], last);
        __syncthreads();
        tok = sh_i[1] < 0 ? 0 : sh_i[1];
    }
    write_outputs(out, accept_len, tokens, b, K, js, tok, out_stride);
}

}  // namespace

int stats_chunks(int V) { return (V + kChunk - 1) / kChunk; }

size_t accept_meta_floats(int B, int V) { return (size_t)B * stats_chunks(V) + (size_t)B * kMeta; }

hipError_t launch_row_stats(const float* target, const float* draft, int n_t, int n_d, int V,
                            float inv_t, int greedy, float* pv, float* ps, int* pi,
                            hipStream_t stream, float* copy, size_t copy_stride) {
    const int rows = n_t + n_d;
    if (rows <= 0) return hipSuccess;
    const int nchunk = stats_chunks(V);
    const int vec4 = (V % 4 == 0) && ((uintptr_t)target % 16 == 0) &&
                     (draft == nullptr || (uintptr_t)draft % 16 == 0);
    const double copied = copy ? (double)n_t * V * 4.0 : 0.0;
    ProfScope prof("row_stats", stream, (double)rows * V * 4.0 + copied, 0.0);
    // beyond the 256 MiB last-level cache the rows stream past it: large batch
    // (657 MB) 117 -> 100 us; below it the draw's re-read of its rows hits the
    // cache (70B share, 37 MB: non-temporal loads cost the stage 1.5 us)
    if ((double)rows * V * 4.0 > kStreamStatsBytes)
        SV_LAUNCH(prof, row_stats_kernel<true>, rows * nchunk, kStatsThreads, stream, target,
                  draft, n_t, V, nchunk, inv_t, greedy, vec4, pv, ps, pi, copy, copy_stride);
    else
        SV_LAUNCH(prof, row_stats_kernel<false>, rows * nchunk, kStatsThreads, stream, target,
                  draft, n_t, V, nchunk, inv_t, greedy, vec4, pv, ps, pi, copy, copy_stride);
    return hipGetLastError();
}

hipError_t launch_accept(const float* target, const float* draft, const int32_t* tokens, int B,
                         int K, int V, float inv_t, int greedy, uint64_t seed, uint32_t step,
                         const float* pv, const float* ps, const int* pi, float* scratch,
                         int32_t* out_tokens, int32_t* accept_len, float* p_at, float* q_at,
                         hipStream_t stream) {
    if (B <= 0) return hipSuccess;
    const int nchunk = stats_chunks(V);
    const uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
    float* ctot = scratch;
    float* meta = scratch + (size_t)B * nchunk;
    // Decisions once per request (decide + chunk_total) when there are many
    // chunk workgroups or nothing to draw (T = 0), else in every chunk
    // workgroup (one launch).  SPEC_VERIFY_ACCEPT_SPLIT = 0 | 1 forces either
    // form (tests, measurements).
    bool split = greedy || (long long)B * nchunk >= kSplitMinGroups;
    if (const char* e = getenv("SPEC_VERIFY_ACCEPT_SPLIT")) split = atoi(e) != 0;
    if (split) {
        {
            ProfScope prof("decide", stream, 0.0, 0.0);
            SV_LAUNCH(prof, decide_kernel, B, kDrawThreads, stream, target, draft, tokens, K, V,
                      nchunk, inv_t, greedy, k0, k1, step, pv, ps, pi, meta, out_tokens,
                      accept_len, p_at, q_at, B, K + 1);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (!greedy) {
            // reads the draw rows once (two rows for a residual, one for a bonus)
            ProfScope prof("chunk_total", stream, (double)B * 2.0 * V * 4.0, 0.0);
            SV_LAUNCH(prof, chunk_total_kernel, B * nchunk, kDrawThreads, stream, target, draft, K,
                      V, nchunk, inv_t, meta, ctot);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    } else {
        // reads the draw rows once (two rows for a residual, one for a bonus)
        ProfScope prof("decide_chunk", stream, greedy ? 0.0 : (double)B * 2.0 * V * 4.0, 0.0);
        SV_LAUNCH(prof, decide_chunk_kernel, B * nchunk, kDrawThreads, stream, target, draft,
                  tokens, K, V, nchunk, inv_t, greedy, k0, k1, step, pv, ps, pi, ctot, meta,
                  out_tokens, accept_len, p_at, q_at, B, K + 1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (greedy) return hipSuccess;
    ProfScope prof("draw", stream, (double)B * 2.0 * kChunk * 4.0, 0.0);
    SV_LAUNCH(prof, draw_kernel, B, kDrawThreads, stream, target, draft, tokens, K, V, nchunk,
              inv_t, k0, k1, step, 1u, 0, ctot, meta, out_tokens, accept_len, K + 1);
    return hipGetLastError();
}

hipError_t launch_sample(const float* logits, int B, int V, float inv_t, int greedy,
                         uint64_t seed, uint32_t step, int slot, const float* pv, const float* ps,
                         const int* pi, float* scratch, int32_t* tokens, int out_stride,
                         hipStream_t stream) {
    if (B <= 0) return hipSuccess;
    const int nchunk = stats_chunks(V);
    const uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
    float* ctot = scratch;
    float* meta = scratch + (size_t)B * nchunk;
    // a verification with no draft positions: every row is a bonus row
    {
        ProfScope prof("decide_chunk", stream, greedy ? 0.0 : (double)B * V * 4.0, 0.0);
        SV_LAUNCH(prof, decide_chunk_kernel, B * nchunk, kDrawThreads, stream, logits,
                  (const float*)nullptr, (const int32_t*)nullptr, 0, V, nchunk, inv_t, greedy, k0,
                  k1, step, pv, ps, pi, ctot, meta, tokens, (int32_t*)nullptr, (float*)nullptr,
                  (float*)nullptr, B, out_stride);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (greedy) return hipSuccess;
    ProfScope prof("draw", stream, (double)B * kChunk * 4.0, 0.0);
    SV_LAUNCH(prof, draw_kernel, B, kDrawThreads, stream, logits, (const float*)nullptr,
              (const int32_t*)nullptr, 0, V, nchunk, inv_t, k0, k1, step, 2u, slot - 1, ctot, meta,
              tokens, (int32_t*)nullptr, out_stride);
    return hipGetLastError();
}

}  // namespace sv
