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
// Layout of the work: the statistics kernel splits every row into chunks of
// kChunk logits (one workgroup each, all of a thread's loads in flight at
// once) and writes per-chunk (max, sum) or (max, argmax) pairs; the accept
// kernel (one workgroup per request) folds the chunk pairs of the rows it
// needs in chunk order, decides, and draws.
#include <float.h>
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

constexpr int kStatsThreads = 256;
constexpr int kChunk = 4096;                      // logits per statistics workgroup
constexpr int kPerThread = kChunk / kStatsThreads; // 16 = 4 float4
constexpr int kAcceptThreads = 1024;
constexpr int kAcceptWaves = kAcceptThreads / kWave;
constexpr int kTile = 4 * kWave;                  // 256 logits per wave tile
constexpr int kBatch = 4;                         // tiles loaded together

__device__ __forceinline__ float prob(float z, float m, float inv_t, float inv_s) {
    return expf((z - m) * inv_t) * inv_s;
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
    s = s * expf((m - mx) * inv_t) + s2 * expf((m2 - mx) * inv_t);
    m = mx;
}

__device__ __forceinline__ void lse_add(float& m, float& s, float v, float inv_t) {
    if (v == -INFINITY) return;
    if (v > m) {
        s = (m == -INFINITY) ? 0.f : s * expf((m - v) * inv_t);
        m = v;
    }
    s += expf((v - m) * inv_t);
}

// Better (value, index): larger value, then smaller index.
__device__ __forceinline__ void arg_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

__global__ __launch_bounds__(kStatsThreads) void row_stats_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int n_t, int V,
    int nchunk, float inv_t, int greedy, int vec4, float* __restrict__ pv,
    float* __restrict__ ps, int* __restrict__ pi) {
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
            if (e < V) q = *reinterpret_cast<const f32x4*>(z + e);   // V % 4 == 0 here
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

    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) lse_add(m, s, x[i], inv_t);
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

// Row statistics folded from the per-chunk pairs, in chunk order.
__device__ __forceinline__ void row_lse(const float* pv, const float* ps, size_t row, int nchunk,
                                        float inv_t, float& m, float& s) {
    m = -INFINITY;
    s = 0.f;
    for (int c = 0; c < nchunk; ++c) lse_merge(m, s, pv[row * nchunk + c], ps[row * nchunk + c], inv_t);
}

__device__ __forceinline__ int row_argmax(const float* pv, const int* pi, size_t row, int nchunk) {
    float v = -INFINITY;
    int i = INT_MAX;
    for (int c = 0; c < nchunk; ++c) arg_merge(v, i, pv[row * nchunk + c], pi[row * nchunk + c]);
    return i == INT_MAX ? 0 : i;
}

struct DrawRows {
    const float* zt;
    const float* zd;     // nullptr: the weights are p itself
    float mt, it_s, md, id_s, inv_t;
};

// Four consecutive logits starting at e (e % 4 == 0), -inf past the end.
__device__ __forceinline__ f32x4 load4(const float* z, int e, int end, bool vec4) {
    if (vec4 && e + 3 < end) return *reinterpret_cast<const f32x4*>(z + e);
    f32x4 q;
    q.x = e < end ? z[e] : -INFINITY;
    q.y = e + 1 < end ? z[e + 1] : -INFINITY;
    q.z = e + 2 < end ? z[e + 2] : -INFINITY;
    q.w = e + 3 < end ? z[e + 3] : -INFINITY;
    return q;
}

__device__ __forceinline__ float weight(const DrawRows& dr, float zt, float zd) {
    const float p = prob(zt, dr.mt, dr.inv_t, dr.it_s);
    if (!dr.zd) return p;
    return fmaxf(0.f, p - prob(zd, dr.md, dr.inv_t, dr.id_s));
}

// Scan of one 256-logit tile by one wave: c[i] = within-tile inclusive sum at
// lane element i (lane exclusive prefix + own running sum).  The tile total is
// defined as the last element's inclusive sum, so both passes agree on it.
__device__ __forceinline__ float tile_scan(const DrawRows& dr, f32x4 zt, f32x4 zd, int lane,
                                           float c[4]) {
    const float w0 = weight(dr, zt.x, zd.x), w1 = weight(dr, zt.y, zd.y);
    const float w2 = weight(dr, zt.z, zd.z), w3 = weight(dr, zt.w, zd.w);
    c[0] = w0;
    c[1] = c[0] + w1;
    c[2] = c[1] + w2;
    c[3] = c[2] + w3;
    float incl = c[3];
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    float excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = excl + c[i];
    return __shfl(c[3], kWave - 1, kWave);
}

// Inverse-CDF draw over [0, V) by one workgroup.  Wave w owns the segment
// [w * seg, (w + 1) * seg) (seg a multiple of 256).  Pass 1 sums each segment
// tile by tile (kBatch tiles' loads in flight together); one thread forms the
// segment prefix sums and the threshold t = u * R; pass 2 rescans the first
// segment whose end exceeds t.  Returns -1 when every weight is zero.
__device__ int block_draw(const DrawRows& dr, int V, float u, bool vec4, float* sh_seg,
                          int* sh_tok) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int seg = ((V + kAcceptWaves - 1) / kAcceptWaves + kTile - 1) / kTile * kTile;
    const int sb = min(V, wave * seg);
    const int se = min(V, sb + seg);

    float total = 0.f;
    for (int b0 = sb; b0 < se; b0 += kBatch * kTile) {
        f32x4 zt[kBatch], zd[kBatch];
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
            const int e = b0 + t * kTile + 4 * lane;
            zt[t] = load4(dr.zt, e, se, vec4);
            zd[t] = dr.zd ? load4(dr.zd, e, se, vec4) : zt[t];
        }
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
            if (b0 + t * kTile >= se) break;
            float c[4];
            total += tile_scan(dr, zt[t], zd[t], lane, c);
        }
    }
    if (lane == 0) sh_seg[wave] = total;
    __syncthreads();
    if (tid == 0) {
        float pre = 0.f;
        for (int w = 0; w < kAcceptWaves; ++w) {
            const float nxt = pre + sh_seg[w];
            sh_seg[w] = pre;              // becomes the exclusive prefix
            pre = nxt;
        }
        sh_seg[kAcceptWaves] = pre;       // total R
        const float t = u * pre;
        int target_w = -1;
        for (int w = 0; w < kAcceptWaves; ++w) {
            const float end = (w + 1 < kAcceptWaves) ? sh_seg[w + 1] : pre;
            if (end > t) {
                target_w = w;
                break;
            }
        }
        sh_tok[0] = -1;
        sh_tok[1] = target_w;
        sh_seg[kAcceptWaves + 1] = t;
    }
    __syncthreads();
    const int target_w = sh_tok[1];
    const float t = sh_seg[kAcceptWaves + 1];
    const float R = sh_seg[kAcceptWaves];
    if (target_w >= 0 && wave == target_w) {
        const float pre = sh_seg[wave];
        float run = 0.f;
        bool found = false;
        for (int b0 = sb; b0 < se && !found; b0 += kBatch * kTile) {
            f32x4 zt[kBatch], zd[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int e = b0 + q * kTile + 4 * lane;
                zt[q] = load4(dr.zt, e, se, vec4);
                zd[q] = dr.zd ? load4(dr.zd, e, se, vec4) : zt[q];
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int tb = b0 + q * kTile;
                if (found || tb >= se) break;
                float c[4];
                const float tt = tile_scan(dr, zt[q], zd[q], lane, c);
                int hit = -1;
#pragma unroll
                for (int i = 3; i >= 0; --i)
                    if (tb + 4 * lane + i < se && pre + (run + c[i]) > t) hit = i;
                const unsigned long long mask = __ballot(hit >= 0);
                if (mask) {
                    const int first = __ffsll((long long)mask) - 1;
                    if (lane == first) sh_tok[0] = tb + 4 * lane + hit;
                    found = true;
                }
                run += tt;
            }
        }
    }
    __syncthreads();
    if (sh_tok[0] >= 0 || R <= 0.f) {
        const int r = R <= 0.f ? -1 : sh_tok[0];
        __syncthreads();
        return r;
    }
    // u * R rounded up to R: take the last token with positive weight.
    int last = -1;
    for (int y = tid; y < V; y += kAcceptThreads) {
        const float w = weight(dr, dr.zt[y], dr.zd ? dr.zd[y] : 0.f);
        if (w > 0.f) last = y;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
    if (lane == 0) sh_tok[2 + wave] = last;
    __syncthreads();
    int r = -1;
    for (int w = 0; w < kAcceptWaves; ++w) r = max(r, sh_tok[2 + w]);
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, int K, int V, int nchunk, float inv_t, int greedy,
    int vec4, uint32_t k0, uint32_t k1, uint32_t step, int n_t, const float* __restrict__ pv,
    const float* __restrict__ ps, const int* __restrict__ pi, int32_t* __restrict__ out,
    int32_t* __restrict__ accept_len, float* __restrict__ p_at, float* __restrict__ q_at) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    __shared__ int sh_first;
    __shared__ int sh_bad;
    __shared__ float sh_seg[kAcceptWaves + 2];
    __shared__ int sh_tok[2 + kAcceptWaves];
    __shared__ float sh_stat[4];
    if (tid == 0) {
        sh_first = K + 1;
        sh_bad = 0;
    }
    __syncthreads();

    const size_t trow0 = (size_t)b * (K + 1);
    for (int j0 = tid; j0 < K; j0 += kAcceptThreads) {
        const int x = tokens[(size_t)b * K + j0];
        if (x < 0 || x >= V) {
            atomicOr(&sh_bad, 1);
            continue;
        }
        const size_t rt = trow0 + j0;
        bool ok;
        float p, q;
        if (greedy) {
            ok = (x == row_argmax(pv, pi, rt, nchunk));
            p = ok ? 1.f : 0.f;
            q = 1.f;
        } else {
            const size_t rd = (size_t)b * K + j0;
            float mt, st, md, sd;
            row_lse(pv, ps, rt, nchunk, inv_t, mt, st);
            row_lse(pv, ps, n_t + rd, nchunk, inv_t, md, sd);
            p = prob(target[rt * V + x], mt, inv_t, 1.0f / st);
            q = prob(draft[rd * V + x], md, inv_t, 1.0f / sd);
            const float u = u_accept(philox_word0((uint32_t)b, (uint32_t)(j0 + 1), 0u, step, k0, k1));
            ok = (u <= p / q);      // q == 0: +inf (accept) or NaN (p == 0: reject)
        }
        if (p_at) p_at[(size_t)b * K + j0] = p;
        if (q_at) q_at[(size_t)b * K + j0] = q;
        if (!ok) atomicMin(&sh_first, j0 + 1);
    }
    __syncthreads();

    int32_t* ob = out + trow0;
    if (sh_bad) {
        for (int y = tid; y <= K; y += kAcceptThreads) ob[y] = -1;
        if (tid == 0) accept_len[b] = 0;
        return;
    }
    const int js = sh_first;                 // 1..K: first rejection; K+1: all accepted
    const size_t rt = trow0 + js - 1;
    int tok;
    if (greedy) {
        tok = row_argmax(pv, pi, rt, nchunk);
    } else {
        const bool resid = js <= K;
        const size_t rd = (size_t)b * K + js - 1;
        if (tid == 0) {
            float m, s;
            row_lse(pv, ps, rt, nchunk, inv_t, m, s);
            sh_stat[0] = m;
            sh_stat[1] = 1.0f / s;
            if (resid) {
                row_lse(pv, ps, n_t + rd, nchunk, inv_t, m, s);
                sh_stat[2] = m;
                sh_stat[3] = 1.0f / s;
            }
        }
        __syncthreads();
        DrawRows dr;
        dr.zt = target + rt * V;
        dr.mt = sh_stat[0];
        dr.it_s = sh_stat[1];
        dr.inv_t = inv_t;
        dr.zd = resid ? draft + rd * V : nullptr;
        dr.md = resid ? sh_stat[2] : 0.f;
        dr.id_s = resid ? sh_stat[3] : 0.f;
        const float u = u_resample(philox_word0((uint32_t)b, (uint32_t)js, 1u, step, k0, k1));
        tok = block_draw(dr, V, u, vec4, sh_seg, sh_tok);
        if (tok < 0 && dr.zd) {              // residual mass rounded to zero: draw from p
            dr.zd = nullptr;
            tok = block_draw(dr, V, u, vec4, sh_seg, sh_tok);
        }
        if (tok < 0) tok = 0;
    }
    for (int y = tid; y <= K; y += kAcceptThreads) {
        int32_t v = -1;
        if (y < js - 1) v = tokens[(size_t)b * K + y];
        else if (y == js - 1) v = tok;
        ob[y] = v;
    }
    if (tid == 0) accept_len[b] = js;
}

}  // namespace

int stats_chunks(int V) { return (V + kChunk - 1) / kChunk; }

hipError_t launch_row_stats(const float* target, const float* draft, int n_t, int n_d, int V,
                            float inv_t, int greedy, float* pv, float* ps, int* pi,
                            hipStream_t stream) {
    const int rows = n_t + n_d;
    if (rows <= 0) return hipSuccess;
    const int nchunk = stats_chunks(V);
    const int vec4 = (V % 4 == 0) && ((uintptr_t)target % 16 == 0) &&
                     (draft == nullptr || (uintptr_t)draft % 16 == 0);
    ProfScope prof("row_stats", stream, (double)rows * V * 4.0, 0.0);
    row_stats_kernel<<<rows * nchunk, kStatsThreads, 0, stream>>>(
        target, draft, n_t, V, nchunk, inv_t, greedy, vec4, pv, ps, pi);
    return hipGetLastError();
}

hipError_t launch_accept(const float* target, const float* draft, const int32_t* tokens, int B,
                         int K, int V, float inv_t, int greedy, uint64_t seed, uint32_t step,
                         const float* pv, const float* ps, const int* pi, int32_t* out_tokens,
                         int32_t* accept_len, float* p_at, float* q_at, hipStream_t stream) {
    if (B <= 0) return hipSuccess;
    const int vec4 = (V % 4 == 0) && ((uintptr_t)target % 16 == 0) &&
                     (draft == nullptr || (uintptr_t)draft % 16 == 0);
    // bytes: worst case reads two rows per request twice (draw passes)
    ProfScope prof("accept_resample", stream, (double)B * (greedy ? 0.0 : 2.0 * V * 4.0), 0.0);
    accept_kernel<<<B, kAcceptThreads, 0, stream>>>(
        target, draft, tokens, K, V, stats_chunks(V), inv_t, greedy, vec4,
        (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32), step, B * (K + 1), pv, ps, pi,
        out_tokens, accept_len, p_at, q_at);
    return hipGetLastError();
}

}  // namespace sv
