// Verification forward of a mixture-of-experts target (C ABI in
// include/spec_verify_moe.h).
//
// Per block: RMSNorm -> router scores -> top_k per position (ties to the
// lower id, softmax weights) -> counting sort of the M * top_k (position,
// slot) pairs by expert, so every expert's rows are one contiguous range ->
// grouped up projection (+ SiLU) -> grouped down projection -> the next
// RMSNorm, which first adds the weighted expert outputs to the residual
// stream (slots in rank order).  The
// grouped kernels give every (expert, 16-row weight fragment) a workgroup
// that returns before touching memory when the expert has no rows, so a step
// streams the weights of the experts it uses and nothing else - the effect
// the pages attribute to MoE verification (Cohere, "Dynamic speculative
// decoding"): more verified positions, more experts loaded.  The matmul core
// is the streaming one of the dense path: weight fragments from HBM straight
// into registers as the A operand of v_mfma_f32_16x16x32_bf16, four waves
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
constexpr int kGroupWaves = 4;        // k slices of a grouped workgroup

// ---- routing ------------------------------------------------------------------
constexpr int kRouterWaves = 4;
constexpr int kMaxRouterSplits = 16;

// Router scores, split three ways so that any M fills the chip: workgroup
// (fe, ks, mb) takes experts 16 fe .. 16 fe + 15, reduction steps (32 wide)
// ks * spw .. ks * spw + spw - 1 and positions 64 mb .. 64 mb + 63, and
// writes part[ks][t][e].  A wave holds one weight fragment per step (A
// operand) and runs the 16-position fragments of activations through it;
// the four waves' sums are added in LDS in wave order.
__device__ __forceinline__ void router_partial(const uint16_t* __restrict__ a,
                                               const uint16_t* __restrict__ Wr, int M, int E, int d,
                                               int spw, int fe, int ks, int m0,
                                               float* __restrict__ part,
                                               float (*red)[4][4][kWave]) {
    constexpr int MF = 4;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int r16 = lane & 15, g = lane >> 4;
    const int S = d / 32;
    const int s0 = ks * spw, s1 = min(S, s0 + spw);
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    f32x4v acc[MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[mf] = f32x4v{0.f, 0.f, 0.f, 0.f};
    for (int s = s0 + wave; s < s1; s += kRouterWaves) {
        const bf16x8 w = *reinterpret_cast<const bf16x8*>(Wr + ((size_t)fe * S + s) * 512 + lane * 8);
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
            const int t = m0 + mf * 16 + r16;
            const bf16x8 x = t < M ? *reinterpret_cast<const bf16x8*>(a + (size_t)t * d + 32 * s + 8 * g)
                                   : zero8;
            acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, x, acc[mf], 0, 0, 0);
        }
    }
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mf][r][lane] = acc[mf][r];
    __syncthreads();
    for (int i = threadIdx.x; i < 256 * MF; i += kRouterWaves * kWave) {
        const int ii = i & 15, jj = (i >> 4) & 15, mf = i >> 8;   // expert ii, position jj
        const int e = fe * 16 + ii, t = m0 + mf * 16 + jj;
        if (e >= E || t >= M) continue;
        const int r = ii & 3, l = ((ii >> 2) << 4) + jj;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kRouterWaves; ++w) v += red[w][mf][r][l];
        part[((size_t)ks * M + t) * E + e] = v;
    }
}

// Scores of `rows` positions t0 .. t0 + rows - 1 into LDS: zs[r][e] (row
// stride Ep, a multiple of 4) = the partial planes added in split order; a
// NaN score, and the padding columns e >= E, become -inf.  A thread loads
// all planes of up to 4 (position, expert) pairs at once.
template <int THREADS>
__device__ __forceinline__ void sum_planes(const float* __restrict__ part, int KS, int M, int E,
                                           int Ep, int t0, int rows, float* zs) {
    constexpr int P = 4;
    const int n = rows * Ep;
    for (int i0 = 0; i0 < n; i0 += P * THREADS) {
        float pv[P][kMaxRouterSplits];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = i0 + p * THREADS + (int)threadIdx.x;
            const int r = i / Ep, e = i - r * Ep;
            const bool in = i < n && e < E;
#pragma unroll
            for (int y = 0; y < kMaxRouterSplits; ++y)
                pv[p][y] = (in && y < KS) ? part[((size_t)y * M + t0 + r) * E + e] : 0.f;
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = i0 + p * THREADS + (int)threadIdx.x;
            if (i >= n) continue;
            const int e = i % Ep;
            float z = 0.f;
#pragma unroll
            for (int y = 0; y < kMaxRouterSplits; ++y)
                if (y < KS) z += pv[p][y];
            zs[i] = (e < E && z == z) ? z : -INFINITY;
        }
    }
}

// Maximum of v over the wave, in every lane: DPP exchanges within rows of
// 16 lanes (quad swaps, half-row and row mirrors), then the four row
// maxima through readlane.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max_all(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));         // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp_f32<0x4E>(v));         // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp_f32<0x141>(v));        // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));        // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// top_k of the rows of zs, one wave per row (rows wave, wave + nwaves, ...):
// k rounds of a wave-wide maximum over the experts not yet taken, the
// lowest expert id among those equal to it (ballot, first set bit) taken;
// the weights are the softmax of the chosen scores, summed in rank order.
template <int THREADS>
__device__ __forceinline__ void topk_rows(const float* zs, int rows, int E, int Ep, int k, int t0,
                                          int32_t* __restrict__ sel, float* __restrict__ wts) {
    constexpr int Q = kMoeMaxExperts / kWave;   // experts lane + 64 j
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int r = wave; r < rows; r += THREADS / kWave) {
        float v[Q];
        unsigned avail = 0;
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const int id = lane + kWave * j;
            v[j] = id < E ? zs[r * Ep + id] : -INFINITY;
            if (id < E) avail |= 1u << j;
        }
        float zsel[kMoeMaxTopK];
        int esel[kMoeMaxTopK];
#pragma unroll
        for (int q = 0; q < kMoeMaxTopK; ++q) {
            zsel[q] = 0.f;
            esel[q] = 0;
            if (q >= k) continue;
            float m = -INFINITY;
#pragma unroll
            for (int j = 0; j < Q; ++j)
                if ((avail >> j) & 1u) m = fmaxf(m, v[j]);
            m = wave_max_all(m);
            int id = -1;
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const unsigned long long b = __ballot(((avail >> j) & 1u) && v[j] == m);
                if (id < 0 && b) id = kWave * j + __ffsll((long long)b) - 1;
            }
            if ((id & (kWave - 1)) == lane) avail &= ~(1u << (id / kWave));
            zsel[q] = m;
            esel[q] = id;
        }
        if (lane == 0) {
            const int t = t0 + r;
            float ex[kMoeMaxTopK], sum = 0.f;
#pragma unroll
            for (int q = 0; q < kMoeMaxTopK; ++q) {
                ex[q] = q < k ? (zsel[0] == -INFINITY ? 1.f : expf(zsel[q] - zsel[0])) : 0.f;   // no number: equal
                sum += ex[q];
            }
#pragma unroll
            for (int q = 0; q < kMoeMaxTopK; ++q) {
                if (q < k) {
                    sel[t * k + q] = esel[q];
                    wts[t * k + q] = ex[q] / sum;
                }
            }
        }
    }
}

// Counting sort of the M * k (position, slot) pairs (expert ids in lsel, in
// LDS) by expert, so every expert's rows are one contiguous range: counts by
// LDS atomics, an exclusive scan over experts (one wave), then every pair
// takes the next free row of its expert by LDS atomics.  The order of an
// expert's rows is therefore not fixed, and nothing depends on it: every
// output row of the grouped kernels is its own dot products, and the fold
// finds each pair's row through inv.  Also lists the experts with rows in
// id order (alist[0 .. *nact - 1]) for the grouped kernels.  With `pad`
// every expert's range is rounded up to a multiple of 16 rows (offs and inv
// count padded rows) and the padding rows get perm = -1.  cnt, loff: LDS [E]
// and [E + 1].
template <int THREADS>
__device__ __forceinline__ void sort_pairs(const int32_t* lsel, int M, int E, int k, int pad,
                                           int32_t* cnt, int32_t* loff, int32_t* __restrict__ offs,
                                           int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                           int32_t* __restrict__ alist, int32_t* __restrict__ nact,
                                           int32_t* __restrict__ active) {
    const int tid = threadIdx.x, n = M * k;
    for (int x = tid; x < E; x += THREADS) cnt[x] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += THREADS) atomicAdd(&cnt[lsel[i]], 1);
    __syncthreads();
    if (tid < kWave) {                       // exclusive scan over experts, one wave
        constexpr int Q = kMoeMaxExperts / kWave;   // experts Q * lane .. Q * lane + Q - 1
        int c[Q], tot = 0, nz = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int x = Q * tid + q;
            c[q] = x < E ? cnt[x] : 0;
            nz += c[q] > 0;
            if (pad) c[q] = (c[q] + 15) & ~15;
            tot += c[q];
        }
        int itot = tot, inz = nz;            // inclusive scans across lanes
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int a1 = __shfl_up(itot, o, kWave), a2 = __shfl_up(inz, o, kWave);
            if (tid >= o) {
                itot += a1;
                inz += a2;
            }
        }
        int base = itot - tot, slot = inz - nz;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int x = Q * tid + q;
            if (x < E) {
                loff[x] = base;
                base += c[q];
                if (c[q] > 0) alist[slot++] = x;
            }
        }
        if (tid == kWave - 1) {
            loff[E] = itot;
            *nact = inz;
            if (active) *active = inz;
        }
    }
    __syncthreads();
    for (int x = tid; x <= E; x += THREADS) {
        offs[x] = loff[x];
        if (x < E) cnt[x] = loff[x];         // next free row of expert x
    }
    if (pad)
        for (int r = tid; r < loff[E]; r += THREADS) perm[r] = -1;
    __syncthreads();
    for (int i = tid; i < n; i += THREADS) {
        const int pos = atomicAdd(&cnt[lsel[i]], 1);
        perm[pos] = i;
        inv[i] = pos;
    }
}

__global__ __launch_bounds__(kRouterWaves * kWave) void moe_router_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ Wr, int M, int E, int d, int spw,
    float* __restrict__ part) {
    __shared__ float red[kRouterWaves][4][4][kWave];
    router_partial(a, Wr, M, E, d, spw, blockIdx.x, blockIdx.y, blockIdx.z * 64, part, red);
}

// top_k of positions 4 blockIdx.x .. 4 blockIdx.x + 3, one wave each.
__global__ __launch_bounds__(256) void moe_topk_kernel(const float* __restrict__ part, int KS, int M,
                                                       int E, int Ep, int k,
                                                       int32_t* __restrict__ sel,
                                                       float* __restrict__ wts) {
    __shared__ float zs[4 * kMoeMaxExperts];
    const int t0 = blockIdx.x * 4;
    const int rows = min(4, M - t0);
    sum_planes<256>(part, KS, M, E, Ep, t0, rows, zs);
    __syncthreads();
    topk_rows<256>(zs, rows, E, Ep, k, t0, sel, wts);
}

__global__ __launch_bounds__(kRouteThreads) void moe_sort_kernel(
    const int32_t* __restrict__ sel, int M, int E, int k, int pad, int32_t* __restrict__ offs,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ alist,
    int32_t* __restrict__ nact, int32_t* __restrict__ active) {
    __shared__ int32_t lsel[kMoeMaxRows * kMoeMaxTopK];
    __shared__ int32_t cnt[kMoeMaxExperts];
    __shared__ int32_t loff[kMoeMaxExperts + 1];
    for (int i = threadIdx.x; i < M * k; i += kRouteThreads) lsel[i] = sel[i];
    __syncthreads();
    sort_pairs<kRouteThreads>(lsel, M, E, k, pad, cnt, loff, offs, perm, inv, alist, nact, active);
}

// Routing of up to 6 positions in one workgroup: router scores, top_k and
// the sort without two launches in between.  Wave w takes expert fragment w
// / wpf (wpf = 16 / fragments waves per fragment) and the w % wpf-th slice of
// its reduction steps, with the positions as the B operand (rows past M read
// as zeros); the slices are summed in slice order, then top_k (one wave per
// position, selections kept in LDS) and the counting sort run as in the
// separate kernels.  One CU reads all the router weights, so the separate
// kernels (router spread over the chip) catch up at about 8 positions
// (64-expert workload, forward: -5% at 1 position, -1% at 5, +0.5% at 8,
// +3% at 16).
constexpr int kRouteSmallRows = 6;
constexpr int kRouteBatch = 8;
constexpr int kRouteSmallMaxSteps = 32;   // steps per wave: more take the separate kernels

// Whether the routing of M positions runs in one workgroup (each wave's
// slice at most kRouteSmallMaxSteps steps).
bool route_small(int M, int E, int d) {
    const int nfe = (E + 15) / 16;
    const int wpf = (kRouteThreads / kWave) / nfe;
    return M <= kRouteSmallRows && (d / 32 + wpf - 1) / wpf <= kRouteSmallMaxSteps;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_small_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ Wr, int M, int E, int Ep, int d,
    int k, int pad, float* __restrict__ wts, int32_t* __restrict__ offs,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ alist,
    int32_t* __restrict__ nact, int32_t* __restrict__ active) {
    constexpr int NW = kRouteThreads / kWave;
    __shared__ float zs[kRouteSmallRows * kMoeMaxExperts];
    __shared__ f32x4v part[NW][kWave];
    __shared__ int32_t lsel[kRouteSmallRows * kMoeMaxTopK];
    __shared__ int32_t cnt[kMoeMaxExperts];
    __shared__ int32_t loff[kMoeMaxExperts + 1];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int S = d / 32;
    const int nfe = (E + 15) / 16;                 // <= 16 (E <= 256)
    const int wpf = NW / nfe;
    const int fe = wave / wpf, ks = wave % wpf;    // fe >= nfe: idle wave
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
    if (fe < nfe) {
        const int r16 = lane & 15, g = lane >> 4;
        const int s0 = S * ks / wpf, s1 = S * (ks + 1) / wpf;
        const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        // kRouteBatch steps of loads in flight before their products (steps
        // past the slice read as zeros)
        for (int s = s0; s < s1; s += kRouteBatch) {
            bf16x8 w[kRouteBatch], x[kRouteBatch];
#pragma unroll
            for (int u = 0; u < kRouteBatch; ++u) {
                const bool in = s + u < s1;
                w[u] = in ? *reinterpret_cast<const bf16x8*>(Wr + ((size_t)fe * S + s + u) * 512 + lane * 8)
                          : zero8;
                x[u] = in && r16 < M
                           ? *reinterpret_cast<const bf16x8*>(a + (size_t)r16 * d + 32 * (s + u) + 8 * g)
                           : zero8;
            }
#pragma unroll
            for (int u = 0; u < kRouteBatch; ++u)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[u], x[u], acc, 0, 0, 0);
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    // lane 16 (e % 16 / 4) + t, element e % 4 of fragment e / 16 holds
    // expert e of position t; a NaN score and the padding columns are -inf
    for (int i = threadIdx.x; i < kRouteSmallRows * Ep; i += kRouteThreads) {
        const int t = i / Ep, e = i - t * Ep;
        float z = -INFINITY;
        if (t < M && e < E) {
            const int f = e / 16, ii = e & 15;
            const int l = ((ii >> 2) << 4) + t;
            float v = 0.f;
            for (int w = 0; w < wpf; ++w) v += part[f * wpf + w][l][ii & 3];
            z = v == v ? v : -INFINITY;
        }
        zs[i] = z;
    }
    __syncthreads();
    topk_rows<kRouteThreads>(zs, M, E, Ep, k, 0, lsel, wts);
    __syncthreads();
    sort_pairs<kRouteThreads>(lsel, M, E, k, pad, cnt, loff, offs, perm, inv, alist, nact, active);
}

// ---- grouped matmul -------------------------------------------------------------
// out[row, n] = sum_c act[src(row), c] * W_e[n, c] for the rows row of expert
// e (offs[e] .. offs[e+1]); src(row) = perm[row] / top_k (gather of the
// positions' activations) when `gather`, else row.  W_e = W + e * wstride, in
// the tiled layout.  Epilogue: SiLU + bf16 (up) or fp32 store (down).
// Workgroup i takes listed expert alist[i / nfr] and the RF 16-row weight
// fragments RF * (i % nfr) .. + RF - 1; workgroups past the *nact listed
// experts return at once.  A wave streams its k slice of those fragments in
// buffers of U 32-wide steps, the first issued before the row indices are
// read, and runs MF 16-row activation fragments per pass over the expert's
// rows through them (one activation load serves RF weight fragments;
// fragments past the expert's rows are skipped by the whole wave).
// Padded rows (offs multiples of 16, perm = -1 on an expert's padding
// rows, which read as zeros): kActIn - `act` is in the operand layout (one
// KiB per 16 rows x 32 k), so an activation load is a wave-uniform base plus
// a lane offset and no row index is read; kActOut - the SiLU output is
// written in that layout for the down projection.
template <int EPI, int MF, int U, int RF, bool kActIn, bool kActOut>
__global__ __launch_bounds__(kGroupWaves * kWave) void moe_grouped_kernel(
    const uint16_t* __restrict__ W, size_t wstride, int N, int K, const uint16_t* __restrict__ act,
    const int32_t* __restrict__ perm, int gather, int top_k, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ alist, const int32_t* __restrict__ nact, void* __restrict__ out) {
    const int nfrag = (N + 15) / 16;
    const int nfr = (nfrag + RF - 1) / RF;
    const int li = blockIdx.x / nfr;
    const int f0 = (blockIdx.x % nfr) * RF;
    // the count of experts in use and this workgroup's entry are read
    // together (li < listed <= E, and alist holds E entries), so the weight
    // address waits for one memory round trip, not two
    const int used = *nact;
    const int e = alist[li];
    asm volatile("" ::"s"(used), "s"(e));  // both loads before the branch
    if (li >= used) return;                // fewer experts in use than the launch allows

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15, g = lane >> 4;
    const int S = K / 32;
    const int s0 = S * wave / kGroupWaves, s1 = S * (wave + 1) / kGroupWaves;
    const uint16_t* wbase = W + (size_t)e * wstride + lane * 8;
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    __shared__ f32x4v red[kGroupWaves][RF][MF][kWave];

    bf16x8 wa[U][RF], wb[U][RF], xa[U][MF], xb[U][MF];
    auto loadw = [&](bf16x8 (&w)[U][RF], int s) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int rf = 0; rf < RF; ++rf)
                w[u][rf] = (s + u < s1 && f0 + rf < nfrag)
                               ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(
                                     wbase + ((size_t)(f0 + rf) * S + s + u) * 512))
                               : zero8;
    };
    loadw(wa, s0);                          // weights first: they need no row index
    const int row0 = offs[e];
    const int rows = offs[e + 1] - row0;

    for (int pass = 0; pass < rows; pass += 16 * MF) {
        const int prow = rows - pass;      // rows left, > 0
        const uint16_t* arow[kActIn ? 1 : MF];
        bool aval[MF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
            if constexpr (kActIn) {
                aval[mf] = mf * 16 < prow;
            } else {
                const int j = pass + mf * 16 + r16;
                aval[mf] = j < rows;
                const int rr = row0 + (aval[mf] ? j : 0);
                int src = rr;
                if (gather) {
                    const int pi = perm[rr];
                    aval[mf] = aval[mf] && pi >= 0;
                    src = pi >= 0 ? pi / top_k : 0;
                }
                arow[mf] = act + (size_t)src * K + 8 * g;
            }
        }
        // operand layout: the KiB of row block mf at step s lies (mf S + s)
        // KiB past the pass's first block
        const char* ablk = reinterpret_cast<const char*>(act) + (size_t)((row0 + pass) >> 4) * S * 1024;
        auto loadx = [&](bf16x8 (&x)[U][MF], int s) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    x[u][mf] = (s + u < s1 && aval[mf])
                                   ? *reinterpret_cast<const bf16x8*>(
                                         kActIn ? ablk + (uint32_t)(lane * 16 + (mf * S + s + u) * 1024)
                                                : reinterpret_cast<const char*>(arow[kActIn ? 0 : mf] + 32 * (s + u)))
                                   : zero8;
        };
        f32x4v acc[RF][MF];
#pragma unroll
        for (int rf = 0; rf < RF; ++rf)
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) acc[rf][mf] = f32x4v{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const bf16x8 (&w)[U][RF], const bf16x8 (&x)[U][MF]) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    if (mf == 0 || mf * 16 < prow)
#pragma unroll
                        for (int rf = 0; rf < RF; ++rf)
                            acc[rf][mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                w[u][rf], x[u][mf], acc[rf][mf], 0, 0, 0);
        };
        if (pass) loadw(wa, s0);
        loadx(xa, s0);
        for (int s = s0; s < s1; s += 2 * U) {
            loadw(wb, s + U);
            loadx(xb, s + U);
            compute(wa, xa);
            loadw(wa, s + 2 * U);
            loadx(xa, s + 2 * U);
            compute(wb, xb);
        }
        // the k slices summed in wave order: each wave stores its accumulators
        // lane-major (16-byte LDS writes), and each task sums the copies of one
        // lane's four outputs n0..n0+3 of one row (16-byte reads, no bank
        // conflicts) and stores them together
        if (pass) __syncthreads();         // the previous pass's readers are done
#pragma unroll
        for (int rf = 0; rf < RF; ++rf)
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) red[wave][rf][mf][lane] = acc[rf][mf];
        __syncthreads();
        for (int i = threadIdx.x; i < kWave * MF * RF; i += kGroupWaves * kWave) {
            const int l = i % kWave, mf = (i / kWave) % MF, rf = i / (kWave * MF);
            const int n0 = (f0 + rf) * 16 + 4 * (l >> 4);
            const int j = pass + mf * 16 + (l & 15);
            if (n0 >= N || j >= rows) continue;
            f32x4v v = red[0][rf][mf][l];
#pragma unroll
            for (int w = 1; w < kGroupWaves; ++w) v += red[w][rf][mf][l];
            const size_t o = (size_t)(row0 + j) * N + n0;
            const bool full = (N & 3) == 0 && n0 + 3 < N;   // rows start 16-byte aligned
            if constexpr (EPI == kEpiSilu) {
                // kActOut: the down projection's operand layout (N % 32 == 0)
                const int pr = row0 + j;
                uint16_t* dst = static_cast<uint16_t*>(out) +
                                (kActOut ? ((size_t)(pr >> 4) * (N >> 5) + (n0 >> 5)) * 512 +
                                               ((pr & 15) + 16 * ((n0 & 31) >> 3)) * 8 + (n0 & 7)
                                         : o);
                if (kActOut || full) {
                    uint2 pk;
                    pk.x = pack_bf16x2(silu(v[0]), silu(v[1]));
                    pk.y = pack_bf16x2(silu(v[2]), silu(v[3]));
                    *reinterpret_cast<uint2*>(dst) = pk;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n0 + r < N) dst[r] = (uint16_t)f32_to_bf16(silu(v[r]));
                }
            } else {
                float* dst = static_cast<float*>(out) + o;
                if (full) {
                    *reinterpret_cast<f32x4v*>(dst) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n0 + r < N) dst[r] = v[r];
                }
            }
        }
    }
}

// ---- host plan --------------------------------------------------------------
constexpr size_t kAlign = 256;
size_t aup(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Mean rows per expert (M top_k / E) from which each expert's rows are
// padded to 16 and the up projection writes its SiLU output in the operand
// layout, which the down projection then reads as one KiB per 16 rows x 32 k.
constexpr int kMoeActTiledMeanRows = 20;

struct MoePlan {
    int act_tiled = 0;         // padded rows, operand-layout up-projection output
    int head_kind = kMfmaSkinny;
    int head_act_tiled = 0;    // the last norm writes the head's activations in the operand layout
    int router_spw = 0, router_splits = 0;   // reduction steps per router split, splits
    size_t rows = 0;           // sorted rows (padded: M top_k + 15 per listed expert at most)
    size_t off_h, off_a, off_part, off_sel, off_w, off_offs, off_list, off_perm, off_inv, off_s,
        off_y, bytes;
};

MoePlan plan_moe(const sv_moe_desc& d, int M) {
    MoePlan p{};
    const size_t Mk = (size_t)M * d.top_k;
    const size_t listed = (size_t)d.n_experts < Mk ? (size_t)d.n_experts : Mk;
    p.act_tiled = (M * d.top_k + d.n_experts - 1) / d.n_experts >= kMoeActTiledMeanRows;
    p.rows = p.act_tiled ? Mk + 15 * listed : Mk;
    p.head_kind = M >= kHeadTiledMinRows ? kMfmaTiled : kMfmaSkinny;
    p.head_act_tiled = M >= kActTiledMinRows;
    const int S = d.d / 32;
    p.router_spw = S / 16 > 8 ? (S + 15) / 16 : 8;    // at most 16 partial score planes
    p.router_splits = (S + p.router_spw - 1) / p.router_spw;
    const size_t arows = (size_t)(M + 15) / 16 * 16;
    size_t o = 0;
    p.off_h = o; o = aup(o + (size_t)M * d.d * 4);
    p.off_a = o; o = aup(o + arows * d.d * 2);
    p.off_part = o; o = aup(o + (size_t)p.router_splits * M * d.n_experts * 4);
    p.off_sel = o; o = aup(o + Mk * 4);
    p.off_w = o; o = aup(o + Mk * 4);
    p.off_offs = o; o = aup(o + (size_t)(d.n_experts + 2) * 4);   // offsets, then the count
    p.off_list = o; o = aup(o + (size_t)d.n_experts * 4);
    p.off_perm = o; o = aup(o + p.rows * 4);
    p.off_inv = o; o = aup(o + Mk * 4);
    p.off_s = o; o = aup(o + p.rows * d.ffn * 2);
    p.off_y = o; o = aup(o + p.rows * d.d * 4);
    p.bytes = o;
    return p;
}

int moe_hip_fail(hipError_t e, const char* what) {
    return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// One grouped projection.  The arrangement follows the rows an expert holds
// on average (M * top_k / E): few rows want many workgroups and deep weight
// buffers; many rows want each activation load shared by several weight
// fragments (measured on the 64-expert top-6 workload over M = 1 .. 576).
template <int EPI, bool kActIn, bool kActOut>
void launch_grouped(ProfScope& prof, int M, int E, int k, int listed, int nfrag, hipStream_t s,
                    const uint16_t* W, size_t wstride, int N, int K, const uint16_t* act,
                    const int32_t* perm, int gather, const int32_t* offs, const int32_t* alist,
                    const int32_t* nact, void* out) {
#define SV_GROUPED(MF, U, RF)                                                                      \
    SV_LAUNCH(prof, (moe_grouped_kernel<EPI, MF, U, RF, kActIn, kActOut>),                        \
              (unsigned)(listed * ((nfrag + RF - 1) / RF)), kGroupWaves * kWave, s, W, wstride, N, \
              K, act, perm, gather, k, offs, alist, nact, out)
    const int mean_rows = (M * k + E - 1) / E;
    if (M <= 16)
        SV_GROUPED(1, 4, 1);      // at most 16 rows per expert
    else if (mean_rows <= 8)
        SV_GROUPED(1, 4, 2);
    else if (mean_rows <= 16)
        SV_GROUPED(2, 2, 2);
    else
        SV_GROUPED(4, 1, 4);
#undef SV_GROUPED
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
    int32_t* sel = reinterpret_cast<int32_t*>(w + p.off_sel);
    float* wts = reinterpret_cast<float*>(w + p.off_w);
    float* part = reinterpret_cast<float*>(w + p.off_part);
    int32_t* offs = reinterpret_cast<int32_t*>(w + p.off_offs);
    int32_t* nact = offs + d.n_experts + 1;
    int32_t* alist = reinterpret_cast<int32_t*>(w + p.off_list);
    int32_t* perm = reinterpret_cast<int32_t*>(w + p.off_perm);
    int32_t* inv = reinterpret_cast<int32_t*>(w + p.off_inv);
    void* S = w + p.off_s;
    float* Y = reinterpret_cast<float*>(w + p.off_y);
    const int E = d.n_experts, k = d.top_k;
    const size_t router_stride = tiled_elems(E, d.d);
    const size_t up_stride = tiled_elems(d.ffn, d.d);
    const size_t down_stride = tiled_elems(d.d, d.ffn);
    hipError_t e;

    e = launch_rmsnorm(hidden, h, nullptr, 0, d.gain, a, M, d.d, d.rms_eps, 1,
                       d.n_layers == 0 && p.head_act_tiled, s);
    if (e != hipSuccess) return moe_hip_fail(e, "rmsnorm launch");
    for (int l = 0; l < d.n_layers; ++l) {
        const uint16_t* wr = static_cast<const uint16_t*>(d.w_router) + (size_t)l * router_stride;
        int32_t* act_out = active_experts ? active_experts + l : nullptr;
        const int Ep = (E + 3) & ~3;
        if (route_small(M, E, d.d)) {
            ProfScope prof("moe_route", s, (double)E * d.d * 2 + (double)M * d.d * 2,
                           2.0 * M * E * (double)d.d);
            SV_LAUNCH(prof, moe_route_small_kernel, 1, kRouteThreads, s,
                      static_cast<const uint16_t*>(a), wr, M, E, Ep, d.d, k, p.act_tiled, wts,
                      offs, perm, inv, alist, nact, act_out);
            e = hipGetLastError();
            if (e != hipSuccess) return moe_hip_fail(e, "routing launch");
        } else {
            {
                ProfScope prof("moe_router", s, (double)E * d.d * 2 + (double)M * d.d * 2,
                               2.0 * M * E * (double)d.d);
                const dim3 grid((unsigned)((E + 15) / 16), (unsigned)p.router_splits,
                                (unsigned)((M + 63) / 64));
                SV_LAUNCH(prof, moe_router_kernel, grid, kRouterWaves * kWave, s,
                          static_cast<const uint16_t*>(a), wr, M, E, d.d, p.router_spw, part);
                e = hipGetLastError();
                if (e != hipSuccess) return moe_hip_fail(e, "router launch");
            }
            {
                ProfScope prof("moe_topk", s, (double)p.router_splits * M * E * 4, 0.0);
                SV_LAUNCH(prof, moe_topk_kernel, (unsigned)((M + 3) / 4), 256, s, part,
                          p.router_splits, M, E, Ep, k, sel, wts);
                e = hipGetLastError();
                if (e != hipSuccess) return moe_hip_fail(e, "top-k launch");
            }
            {
                ProfScope prof("moe_sort", s, (double)M * k * 12, 0.0);
                SV_LAUNCH(prof, moe_sort_kernel, 1, kRouteThreads, s, sel, M, E, k, p.act_tiled, offs,
                          perm, inv, alist, nact, act_out);
                e = hipGetLastError();
                if (e != hipSuccess) return moe_hip_fail(e, "sort launch");
            }
        }
        const int listed = E < M * k ? E : M * k;   // experts a block can use
        {
            // bytes depend on the experts the device picks: counted by the caller
            ProfScope prof("moe_up_silu", s, 0.0, 2.0 * M * k * (double)d.ffn * d.d);
            const uint16_t* wu = static_cast<const uint16_t*>(d.w_up) + (size_t)l * E * up_stride;
            if (p.act_tiled)
                launch_grouped<kEpiSilu, false, true>(prof, M, E, k, listed, (d.ffn + 15) / 16, s, wu,
                                                      up_stride, d.ffn, d.d,
                                                      static_cast<const uint16_t*>(a), perm, 1, offs,
                                                      alist, nact, S);
            else
                launch_grouped<kEpiSilu, false, false>(prof, M, E, k, listed, (d.ffn + 15) / 16, s,
                                                       wu, up_stride, d.ffn, d.d,
                                                       static_cast<const uint16_t*>(a), perm, 1, offs,
                                                       alist, nact, S);
            e = hipGetLastError();
            if (e != hipSuccess) return moe_hip_fail(e, "grouped up launch");
        }
        {
            ProfScope prof("moe_down", s, 0.0, 2.0 * M * k * (double)d.ffn * d.d);
            const uint16_t* wd = static_cast<const uint16_t*>(d.w_down) + (size_t)l * E * down_stride;
            if (p.act_tiled)
                launch_grouped<kEpiStore, true, false>(prof, M, E, k, listed, (d.d + 15) / 16, s, wd,
                                                down_stride, d.d, d.ffn,
                                                static_cast<const uint16_t*>(S), perm, 0, offs, alist,
                                                nact, Y);
            else
                launch_grouped<kEpiStore, false, false>(prof, M, E, k, listed, (d.d + 15) / 16, s, wd,
                                                 down_stride, d.d, d.ffn,
                                                 static_cast<const uint16_t*>(S), perm, 0, offs, alist,
                                                 nact, Y);
            e = hipGetLastError();
            if (e != hipSuccess) return moe_hip_fail(e, "grouped down launch");
        }
        MoeFold fold;
        fold.Y = Y;
        fold.wts = wts;
        fold.inv = inv;
        fold.k = k;
        e = launch_rmsnorm_moe(h, fold, d.gain + (size_t)(l + 1) * d.d, a, M, d.d, d.rms_eps,
                               l + 1 == d.n_layers && p.head_act_tiled, s);
        if (e != hipSuccess) return moe_hip_fail(e, "rmsnorm launch");
    }
    MatmulArgs hd{};
    hd.W = d.w_head;
    hd.act = a;
    hd.M = M; hd.N = d.vocab; hd.K = d.d;
    hd.epi = kEpiStore; hd.out = logits; hd.bf16 = 1; hd.tiled = 1;
    hd.act_tiled = p.head_act_tiled;
    e = launch_matmul(hd, p.head_kind, s);
    if (e != hipSuccess) return moe_hip_fail(e, "LM-head launch");
    return SV_OK;
}

}  // extern "C"
