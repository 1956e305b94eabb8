// Causal attention of the T = K + 1 verified positions over a paged KV cache,
// the append of their keys/values, and the commit after acceptance (C ABI in
// include/spec_verify_attn.h).
//
// The target scores every drafted slot in one pass (NVIDIA co-design post,
// "What is speculative decoding?"; its "Draft length and attention
// performance": with G query heads per KV head the attention GEMM-M is
// G (1 + D)).  A wave owns tiles of 16 of the G*T query rows of one
// (request, KV head) and one range of KV blocks; both products run on the
// matrix cores with the keys as the row dimension:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims of a block
//                 (contiguous in k_cache), B = Q^T (each lane's query row);
//   O^T += V^T P^T  A = V^T (16 dims x 32 keys; V is stored transposed per
//                 block), B = P^T.
// In the MFMA output layout a lane holds four keys of S^T for one query row,
// and its eight probabilities (two key tiles) are exactly the B operand of
// the second product once the 32 k slots are ordered (keys 4g..4g+3 of tile
// 0, then keys 16+4g..16+4g+3 of tile 1) - the A operand V^T uses the same
// order - so the softmax needs no transpose and no LDS; each query row's
// running max and sum are shared by its four lane groups through two
// shuffles.  The four waves of a workgroup walk the same blocks of one
// context range, which pass once through an LDS ring (attn_ring_kernel);
// long contexts are further split over workgroups (flash-decoding style) and
// the partial states are merged in a second kernel in split order.  Probabilities enter
// the second product rounded to bf16 and the softmax sum is taken over the
// same rounded values, so every output row is a convex combination of the
// visible value rows.
#include <math.h>

#include "common.hpp"
#include "host.hpp"
#include "kernels.hpp"
#include "spec_verify.h"
#include "spec_verify_attn.h"

namespace sv {
namespace {

constexpr int kBlk = SV_KV_BLOCK;
constexpr int kWavesPerGroup = 4;
constexpr int kTargetUnits = 512;     // workgroups the context split aims for (2 per CU)
constexpr int kMinBlocksPerSplit = 8; // KV blocks per context split at least
constexpr float kLazyMargin = 8.0f;   // log2 units a score may exceed the running max by

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Query tiles (16 rows each) per wave: four waves of QTW tiles share one
// pass of every block (QTW 1 or 2 at head_dim 128, up to 4 at 64; with fewer
// tiles than waves the spare waves only help copy).  Measured against a
// kernel in which every wave streamed its own blocks into registers (next
// block in flight), the ring was 0-8% faster with one tile per KV head and
// 4-12% faster with two (8B heads, B = 1 over 32K: 37.1 -> 34.3 us at K = 0,
// 43.5 -> 38.3 us at K = 7).
int ring_tiles_per_wave(int nq, int Dh) {
    const int want = (nq + kWavesPerGroup - 1) / kWavesPerGroup;
    if (want <= 1) return 1;
    if (want <= 2 || Dh == 128) return 2;
    return 4;
}

struct AttnPlan {
    int G = 0, nq = 0, qt = 1, nqg = 0, nsplit = 1, bps = 0;
    long long units = 0;     // workgroups: (request, KV head, split, group of qt tiles)
    long long rows16 = 0;    // 16-row partial-state slots: (request, KV head, split, tile)
    size_t ws_bytes = 0;
};

AttnPlan plan_attention(int B, int T, int Hq, int Hkv, int Dh, int max_blocks) {
    AttnPlan p;
    p.G = Hq / Hkv;
    p.nq = (p.G * T + 15) / 16;
    p.qt = ring_tiles_per_wave(p.nq, Dh);
    const int group = kWavesPerGroup * p.qt;    // tiles per workgroup
    p.nqg = (p.nq + group - 1) / group;
    const long long base = (long long)B * Hkv * p.nqg;
    long long ns = (kTargetUnits + base - 1) / base;
    ns = ns < 1 ? 1 : ns;
    const long long cap = max_blocks / kMinBlocksPerSplit > 0 ? max_blocks / kMinBlocksPerSplit : 1;
    ns = ns > cap ? cap : ns;
    p.bps = (int)((max_blocks + ns - 1) / ns);
    p.nsplit = (max_blocks + p.bps - 1) / p.bps;
    p.units = base * p.nsplit;
    p.rows16 = (long long)B * Hkv * p.nq * p.nsplit;
    // partial output rows (16 per tile and split) and their (max, sum) pairs
    p.ws_bytes = p.nsplit > 1 ? (size_t)p.rows16 * 16 * (Dh + 2) * 4 : 0;
    return p;
}

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* table;
    const int32_t* ctx;
    int B, T, Hq, Hkv, max_blocks, num_blocks, nq, nqg, nsplit, bps;
    float scale_log2;     // softmax scale times log2(e): scores in the exp2 domain
    float* part_o;        // [rows16*16, Dh] unnormalised partial outputs (split runs)
    float* part_ml;       // [rows16*16, 2] partial (max, sum)
    float* out;           // [B, T, Hq, Dh]
};

__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

// Entry kb of a request's block-table row (row and kb the same for the whole
// wave).  The table is read-only while attention runs, so the lookup goes
// through the constant address space: a scalar load, counted on lgkmcnt.  As
// a vector load its wait (vmcnt, which retires in order) would also wait for
// every K/V copy issued before it, taking the prefetch depth away.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int table_entry(const int32_t* row, int kb) {
    return ((const const_i32*)row)[__builtin_amdgcn_readfirstlane(kb)];
}

// The four waves own QTW tiles each (4 * QTW tiles = up to 128 query rows per
// workgroup; tiles past the last one are skipped) and walk the SAME blocks of the
// context range, which pass once through a ring of kRingStages LDS stages
// (global_load_lds_dwordx4) two blocks at a time: the next pair's copies are
// in flight while a pair is used, paced by vmcnt and one bare barrier per pair
// (halving the barriers against one block per step: 4-7% faster at 64-128
// query rows per KV head).  A stage holds the block in operand order: the K
// tiles as 1 KiB MFMA fragments (lane l: key 16 kt + l % 16, dims 32 s + 8 (l
// / 16)), then the V^T tiles as 64 16-byte chunks (row c of the tile, keys 8 k
// .. 8 k + 7) with the chunk index XORed by (c / 4) % 4, so each lane's two
// 8-byte halves are read without bank conflicts.  Each wave then finishes its
// own rows over the whole range: no merge between waves.
constexpr int kRingStages = 4;

template <int DH, bool kDirect, int QTW>
__global__ __launch_bounds__(kWavesPerGroup * kWave, QTW <= 2 ? 2 : 1) void attn_ring_kernel(AttnArgs a) {
    constexpr int KS = DH / 32;
    constexpr int DT = DH / 16;
    constexpr int NF = 2 * KS + DT;                    // 1 KiB fragments per block
    static_assert(NF % kWavesPerGroup == 0, "every wave issues the same number of copies");
    constexpr int PER_WAVE = NF / kWavesPerGroup;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[kRingStages][NF * 512];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wg = blockIdx.x, Gn = gridDim.x;
    const int q8 = Gn / 8, r8 = Gn % 8, x8 = wg % 8, j8 = wg / 8;
    const long long unit = x8 < r8 ? x8 * (q8 + 1) + j8 : r8 * (q8 + 1) + (x8 - r8) * q8 + j8;
    const int qg = (int)(unit % a.nqg);
    long long rest = unit / a.nqg;
    const int sp = (int)(rest % a.nsplit);
    rest /= a.nsplit;
    const int kvh = (int)(rest % a.Hkv);
    const int b = (int)(rest / a.Hkv);
    const int G = a.Hq / a.Hkv;
    const int c = lane & 15, g = lane >> 4;
    const int cap = a.max_blocks * kBlk;
    const int ctx = clamp_ctx(a.ctx[b], cap);
    const int n_all = min(ctx + a.T, cap);
    const int kb0 = sp * a.bps;
    const int kb_end = min((n_all + kBlk - 1) / kBlk, (sp + 1) * a.bps);
    const int nblk = kb_end > kb0 ? kb_end - kb0 : 0;

    int t[QTW], h[QTW], vis[QTW];
    bool row_ok[QTW], tile_ok[QTW];
#pragma unroll
    for (int i = 0; i < QTW; ++i) {
        const int qt = (qg * kWavesPerGroup + wave) * QTW + i;
        const int r = qt * 16 + c;
        tile_ok[i] = qt < a.nq;
        row_ok[i] = r < G * a.T;
        t[i] = row_ok[i] ? r / G : 0;
        h[i] = kvh * G + r % G;
        vis[i] = row_ok[i] ? min(ctx + t[i] + 1, cap) : 0;
    }
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    bf16x8 qv[QTW][KS];
#pragma unroll
    for (int i = 0; i < QTW; ++i) {
        const uint16_t* qrow = a.q + (((size_t)b * a.T + t[i]) * a.Hq + (h[i] < a.Hq ? h[i] : 0)) * DH;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qv[i][s] = row_ok[i] ? *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * g) : zero8;
    }
    float m[QTW], lpart[QTW];
    f32x4v acc[QTW][DT];
#pragma unroll
    for (int i = 0; i < QTW; ++i) {
        m[i] = -INFINITY;
        lpart[i] = 0.f;
#pragma unroll
        for (int u = 0; u < DT; ++u) acc[i][u] = f32x4v{0.f, 0.f, 0.f, 0.f};
    }

    // copies of block kb into stage st: fragment f = wave + 4 j of the block
    const int32_t* trow = a.table + (size_t)b * a.max_blocks;
    const int vrow_c = lane >> 2;                              // V chunk copy: tile row
    const int vchunk = (lane & 3) ^ ((vrow_c >> 2) & 3);       // ... and its swizzled chunk
    auto issue = [&](int blk, int st) {
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        const uint16_t* kbase = a.kc + ((size_t)blk * a.Hkv + kvh) * kBlk * DH;
        const uint16_t* vbase = a.vc + ((size_t)blk * a.Hkv + kvh) * DH * kBlk;
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int f = wave + kWavesPerGroup * j;
            const uint16_t* src;
            if (f < 2 * KS) {
                const int kt = f / KS, s = f % KS;
                src = kbase + (16 * kt + c) * DH + 32 * s + 8 * g;
            } else {
                const int u = f - 2 * KS;
                src = vbase + (16 * u + vrow_c) * kBlk + 8 * vchunk;
            }
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)&ring[st][f * 512], 16, 0, 0);
        }
    };

    // blocks go through the ring two at a time, one wait and one barrier per
    // pair: the copies of pair i + 2 are in flight while pair i is used.  The
    // ids of the next pair are read one pair ahead, so their scalar loads have
    // landed by the time the copies are issued.
    if (0 < nblk) issue(table_entry(trow, kb0), 0);
    if (1 < nblk) issue(table_entry(trow, kb0 + 1), 1);
    int next_blk = 2 < nblk ? table_entry(trow, kb0 + 2) : 0;
    int next_blk2 = 3 < nblk ? table_entry(trow, kb0 + 3) : 0;
    const int sw = (c >> 2) & 3;
    for (int i = 0; i < nblk; ++i) {
        if ((i & 1) == 0) {
            // only this pair's copies are in flight; the barrier also means
            // every wave is done with the pair the next copies overwrite
            wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            if (i + 2 < nblk) issue(next_blk, (i + 2) % kRingStages);
            if (i + 3 < nblk) issue(next_blk2, (i + 3) % kRingStages);
            if (i + 4 < nblk) next_blk = table_entry(trow, kb0 + i + 4);
            if (i + 5 < nblk) next_blk2 = table_entry(trow, kb0 + i + 5);
        }
        const uint16_t* stage = ring[i % kRingStages];
        bf16x8 k0[KS], k1[KS], v[DT];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            k0[s] = *reinterpret_cast<const bf16x8*>(stage + s * 512 + lane * 8);
            k1[s] = *reinterpret_cast<const bf16x8*>(stage + (KS + s) * 512 + lane * 8);
        }
#pragma unroll
        for (int u = 0; u < DT; ++u) {
            const uint16_t* vf = stage + (2 * KS + u) * 512;
            const uint2 lo = *reinterpret_cast<const uint2*>(vf + (c * 4 + ((g >> 1) ^ sw)) * 8 + 4 * (g & 1));
            const uint2 hi = *reinterpret_cast<const uint2*>(vf + (c * 4 + ((2 + (g >> 1)) ^ sw)) * 8 + 4 * (g & 1));
            v[u] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
        const int kb = kb0 + i;
#pragma unroll
        for (int q = 0; q < QTW; ++q) {
            if (!tile_ok[q]) continue;                         // uniform over the wave
            f32x4v s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[s], qv[q][s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[s], qv[q][s], s1, 0, 0, 0);
            }
            const int p0 = kb * kBlk + 4 * g;
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = p0 + j < vis[q] ? s0[j] * a.scale_log2 : -INFINITY;
                x[4 + j] = p0 + 16 + j < vis[q] ? s1[j] * a.scale_log2 : -INFINITY;
            }
            float lm = x[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) lm = fmaxf(lm, x[j]);
            // Lazy running max: the reference m (equal in the row's four lane
            // groups) moves only when some score exceeds it by more than
            // kLazyMargin (log2 units), found with one wave-wide vote; the
            // exact row max and the rescale then run.  Otherwise p <= 2^margin
            // and no cross-lane exchange is needed; the sum stays per lane group.
            if (__ballot(lm > m[q] + kLazyMargin)) {
                float bm = fmaxf(lm, __shfl_xor(lm, 16, kWave));
                bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
                const float mn = fmaxf(m[q], bm);
                const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[q] - mn);
                lpart[q] *= alpha;
#pragma unroll
                for (int u = 0; u < DT; ++u) acc[q][u] *= alpha;
                m[q] = mn;
            }
            const float mref = m[q] == -INFINITY ? 0.f : m[q];
            uint32_t pw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pw[j] = pack_bf16x2(__builtin_amdgcn_exp2f(x[2 * j] - mref),
                                    __builtin_amdgcn_exp2f(x[2 * j + 1] - mref));
                lpart[q] += bf16lo(pw[j]);     // in key order, as the product sums them
                lpart[q] += bf16hi(pw[j]);
            }
            const bf16x8 pv = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
            for (int u = 0; u < DT; ++u)
                acc[q][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[u], pv, acc[q][u], 0, 0, 0);
        }
    }

    // every wave finishes its own tiles: lane holds O^T[dim 16u+4g+j][row] in
    // acc[q][u][j], its row's m, and a quarter of its row's sum
#pragma unroll
    for (int q = 0; q < QTW; ++q) {
        if (!tile_ok[q]) continue;
        float l = lpart[q] + __shfl_xor(lpart[q], 16, kWave);
        l += __shfl_xor(l, 32, kWave);
        const int qt = (qg * kWavesPerGroup + wave) * QTW + q;
        const long long slot = (((long long)b * a.Hkv + kvh) * a.nsplit + sp) * a.nq + qt;
        const size_t prow = (size_t)slot * 16 + c;
        if constexpr (kDirect) {
            if (row_ok[q]) {
                const float inv = l > 0.f ? 1.0f / l : 0.f;
                float* orow = a.out + (((size_t)b * a.T + t[q]) * a.Hq + h[q]) * DH + 4 * g;
#pragma unroll
                for (int u = 0; u < DT; ++u) *reinterpret_cast<f32x4v*>(orow + 16 * u) = acc[q][u] * inv;
            }
        } else {
#pragma unroll
            for (int u = 0; u < DT; ++u)
                *reinterpret_cast<f32x4v*>(a.part_o + prow * DH + 16 * u + 4 * g) = acc[q][u];
            if (g == 0) {
                a.part_ml[2 * prow] = m[q];
                a.part_ml[2 * prow + 1] = l;
            }
        }
    }
}

// Merge the context splits of every query row, in split order:
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
template <int DH>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;   // (row unit group, row, dim/4)
    const int d4 = (int)(idx % (DH / 4));
    long long rest = idx / (DH / 4);
    const int c = (int)(rest % 16);
    rest /= 16;
    const int qt = (int)(rest % a.nq);
    const long long bk = rest / a.nq;                                    // b * Hkv + kvh
    if (bk >= (long long)a.B * a.Hkv) return;
    const int G = a.Hq / a.Hkv;
    const int r = qt * 16 + c;
    if (r >= G * a.T) return;
    const int kvh = (int)(bk % a.Hkv), b = (int)(bk / a.Hkv);
    const int t = r / G, h = kvh * G + r % G;
    float M = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < a.nsplit; ++s) {
        const size_t prow = ((size_t)(bk * a.nsplit + s) * a.nq + qt) * 16 + c;
        M = fmaxf(M, a.part_ml[2 * prow]);
    }
    f32x4v o = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
        for (int s = 0; s < a.nsplit; ++s) {
            const size_t prow = ((size_t)(bk * a.nsplit + s) * a.nq + qt) * 16 + c;
            const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * prow] - M);
            L += w * a.part_ml[2 * prow + 1];
            o += w * *reinterpret_cast<const f32x4v*>(a.part_o + prow * DH + 4 * d4);
        }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    *reinterpret_cast<f32x4v*>(a.out + (((size_t)b * a.T + t) * a.Hq + h) * DH + 4 * d4) = o * inv;
}

template <int DH>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctx_len, int B, int T, int Hkv, int max_blocks, int num_blocks) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;    // (b, t, kvh, dim)
    const long long total = (long long)B * T * Hkv * DH;
    if (idx >= total) return;
    const int d = (int)(idx % DH);
    long long rest = idx / DH;
    const int kvh = (int)(rest % Hkv);
    rest /= Hkv;
    const int t = (int)(rest % T);
    const int b = (int)(rest / T);
    const int cap = max_blocks * kBlk;
    const int p = clamp_ctx(ctx_len[b], cap) + t;
    if (p >= cap) return;
    int blk = table[(size_t)b * max_blocks + p / kBlk];
    blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
    const int slot = p % kBlk;
    kc[(((size_t)blk * Hkv + kvh) * kBlk + slot) * DH + d] = k_new[idx];
    vc[(((size_t)blk * Hkv + kvh) * DH + d) * kBlk + slot] = v_new[idx];
}

__global__ void kv_commit_kernel(int32_t* ctx_len, const int32_t* accept_len, int B) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b < B && accept_len[b] >= 1) ctx_len[b] += accept_len[b];
}

int check_shapes(int B, int T, int Hq, int Hkv, int Dh, int max_blocks, int num_blocks) {
    if (B < 0 || T < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv)
        return fail(SV_ERR_INVALID_ARG, "attention: need B >= 0, T >= 1, Hq a multiple of Hkv >= 1");
    if (Dh != 64 && Dh != 128) return fail(SV_ERR_UNSUPPORTED, "attention: head_dim must be 64 or 128");
    if (max_blocks < 1 || num_blocks < 1)
        return fail(SV_ERR_INVALID_ARG, "attention: max_blocks and num_blocks must be >= 1");
    if ((long long)max_blocks * kBlk > (1 << 30))
        return fail(SV_ERR_INVALID_ARG, "attention: max_blocks too large");
    return SV_OK;
}

int launch_fail(hipError_t e, const char* what) {
    return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

size_t spec_verify_attention_workspace_bytes(int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                                             int32_t head_dim, int32_t max_blocks) {
    if (check_shapes(B, T, Hq, Hkv, head_dim, max_blocks, 1) != SV_OK || B == 0) return 0;
    const size_t bytes = plan_attention(B, T, Hq, Hkv, head_dim, max_blocks).ws_bytes;
    return bytes ? (bytes + 255) / 256 * 256 : 0;
}

int spec_verify_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          const int32_t* block_table, const int32_t* ctx_len, int32_t B, int32_t T,
                          int32_t Hkv, int32_t head_dim, int32_t max_blocks, int32_t num_blocks,
                          hipStream_t stream) {
    int rc = check_shapes(B, T, Hkv, Hkv, head_dim, max_blocks, num_blocks);
    if (rc != SV_OK) return rc;
    if (B == 0) return SV_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !ctx_len)
        return fail(SV_ERR_INVALID_ARG, "kv_append: null pointer");
    const long long total = (long long)B * T * Hkv * head_dim;
    const unsigned grid = (unsigned)((total + 255) / 256);
    ProfScope prof("kv_append", stream, 2.0 * total * 2 * 2, 0.0);
    const uint16_t* kn = static_cast<const uint16_t*>(k_new);
    const uint16_t* vn = static_cast<const uint16_t*>(v_new);
    uint16_t* kc = static_cast<uint16_t*>(k_cache);
    uint16_t* vc = static_cast<uint16_t*>(v_cache);
    if (head_dim == 128)
        SV_LAUNCH(prof, kv_append_kernel<128>, grid, 256, stream, kn, vn, kc, vc, block_table,
                  ctx_len, B, T, Hkv, max_blocks, num_blocks);
    else
        SV_LAUNCH(prof, kv_append_kernel<64>, grid, 256, stream, kn, vn, kc, vc, block_table,
                  ctx_len, B, T, Hkv, max_blocks, num_blocks);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : launch_fail(e, "kv_append launch");
}

int spec_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* ctx_len, int32_t B, int32_t T,
                          int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t max_blocks,
                          int32_t num_blocks, float scale, float* out, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
    int rc = check_shapes(B, T, Hq, Hkv, head_dim, max_blocks, num_blocks);
    if (rc != SV_OK) return rc;
    if (B == 0) return SV_OK;
    if (!q || !k_cache || !v_cache || !block_table || !ctx_len || !out)
        return fail(SV_ERR_INVALID_ARG, "attention: null pointer");
    if (!isfinite(scale)) return fail(SV_ERR_INVALID_ARG, "attention: scale must be finite");
    const AttnPlan p = plan_attention(B, T, Hq, Hkv, head_dim, max_blocks);
    if (p.ws_bytes && (!ws || ws_bytes < p.ws_bytes))
        return fail(SV_ERR_WORKSPACE, "attention: workspace of %zu bytes needed, %zu given",
                    p.ws_bytes, ws_bytes);
    AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.kc = static_cast<const uint16_t*>(k_cache);
    a.vc = static_cast<const uint16_t*>(v_cache);
    a.table = block_table;
    a.ctx = ctx_len;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv;
    a.max_blocks = max_blocks; a.num_blocks = num_blocks;
    a.nq = p.nq; a.nqg = p.nqg; a.nsplit = p.nsplit; a.bps = p.bps;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = out;
    if (p.nsplit > 1) {
        a.part_o = static_cast<float*>(ws);
        a.part_ml = a.part_o + (size_t)p.rows16 * 16 * head_dim;
    }
    const unsigned grid = (unsigned)p.units;
    // algorithmic bytes: every visible key and value once per (request, KV head) at the
    // table's capacity, queries and outputs once
    const double kv_bytes = (double)B * Hkv * max_blocks * kBlk * head_dim * 2 * 2;
    const double flops = 4.0 * B * Hq * T * (double)max_blocks * kBlk * head_dim;
    {
        ProfScope prof("attention", stream, kv_bytes + (double)B * T * Hq * head_dim * 6, flops);
#define SV_RING(DH, DIRECT, QTW)                                                            \
        SV_LAUNCH(prof, (attn_ring_kernel<DH, DIRECT, QTW>), grid, kWavesPerGroup * kWave, stream, a)
#define SV_RING_128(DIRECT)                                                                 \
        if (p.qt == 1) SV_RING(128, DIRECT, 1); else SV_RING(128, DIRECT, 2);
#define SV_RING_64(DIRECT)                                                                  \
        if (p.qt == 1) SV_RING(64, DIRECT, 1);                                              \
        else if (p.qt == 2) SV_RING(64, DIRECT, 2);                                         \
        else SV_RING(64, DIRECT, 4);
        if (head_dim == 128) {
            if (p.nsplit > 1) { SV_RING_128(false) } else { SV_RING_128(true) }
        } else {
            if (p.nsplit > 1) { SV_RING_64(false) } else { SV_RING_64(true) }
        }
#undef SV_RING_64
#undef SV_RING_128
#undef SV_RING
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return launch_fail(e, "attention launch");
    if (p.nsplit > 1) {
        const long long threads = (long long)B * Hkv * p.nq * 16 * (head_dim / 4);   // (request, KV head, tile, row, dim/4)
        const unsigned cgrid = (unsigned)((threads + 255) / 256);
        ProfScope prof("attention_combine", stream,
                       (double)p.rows16 * 16 * (head_dim + 2) * 4 + (double)B * T * Hq * head_dim * 4,
                       0.0);
        if (head_dim == 128)
            SV_LAUNCH(prof, attn_combine_kernel<128>, cgrid, 256, stream, a);
        else
            SV_LAUNCH(prof, attn_combine_kernel<64>, cgrid, 256, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return launch_fail(e, "attention combine launch");
    }
    return SV_OK;
}

int spec_verify_kv_commit(int32_t* ctx_len, const int32_t* accept_len, int32_t B,
                          hipStream_t stream) {
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "kv_commit: B < 0");
    if (B == 0) return SV_OK;
    if (!ctx_len || !accept_len) return fail(SV_ERR_INVALID_ARG, "kv_commit: null pointer");
    ProfScope prof("kv_commit", stream, (double)B * 12, 0.0);
    SV_LAUNCH(prof, kv_commit_kernel, (B + 255) / 256, 256, stream, ctx_len, accept_len, B);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : launch_fail(e, "kv_commit launch");
}

}  // extern "C"
