// LDS-staged bf16 MFMA GEMM for the verification forward at large B*(K+1).
//
// Once B*(K+1) reaches the hundreds the product becomes a real contraction
// (p1 "Draft length and performance of linear layers": GEMM-M grows to
// M(1+D) and crosses from memory- to compute-bound), and the weights must be
// reused across many activation rows from on-chip memory instead of being
// streamed once per 64 rows.
//
// out^T tile [BN weight rows x BM activation rows] per workgroup.  Weights and
// activations are both in the matrix-core operand layout (16 x 32 blocks of
// one KiB in lane order; the activations are written that way, rows padded to
// 16, by the RMSNorm and by this kernel's SiLU epilogue), so each k step of
// 32 the workgroup's waves copy BN/16 + BM/16 contiguous KiB straight from
// global memory into LDS with global_load_lds_dwordx4, through a ring of NS
// stages (NS - 1 steps in flight).  Wave (wn, wm) then reads its FN weight
// and FM activation operands from LDS (contiguous 1 KiB each, no bank
// conflicts) and issues FN x FM v_mfma_f32_16x16x32_bf16.  The K range can be
// split; split results go to fp32 partial planes that the following RMSNorm
// folds in (in split order, so results are deterministic).
//
// Tile order: the grid is one-dimensional and workgroup i runs on XCD i % 8,
// so tiles are renumbered to give every XCD a contiguous run, activation
// tile fastest: the tiles that share one weight panel run together on one
// XCD and the panel is fetched into that XCD's L2 once, not once per
// activation tile (measured 1.8x on the LM head at 768 rows).
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int WN, int WM, int FN, int FM, int NS, int WPE, int EPI>
__global__ __launch_bounds__(WN * WM * kWave, WPE) void mfma_tiled_kernel(
    const uint16_t* __restrict__ Wt, const uint16_t* __restrict__ act, int M, int N, int K,
    int splits, int steps_per_split, void* __restrict__ out, size_t split_stride) {
    constexpr int NW = WN * WM;
    constexpr int BNF = WN * FN;                 // weight blocks (16 rows) per tile
    constexpr int BMF = WM * FM;                 // activation blocks (16 rows) per tile
    constexpr int FR = BNF + BMF;                // 1 KiB fragments per stage
    static_assert(FR % NW == 0, "every wave issues the same number of copies");
    constexpr int PER_WAVE = FR / NW;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS][FR * 512];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wn = wave / WM, wm = wave % WM;

    // XCD-contiguous renumbering of the G workgroups (XCD x = i % 8 gets
    // G/8 tiles, the first G%8 XCDs one more), then activation tile fastest,
    // K split next, weight tile slowest
    const int G = gridDim.x, L = blockIdx.x;
    const int q = G / 8, r = G % 8, x = L % 8, j = L / 8;
    const int t = x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
    const int MT = (M + BMF * 16 - 1) / (BMF * 16);
    const int tm = t % MT;
    const int split = (t / MT) % splits;
    const int tn = t / (MT * splits);
    const int nb0 = tn * BNF;                    // first 16-row weight block
    const int mb0 = tm * BMF;
    const int S = K / 32;
    const int s_begin = split * steps_per_split;
    const int s_end = min(S, s_begin + steps_per_split);
    const int nblk = (N + 15) / 16;              // weight blocks present in the tiled layout

    const int mblk = (M + 15) / 16;              // activation blocks (rows padded to 16)

    // global source of this lane's 16 bytes for fragment f at step s: block
    // row + 512 * s (weights and activations share the layout)
    const uint16_t* src[PER_WAVE];
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int f = wave + NW * i;
        if (f < BNF) src[i] = Wt + (size_t)min(nb0 + f, nblk - 1) * S * 512 + lane * 8;
        else src[i] = act + (size_t)min(mb0 + f - BNF, mblk - 1) * S * 512 + lane * 8;
    }
    auto issue = [&](int s) {
        const int st = (s - s_begin) % NS;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int f = wave + NW * i;
            __builtin_amdgcn_global_load_lds((const void*)(src[i] + (size_t)512 * s),
                                             (lds_void*)(&lds[st][f * 512]), 16, 0, 0);
        }
    };

    f32x4v acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (s_begin + p < s_end) issue(s_begin + p);

    for (int s = s_begin; s < s_end; ++s) {
        // the copies of step s are done once at most NS-2 later steps remain
        if (s + NS - 2 < s_end) wait_vmcnt<PER_WAVE * (NS - 2)>();
        else wait_vmcnt<0>();
        // A bare workgroup barrier: this wave's copies of step s are complete
        // (the wait above), every wave passes only after its own copies are,
        // and every wave has finished reading step s-1's stage.  (A fenced
        // barrier would also wait for the copies of later steps.)
        __builtin_amdgcn_s_barrier();
        if (s + NS - 1 < s_end) issue(s + NS - 1);
        const uint16_t* stage = lds[(s - s_begin) % NS];
        bf16x8 a[FN], b[FM];
#pragma unroll
        for (int i = 0; i < FN; ++i)
            a[i] = *reinterpret_cast<const bf16x8*>(stage + (wn * FN + i) * 512 + lane * 8);
#pragma unroll
        for (int j = 0; j < FM; ++j)
            b[j] = *reinterpret_cast<const bf16x8*>(stage + (BNF + wm * FM + j) * 512 + lane * 8);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }

    // epilogue: lane holds rows n = base + 4*(lane/16) + r, column m = lane % 16.
    // The SiLU output (next matmul's activations) is written in the operand
    // layout over all padded rows; the fp32 outputs row-major for m < M.
    const int mpad = mblk * 16;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        const int n = (nb0 + wn * FN + i) * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = (mb0 + wm * FM + j) * 16 + (lane & 15);
            const f32x4v v = acc[i][j];
            if constexpr (EPI == kEpiSilu) {
                // N % 32 == 0: the four outputs are 8 contiguous bytes of one block
                if (m >= mpad || n >= N) continue;
                const size_t o = ((size_t)(m >> 4) * (N >> 5) + (n >> 5)) * 512 +
                                 ((m & 15) + 16 * ((n & 31) >> 3)) * 8 + (n & 7);
                uint2 pk;
                pk.x = pack_bf16x2(silu(v[0]), silu(v[1]));
                pk.y = pack_bf16x2(silu(v[2]), silu(v[3]));
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = pk;
                continue;
            }
            if (m >= M) continue;
            float* dst = static_cast<float*>(out) + (EPI == kEpiResidual ? split * split_stride : 0);
            const size_t o0 = (size_t)m * N + n;
            if (n + 3 < N && (N & 3) == 0) {
                *reinterpret_cast<f32x4v*>(dst + o0) = v;   // four consecutive outputs of one row
                continue;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) dst[o0 + r] = v[r];
        }
    }
}

// Tile shapes (measured at 80 - 768 rows on the 8B-shaped matrices and the
// large-batch LM head, random operands, weights not cache-resident):
//  thin  - 2 x 2 waves of 32 x 32: 64 x 64 tiles, 3 stages of 8 KiB; the up
//          projection up to 128 rows (it cannot split K, so it needs narrow
//          tiles for enough workgroups)
//  tall  - 2 x 2 waves of 32 x 64: 64 x 128 tiles, 3 stages of 12 KiB; the up
//          projection at 129 - 256 rows
//  small - 2 x 2 waves of 64 x 64: 128 x 128 tiles, 3 stages of 16 KiB; the up
//          projection above 256 rows, the down projection (K split) and the
//          LM head up to 128 rows
//  wide  - 4 x 2 waves of 64 x 64: 256 x 128 tiles, 3 stages of 24 KiB, two
//          workgroups per CU; the down projection above 128 rows and the LM
//          head with many tiles
//  large - 2 x 4 waves of 128 x 64: 256 x 256 tiles, 4 stages of 32 KiB, one
//          workgroup per CU; the LM head of a large vocabulary at a few
//          hundred rows
// (WPE: waves per SIMD the register allocation must allow)
struct TileThin { static constexpr int WN = 2, WM = 2, FN = 2, FM = 2, NS = 3, WPE = 2; };
struct TileTall { static constexpr int WN = 2, WM = 2, FN = 2, FM = 4, NS = 3, WPE = 2; };
struct TileSmall { static constexpr int WN = 2, WM = 2, FN = 4, FM = 4, NS = 3, WPE = 2; };
struct TileWide { static constexpr int WN = 4, WM = 2, FN = 4, FM = 4, NS = 3, WPE = 2; };
struct TileLarge { static constexpr int WN = 2, WM = 4, FN = 8, FM = 4, NS = 4, WPE = 2; };

template <class T> constexpr int tile_n() { return T::WN * T::FN * 16; }
template <class T> constexpr int tile_m() { return T::WM * T::FM * 16; }
template <class T> long long tile_count(int M, int N) {
    return (long long)((N + tile_n<T>() - 1) / tile_n<T>()) * ((M + tile_m<T>() - 1) / tile_m<T>());
}

template <class T>
int splits_for(int M, int N, int K) {
    // enough workgroups for 256 CUs: split K when the tile grid is small
    const long long tiles = tile_count<T>(M, N);
    int splits = 1;
    while (tiles * splits < 256 && splits < 8 && (K / 32) / (splits * 2) >= 16) splits *= 2;
    return splits;
}

// The down projection's tile: 128 x 128 up to 128 rows, 256 x 128 above.
bool down_small(int M) { return M <= 128; }

}  // namespace

int tiled_splits(int M, int N, int K) {
    return down_small(M) ? splits_for<TileSmall>(M, N, K) : splits_for<TileWide>(M, N, K);
}

namespace {

template <class T, int EPI>
hipError_t launch_tile(const MatmulArgs& a, int splits, hipStream_t stream) {
    const int S = a.K / 32;
    const int sps = (S + splits - 1) / splits;
    const long long G = tile_count<T>(a.M, a.N) * splits;
    if (G > 0x7fffffff) return hipErrorInvalidValue;
    const size_t stride = (size_t)a.M * a.N;
    ProfScope prof(a.name, stream, matmul_bytes(a, a.M), 2.0 * a.M * (double)a.N * a.K);
    SV_LAUNCH(prof, (mfma_tiled_kernel<T::WN, T::WM, T::FN, T::FM, T::NS, T::WPE, EPI>), (unsigned)G,
              T::WN * T::WM * kWave, stream, static_cast<const uint16_t*>(a.W),
              static_cast<const uint16_t*>(a.act), a.M, a.N, a.K, splits, sps, a.out, stride);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const MatmulArgs& a, hipStream_t stream) {
    if constexpr (EPI == kEpiSilu) {
        if (a.M <= 128) return launch_tile<TileThin, EPI>(a, 1, stream);
        if (a.M <= 256) return launch_tile<TileTall, EPI>(a, 1, stream);
        return launch_tile<TileSmall, EPI>(a, 1, stream);
    } else if constexpr (EPI == kEpiResidual) {
        // only the down projection splits K; its split count sizes the
        // caller's partial planes (tiled_splits, same tile rule)
        const int splits = a.splits > 0 ? a.splits : 1;
        return down_small(a.M) ? launch_tile<TileSmall, EPI>(a, splits, stream)
                               : launch_tile<TileWide, EPI>(a, splits, stream);
    } else {
        if (a.M <= 128) return launch_tile<TileSmall, EPI>(a, 1, stream);
        if (tile_count<TileWide>(a.M, a.N) >= 1200) return launch_tile<TileWide, EPI>(a, 1, stream);
        if (tile_count<TileLarge>(a.M, a.N) >= 400) return launch_tile<TileLarge, EPI>(a, 1, stream);
        return launch_tile<TileWide, EPI>(a, 1, stream);
    }
}

}  // namespace

hipError_t launch_mfma_tiled(const MatmulArgs& a, hipStream_t stream) {
    if (!a.bf16 || !a.tiled || !a.act_tiled || a.K % 32) return hipErrorInvalidValue;
    if (a.epi == kEpiSilu && a.N % 32) return hipErrorInvalidValue;
    switch (a.epi) {
        case kEpiSilu: return launch_epi<kEpiSilu>(a, stream);
        case kEpiResidual: return launch_epi<kEpiResidual>(a, stream);
        case kEpiStore: return launch_epi<kEpiStore>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sv
