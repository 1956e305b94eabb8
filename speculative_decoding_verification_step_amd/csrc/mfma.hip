// bf16 MFMA matmuls out[m, n] = sum_k act[m, k] * W[n, k] on gfx950 matrix
// cores, for the verification forward at B*(K+1) = 1..64 rows per pass.
//
// The weights are the stream (read once, publishertech section 1 "The
// Speculative Cycle"); the activations are small and stay in L1/L2.  A wave
// owns RF 16-row weight fragments and one slice of the reduction dimension:
// it streams its fragments straight from HBM into registers (16 bytes per
// lane, double-buffered U steps deep) and feeds them to
// v_mfma_f32_16x16x32_bf16 as the A operand (rows = weight rows), with the
// activation rows as the B operand (columns = positions, 16 per fragment, MF
// fragments).  A workgroup holds NR row groups x NKS k slices of waves; the
// k slices are summed through LDS in a fixed order and the epilogue (SiLU +
// bf16, residual add, or fp32 store) is applied once per output.  The grid's
// y dimension can split K further; the down projection then writes fp32
// partial planes that the next RMSNorm folds in, in split order.
//
// Every weight fragment needs one 1 KiB load and every activation fragment
// another, so the activation loads per weight byte fall as MF / RF: one
// fragment per wave suits up to 8 rows, two suit 9..16 rows of a wide
// projection, eight 17..64 rows.
//
// Weights come either row-major or packed in the tiled layout of pack.hip,
// where each 16 x 32 operand block is one contiguous KiB in lane order (one
// wave load = one contiguous KiB; measured about 1.4x the row-major rate).
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int MF, int RF, int NR, int NKS, int U, int EPI, bool kTiled>
__global__ __launch_bounds__(NR * NKS * kWave) void mfma_skinny_kernel(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ act, int M, int N, int K,
    int steps_per_split, void* __restrict__ out, size_t split_stride) {
    static_assert(NKS >= 2, "the k slices are reduced through LDS");
    constexpr int NWK = NR * NKS;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int rg = wave % NR;           // row group of this wave
    const int ks = wave / NR;           // k slice of this wave
    const int r16 = lane & 15;          // row of the A fragment / column of B
    const int g = lane >> 4;            // which 8-element k slice of the step
    const int S = K / 32;
    const int nblk = (N + 15) / 16;     // 16-row fragments of W

    // the workgroup's k range (grid split), then this wave's slice of it
    const int gs0 = blockIdx.y * steps_per_split;
    const int len = max(min(S, gs0 + steps_per_split) - gs0, 0);
    const int s0 = gs0 + (int)((long long)len * ks / NKS);
    const int s1 = gs0 + (int)((long long)len * (ks + 1) / NKS);
    const int fb0 = (blockIdx.x * NR + rg) * RF;

    // weight operand of step s for fragment rf: wrow[rf] + wstep * s
    const uint16_t* wrow[RF];
    constexpr int wstep = kTiled ? 512 : 32;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        const int fb = min(fb0 + rf, nblk - 1);
        if constexpr (kTiled) {
            wrow[rf] = W + (size_t)fb * S * 512 + lane * 8;
        } else {
            const int n = min(fb * 16 + r16, N - 1);
            wrow[rf] = W + (size_t)n * K + 8 * g;
        }
    }
    const uint16_t* arow[MF];
    bool aval[MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
        const int m = mf * 16 + r16;
        aval[mf] = m < M;
        arow[mf] = act + (size_t)min(m, M - 1) * K + 8 * g;
    }

    f32x4v acc[RF][MF];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) acc[rf][mf] = f32x4v{0.f, 0.f, 0.f, 0.f};

    bf16x8 wa[U][RF], wb[U][RF], xa[U][MF], xb[U][MF];
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

    auto load = [&](bf16x8 (&w)[U][RF], bf16x8 (&x)[U][MF], int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ss = s + u;
            const bool in = ss < s1;
            const int k = 32 * ss;
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
                x[u][mf] = (in && aval[mf]) ? *reinterpret_cast<const bf16x8*>(arow[mf] + k) : zero8;
#pragma unroll
            for (int rf = 0; rf < RF; ++rf)
                w[u][rf] = in ? __builtin_nontemporal_load(
                                    reinterpret_cast<const bf16x8*>(wrow[rf] + (size_t)wstep * ss))
                              : zero8;
        }
    };
    auto compute = [&](const bf16x8 (&w)[U][RF], const bf16x8 (&x)[U][MF]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int rf = 0; rf < RF; ++rf)
#pragma unroll
                for (int mf = 0; mf < MF; ++mf)
                    acc[rf][mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[u][rf], x[u][mf],
                                                                           acc[rf][mf], 0, 0, 0);
    };

    load(wa, xa, s0);
    for (int s = s0; s < s1; s += 2 * U) {
        load(wb, xb, s + U);
        compute(wa, xa);
        load(wa, xa, s + 2 * U);
        compute(wb, xb);
    }

    // fixed-order reduction of the NKS k slices through LDS, one weight
    // fragment of every row group at a time
    __shared__ float red[NKS][NR][MF][4][kWave];
    float* plane = static_cast<float*>(out) + (size_t)blockIdx.y * split_stride;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        if (rf) __syncthreads();        // the previous fragment's readers are done
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[ks][rg][mf][r][lane] = acc[rf][mf][r];
        __syncthreads();
        constexpr int kOut = 256 * MF * NR;
        for (int e = threadIdx.x; e < kOut; e += NWK * kWave) {
            const int i = e & 15;                 // row within the 16-row fragment
            const int j = (e >> 4) & 15;          // column (position) within the fragment
            const int mf = (e >> 8) % MF;
            const int rr = (e >> 8) / MF;
            const int n = ((blockIdx.x * NR + rr) * RF + rf) * 16 + i;
            const int m = mf * 16 + j;
            if (n >= N || m >= M) continue;
            const int r = i & 3, l = ((i >> 2) << 4) + j;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < NKS; ++w) v += red[w][rr][mf][r][l];
            const size_t o = (size_t)m * N + n;
            if constexpr (EPI == kEpiSilu) {
                static_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(silu(v));
            } else if constexpr (EPI == kEpiResidual) {
                if (split_stride) plane[o] = v;            // partial plane of this K split
                else static_cast<float*>(out)[o] += v;     // one owner per element
            } else {
                static_cast<float*>(out)[o] = v;
            }
        }
    }
}

// Wave arrangements (measured on the tiled layout at 5, 40 and 64 rows and the
// 8B/70B-share matrix shapes).
enum SkinnyCfg : int {
    kCfg1 = 0,     // RF 1, 8 k slices, 4-step buffers: up to 8 rows (16 when N < 8192), and row-major W
    kCfg4 = 1,     // RF 4, 4 k slices, 2-step buffers: 17..64 rows, few output rows
    kCfg8 = 2,     // RF 8, 4 k slices, 1-step buffers: 17..64 rows
    kCfg8R2 = 3,   // RF 8, 2 row groups x 2 k slices: 17..64 rows, very many output rows
};

int skinny_cfg(int MF, int N, int epi, int tiled) {
    if (MF == 1 || !tiled) return kCfg1;
    if (epi == kEpiResidual) return kCfg8;      // the grid K split supplies the workgroups
    if (epi == kEpiStore && (N + 255) / 256 >= 400) return kCfg8R2;
    return (N + 127) / 128 >= 200 ? kCfg8 : kCfg4;
}

template <int MF, int RF, int NR, int NKS, int U, int EPI>
hipError_t launch_shape(const MatmulArgs& a, const uint16_t* act, void* out, int Mc, int ksg,
                        size_t stride, hipStream_t stream) {
    const int rows = 16 * RF * NR;
    const dim3 grid((a.N + rows - 1) / rows, ksg);
    const int S = a.K / 32;
    const int sps = (S + ksg - 1) / ksg;
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    ProfScope prof(a.name, stream, matmul_bytes(a, Mc), 2.0 * Mc * (double)a.N * a.K);
    if (a.tiled) {
        SV_LAUNCH(prof, (mfma_skinny_kernel<MF, RF, NR, NKS, U, EPI, true>), grid,
                  NR * NKS * kWave, stream, W, act, Mc, a.N, a.K, sps, out, stride);
    } else if constexpr (RF == 1) {
        SV_LAUNCH(prof, (mfma_skinny_kernel<MF, RF, NR, NKS, U, EPI, false>), grid,
                  NR * NKS * kWave, stream, W, act, Mc, a.N, a.K, sps, out, stride);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int MF, int EPI>
hipError_t launch_mf(const MatmulArgs& a, const uint16_t* act, void* out, int Mc, int ksg,
                     size_t stride, hipStream_t stream) {
    if constexpr (MF == 1) {
        // 9..16 rows: every activation load is as large as the weight load
        // it meets, so wide projections share it between two fragments
        if (Mc > 8 && a.N >= 8192 && a.tiled)
            return launch_shape<1, 2, 1, 4, 4, EPI>(a, act, out, Mc, ksg, stride, stream);
        return launch_shape<1, 1, 1, 8, 4, EPI>(a, act, out, Mc, ksg, stride, stream);
    }
    switch (skinny_cfg(MF, a.N, EPI, a.tiled)) {
        case kCfg1: return launch_shape<MF, 1, 1, 8, 4, EPI>(a, act, out, Mc, ksg, stride, stream);
        case kCfg4:
            if constexpr (EPI != kEpiResidual)
                return launch_shape<MF, 4, 1, 4, 2, EPI>(a, act, out, Mc, ksg, stride, stream);
            return hipErrorInvalidValue;
        case kCfg8: return launch_shape<MF, 8, 1, 4, 1, EPI>(a, act, out, Mc, ksg, stride, stream);
        default:
            if constexpr (EPI == kEpiStore)
                return launch_shape<MF, 8, 2, 2, 1, EPI>(a, act, out, Mc, ksg, stride, stream);
            return hipErrorInvalidValue;
    }
}

template <int EPI>
hipError_t launch_skinny_epi(const MatmulArgs& a, hipStream_t stream) {
    const size_t out_es = EPI == kEpiSilu ? 2 : 4;
    // down projection with a K split: `splits` partial planes of [M, N]
    const bool planes = EPI == kEpiResidual && a.splits > 0;
    const int ksg = planes ? a.splits : 1;
    const size_t stride = planes ? (size_t)a.M * a.N : 0;
    for (int mb = 0; mb < a.M; mb += 64) {
        const int Mc = a.M - mb < 64 ? a.M - mb : 64;
        const uint16_t* act = static_cast<const uint16_t*>(a.act) + (size_t)mb * a.K;
        void* out = static_cast<char*>(a.out) + (size_t)mb * a.N * out_es;
        hipError_t e;
        switch ((Mc + 15) / 16) {
            case 1: e = launch_mf<1, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 2: e = launch_mf<2, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 3: e = launch_mf<3, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            default: e = launch_mf<4, EPI>(a, act, out, Mc, ksg, stride, stream); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int skinny_splits(int M, int N, int K, int tiled) {
    // 17+ rows run eight fragments per wave, so a d-row down projection has
    // few workgroups: split K until the grid fills 256 CUs (>= 16 steps of 32
    // per split half, so every k slice keeps a few steps)
    if (!tiled || M <= 16) return 0;
    const long long wg = (N + 127) / 128;
    int ksg = 1;
    while (wg * ksg < 256 && ksg < 8 && (K / 32) / (ksg * 2) >= 16) ksg *= 2;
    return ksg > 1 ? ksg : 0;
}

hipError_t launch_mfma_skinny(const MatmulArgs& a, hipStream_t stream) {
    if (!a.bf16 || a.K % 32) return hipErrorInvalidValue;
    switch (a.epi) {
        case kEpiSilu: return launch_skinny_epi<kEpiSilu>(a, stream);
        case kEpiResidual: return launch_skinny_epi<kEpiResidual>(a, stream);
        case kEpiStore: return launch_skinny_epi<kEpiStore>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sv
