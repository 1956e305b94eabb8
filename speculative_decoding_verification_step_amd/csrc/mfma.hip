// bf16 MFMA matmuls out[m, n] = sum_k act[m, k] * W[n, k] on gfx950 matrix
// cores, for the verification forward at B*(K+1) = 1..64 rows per pass.
//
// The weights are the stream (read once, publishertech section 1 "The
// Speculative Cycle"); the activations are small and stay in L1/L2.  One
// workgroup owns 16 * RF weight rows; its NWK waves split the reduction
// dimension, each streaming its share of the rows straight from HBM into
// registers (16 bytes per lane, double-buffered U steps deep) and feeding
// them to v_mfma_f32_16x16x32_bf16 as the A operand (rows = weight rows),
// with the activation rows as the B operand (columns = positions, 16 per
// fragment, MF fragments).  The matrix cores do the k reduction; the NWK
// partial tiles are summed through LDS in a fixed order and the epilogue
// (SiLU + bf16, residual add, or fp32 store) is applied once per output.
//
// Weights come either row-major or packed in the tiled layout of pack.hip,
// where each 16 x 32 operand block is one contiguous KiB in lane order (one
// wave load = one contiguous KiB; measured about 1.4x the row-major rate).
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kSteps = 4;   // 32-wide k steps per buffer (double-buffered)

template <int MF, int RF, int NWK, int EPI, bool kTiled>
__global__ __launch_bounds__(NWK * kWave) void mfma_skinny_kernel(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ act, int M, int N, int K,
    void* __restrict__ out) {
    constexpr int U = kSteps;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15;          // row of the A fragment / column of B
    const int g = lane >> 4;            // which 8-element k slice of the step
    const int nb = blockIdx.x * 16 * RF;

    // this wave's share of the k steps
    const int S = K / 32;
    const int s0 = (int)((long long)S * wave / NWK);
    const int s1 = (int)((long long)S * (wave + 1) / NWK);

    // weight operand of step s for fragment rf: wrow[rf] + wstep * s
    const uint16_t* wrow[RF];
    constexpr int wstep = kTiled ? 512 : 32;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        if constexpr (kTiled) {
            wrow[rf] = W + ((size_t)(nb / 16 + rf) * S) * 512 + lane * 8;
        } else {
            const int n = min(nb + rf * 16 + r16, N - 1);
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

    // fixed-order reduction of the NWK partial tiles through LDS
    __shared__ float red[NWK][RF][MF][4][kWave];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][rf][mf][r][lane] = acc[rf][mf][r];
    __syncthreads();

    constexpr int kOut = 256 * RF * MF;
    for (int e = threadIdx.x; e < kOut; e += NWK * kWave) {
        const int i = e & 15;                 // row within the 16-row fragment
        const int j = (e >> 4) & 15;          // column (position) within the fragment
        const int mf = (e >> 8) % MF;
        const int rf = (e >> 8) / MF;
        const int n = nb + rf * 16 + i;
        const int m = mf * 16 + j;
        if (n >= N || m >= M) continue;
        const int r = i & 3, l = ((i >> 2) << 4) + j;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NWK; ++w) v += red[w][rf][mf][r][l];
        const size_t o = (size_t)m * N + n;
        if constexpr (EPI == kEpiSilu) {
            static_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(silu(v));
        } else if constexpr (EPI == kEpiResidual) {
            static_cast<float*>(out)[o] += v;
        } else {
            static_cast<float*>(out)[o] = v;
        }
    }
}

template <int MF, int EPI>
hipError_t launch_skinny_mf(const MatmulArgs& a, const uint16_t* act, void* out, int Mc,
                            hipStream_t stream) {
    constexpr int RF = 1, NWK = 8;
    const dim3 grid((a.N + 16 * RF - 1) / (16 * RF));
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    ProfScope prof(a.name, stream, matmul_bytes(a, Mc), 2.0 * Mc * (double)a.N * a.K);
    if (a.tiled)
        SV_LAUNCH(prof, (mfma_skinny_kernel<MF, RF, NWK, EPI, true>), grid, NWK * kWave, stream,
                  W, act, Mc, a.N, a.K, out);
    else
        SV_LAUNCH(prof, (mfma_skinny_kernel<MF, RF, NWK, EPI, false>), grid, NWK * kWave, stream,
                  W, act, Mc, a.N, a.K, out);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_skinny_epi(const MatmulArgs& a, hipStream_t stream) {
    const size_t out_es = EPI == kEpiSilu ? 2 : 4;
    for (int mb = 0; mb < a.M; mb += 64) {
        const int Mc = a.M - mb < 64 ? a.M - mb : 64;
        const uint16_t* act = static_cast<const uint16_t*>(a.act) + (size_t)mb * a.K;
        void* out = static_cast<char*>(a.out) + (size_t)mb * a.N * out_es;
        hipError_t e;
        switch ((Mc + 15) / 16) {
            case 1: e = launch_skinny_mf<1, EPI>(a, act, out, Mc, stream); break;
            case 2: e = launch_skinny_mf<2, EPI>(a, act, out, Mc, stream); break;
            case 3: e = launch_skinny_mf<3, EPI>(a, act, out, Mc, stream); break;
            default: e = launch_skinny_mf<4, EPI>(a, act, out, Mc, stream); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

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
