// Weight-streaming matmul for a handful of rows on the vector ALUs.
//
// out[m, n] = sum_k act[m, k] * W[n, k] for M <= 8 rows per launch.  This is
// the verification forward at small B*(K+1): every weight is read from HBM
// once and used for all M positions (publishertech section 1 "The Speculative
// Cycle": the target's weights are streamed exactly once for all drafted
// tokens).  Each wavefront owns kRowsPerWave weight rows; its 64 lanes walk
// the reduction dimension in 16-byte vectors (fully coalesced 1 KiB per wave
// per row and step), multiply them with the matching activation vectors (all
// waves of a CU read the same activation bytes, which stay in L1/L2) and keep
// RW x M fp32 partial sums per lane; the lanes are summed at the end.  bf16
// products use the packed dot instruction (two bf16 products per lane and
// instruction, fp32 accumulate).
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRowsPerWave = 4;
constexpr int kMaxRows = 8;

template <bool kBf16>
__device__ __forceinline__ float dot16(const u32x4& w, const u32x4& a, float acc) {
    if constexpr (kBf16) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(a.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(a.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(a.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(a.w), acc, false);
    } else {
        acc = fmaf(__uint_as_float(w.x), __uint_as_float(a.x), acc);
        acc = fmaf(__uint_as_float(w.y), __uint_as_float(a.y), acc);
        acc = fmaf(__uint_as_float(w.z), __uint_as_float(a.z), acc);
        acc = fmaf(__uint_as_float(w.w), __uint_as_float(a.w), acc);
    }
    return acc;
}

template <bool kBf16, int MB, int EPI>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const void* __restrict__ Wp, const void* __restrict__ Ap, int N, int K,
    void* __restrict__ out, int ldo) {
    constexpr int E = kBf16 ? 8 : 4;      // elements per 16-byte vector
    constexpr int ES = kBf16 ? 2 : 4;     // bytes per element
    constexpr int RW = kRowsPerWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int n0 = (blockIdx.x * kWaves + wave) * RW;
    if (n0 >= N) return;                  // no workgroup barrier below
    const int kb = 0, ke = K;
    const char* W = static_cast<const char*>(Wp);
    const char* A = static_cast<const char*>(Ap);

    size_t wrow[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) wrow[r] = (size_t)min(n0 + r, N - 1) * K;

    float acc[RW][MB];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = 0.f;

    // Software pipeline: the next step's weight vectors are requested before
    // the current step is computed; the activation vectors of the current
    // step are requested first so that waiting for them never waits on the
    // longer weight stream behind them.
    u32x4 wc[RW], wn[RW];
    int k = kb + lane * E;
#pragma unroll
    for (int r = 0; r < RW; ++r)
        wc[r] = k < ke ? *reinterpret_cast<const u32x4*>(W + (wrow[r] + k) * ES) : u32x4{0, 0, 0, 0};
    for (; k < ke; k += kWave * E) {
        u32x4 a[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m)
            a[m] = *reinterpret_cast<const u32x4*>(A + ((size_t)m * K + k) * ES);
        const int kn = k + kWave * E;
#pragma unroll
        for (int r = 0; r < RW; ++r)
            wn[r] = kn < ke ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + (wrow[r] + kn) * ES))
                            : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[r][m] = dot16<kBf16>(wc[r], a[m], acc[r][m]);
#pragma unroll
        for (int r = 0; r < RW; ++r) wc[r] = wn[r];
    }

#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[r][m] = wave_sum(acc[r][m]);

    if (lane != 0) return;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int n = n0 + r;
        if (n >= N) break;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const size_t o = (size_t)m * ldo + n;
            if constexpr (EPI == kEpiSilu) {
                const float v = silu(acc[r][m]);
                if constexpr (kBf16) static_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(v);
                else static_cast<float*>(out)[o] = v;
            } else if constexpr (EPI == kEpiResidual) {
                static_cast<float*>(out)[o] += acc[r][m];
            } else {
                static_cast<float*>(out)[o] = acc[r][m];
            }
        }
    }
}

template <bool kBf16, int EPI>
hipError_t launch_gemv_rows(const MatmulArgs& a, int mb, int mc, hipStream_t stream) {
    const int es = kBf16 ? 2 : 4;
    const void* A = static_cast<const char*>(a.act) + (size_t)mb * a.K * es;
    const size_t out_es = (EPI == kEpiSilu) ? es : 4;
    void* out = static_cast<char*>(a.out) + (size_t)mb * a.N * out_es;
    const dim3 grid((a.N + kWaves * kRowsPerWave - 1) / (kWaves * kRowsPerWave));
    ProfScope prof(a.name, stream, matmul_bytes(a, mc), 2.0 * mc * (double)a.N * a.K);
#define SV_GEMV_CASE(MBV)                                                                  \
    case MBV:                                                                              \
        SV_LAUNCH(prof, (gemv_kernel<kBf16, MBV, EPI>), grid, kThreads, stream, a.W, A, a.N, a.K, \
                  out, a.N);                                                               \
        break;
    switch (mc) {
        SV_GEMV_CASE(1) SV_GEMV_CASE(2) SV_GEMV_CASE(3) SV_GEMV_CASE(4)
        SV_GEMV_CASE(5) SV_GEMV_CASE(6) SV_GEMV_CASE(7) SV_GEMV_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef SV_GEMV_CASE
    return hipGetLastError();
}

template <bool kBf16>
hipError_t launch_gemv_dtype(const MatmulArgs& a, hipStream_t stream) {
    for (int mb = 0; mb < a.M; mb += kMaxRows) {
        const int mc = a.M - mb < kMaxRows ? a.M - mb : kMaxRows;
        hipError_t e;
        switch (a.epi) {
            case kEpiSilu: e = launch_gemv_rows<kBf16, kEpiSilu>(a, mb, mc, stream); break;
            case kEpiResidual: e = launch_gemv_rows<kBf16, kEpiResidual>(a, mb, mc, stream); break;
            case kEpiStore: e = launch_gemv_rows<kBf16, kEpiStore>(a, mb, mc, stream); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv(const MatmulArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_gemv_dtype<true>(a, stream) : launch_gemv_dtype<false>(a, stream);
}

}  // namespace sv
