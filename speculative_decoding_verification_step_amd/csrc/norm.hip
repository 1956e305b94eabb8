// RMSNorm of the residual stream before every block and before the LM head.
//
// The pre-norm residual block of the synthetic target:
// a = round_act(h / sqrt(mean(h^2) + eps) * g).  One workgroup owns one row;
// every thread holds its VPT float4 vectors of the row in registers, so all of
// the row's loads are in flight at once, and the sum of squares is reduced
// inside the workgroup in a fixed order.  When the previous down projection
// left split-K partial planes, they are folded in first, in split order:
// h = src + (part[0] + part[1] + ...), and h is written back.
//
// For the LDS-staged GEMM the bf16 activations are written in the matrix-core
// operand layout (16 x 32 blocks of one KiB, as the tiled weights), rows
// padded to a multiple of 16 with zeros.
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

template <bool kBf16, int VPT, int THREADS>
__global__ __launch_bounds__(THREADS) void rmsnorm_kernel(
    const float* src, float* hout,  // src may equal hout
    const float* __restrict__ part, int splits, size_t split_stride,
    const float* __restrict__ gain, void* __restrict__ act, int M, int d, float eps,
    int act_tiled) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t off = (size_t)row * d;
    const int n4 = d >> 2;
    // element offset of act[row][4c .. 4c+3] (four consecutive, 8-byte aligned)
    auto act_off = [&](int c) -> size_t {
        if (!act_tiled) return off + 4 * (size_t)c;
        const int k = 4 * c;
        return ((size_t)(row >> 4) * (d >> 5) + (k >> 5)) * 512 +
               ((row & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
    };
    if (row >= M) {                 // padding rows of the operand layout
        if constexpr (kBf16) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int c = tid + v * THREADS;
                if (c < n4)
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(act) + act_off(c)) = uint2{0u, 0u};
            }
        }
        return;
    }
    const f32x4* s4 = reinterpret_cast<const f32x4*>(src + off);

    // the row and the gains are loaded together, so the gains do not add a
    // second memory round trip after the reduction
    const f32x4* g4 = reinterpret_cast<const f32x4*>(gain);
    f32x4 h[VPT], g[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = tid + v * THREADS;
        h[v] = c < n4 ? s4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
        g[v] = c < n4 ? g4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (splits > 0) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = tid + v * THREADS;
            if (c >= n4) continue;
            f32x4 acc = reinterpret_cast<const f32x4*>(part + off)[c];
            for (int s = 1; s < splits; ++s)
                acc += reinterpret_cast<const f32x4*>(part + s * split_stride + off)[c];
            h[v] += acc;
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        ss += h[v].x * h[v].x;
        ss += h[v].y * h[v].y;
        ss += h[v].z * h[v].z;
        ss += h[v].w * h[v].w;
    }
    if (hout != src || splits > 0) {
        f32x4* h4 = reinterpret_cast<f32x4*>(hout + off);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int c = tid + v * THREADS;
            if (c < n4) h4[c] = h[v];
        }
    }

    __shared__ float red[THREADS / kWave];
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < THREADS / kWave; ++w) tot += red[w];
    const float inv_rms = 1.0f / sqrtf(tot / (float)d + eps);

#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = tid + v * THREADS;
        if (c >= n4) continue;
        const f32x4 y = {h[v].x * inv_rms * g[v].x, h[v].y * inv_rms * g[v].y,
                         h[v].z * inv_rms * g[v].z, h[v].w * inv_rms * g[v].w};
        if constexpr (kBf16) {
            uint2 packed;
            packed.x = f32_to_bf16(y.x) | (f32_to_bf16(y.y) << 16);
            packed.y = f32_to_bf16(y.z) | (f32_to_bf16(y.w) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(act) + act_off(c)) = packed;
        } else {
            reinterpret_cast<f32x4*>(static_cast<float*>(act) + off)[c] = y;
        }
    }
}

template <bool kBf16>
hipError_t launch_norm_dtype(const float* src, float* hout, const float* part, int splits,
                             size_t stride, const float* gain, void* act, int M, int d, float eps,
                             int act_tiled, hipStream_t stream, const ProfScope& prof) {
    const int n4 = d / 4;
    const int rows = act_tiled ? (M + 15) / 16 * 16 : M;
#define SV_NORM(VPT, T)                                                                       \
    SV_LAUNCH(prof, (rmsnorm_kernel<kBf16, VPT, T>), rows, T, stream, src, hout, part, splits, \
              stride, gain, act, M, d, eps, act_tiled)
    if (n4 <= 256) SV_NORM(1, 256);
    else if (n4 <= 1024) SV_NORM(1, 1024);
    else if (n4 <= 2048) SV_NORM(2, 1024);
    else if (n4 <= 4096) SV_NORM(4, 1024);
    else if (n4 <= 8192) SV_NORM(8, 1024);
    else return hipErrorInvalidValue;
#undef SV_NORM
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const float* src, float* hout, const float* part, int splits,
                          const float* gain, void* act, int M, int d, float eps, int bf16,
                          int act_tiled, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    if (act_tiled && (!bf16 || d % 32)) return hipErrorInvalidValue;
    const bool writes_h = hout != src || splits > 0;
    const double bytes =
        (double)M * d * (4.0 + 4.0 * splits + (writes_h ? 4.0 : 0.0) + (bf16 ? 2.0 : 4.0));
    ProfScope prof("rmsnorm", stream, bytes, 0.0);
    const size_t stride = (size_t)M * d;
    return bf16 ? launch_norm_dtype<true>(src, hout, part, splits, stride, gain, act, M, d, eps,
                                          act_tiled, stream, prof)
                : launch_norm_dtype<false>(src, hout, part, splits, stride, gain, act, M, d, eps,
                                           act_tiled, stream, prof);
}

}  // namespace sv
