// RMSNorm of the residual stream before every block and before the LM head.
//
// The pre-norm residual block of the synthetic target:
// a = round_act(h / sqrt(mean(h^2) + eps) * g).  One workgroup owns one row;
// every thread holds its VPT float4 vectors of the row in registers, so all of
// the row's loads are in flight at once, and the sum of squares is reduced
// inside the workgroup in a fixed order.  When the previous down projection
// left split-K partial planes, they are folded in first, in split order:
// h = src + (part[0] + part[1] + ...), and h is written back.  After a
// mixture-of-experts block the weighted expert outputs are folded in the
// same way: h = src + (w_0 Y[inv_0] + w_1 Y[inv_1] + ...), slots in rank
// order.
//
// For the LDS-staged GEMM the bf16 activations are written in the matrix-core
// operand layout (16 x 32 blocks of one KiB, as the tiled weights), rows
// padded to a multiple of 16 with zeros.
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

constexpr int kNormGroupMaxRows = 256;

template <bool kBf16, bool kMoe, int VPT, int THREADS>
__global__ __launch_bounds__(THREADS) void rmsnorm_kernel(
    const float* src, float* hout,  // src may equal hout
    const float* __restrict__ part, int splits, size_t split_stride,
    const float* __restrict__ gain, void* __restrict__ act, int M, int d, float eps,
    int act_tiled, const MoeFold fold) {
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
    // second memory round trip after the reduction (rows of more than 16384
    // elements load the gains afterwards, to stay within the registers)
    constexpr bool kHoldGain = VPT <= 4;
    const f32x4* g4 = reinterpret_cast<const f32x4*>(gain);
    f32x4 h[VPT], g[kHoldGain ? VPT : 1];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int c = tid + v * THREADS;
        h[v] = c < n4 ? s4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kHoldGain) g[v] = c < n4 ? g4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (splits > 0) {
        // acc = part[0] + part[1] + ... per element, planes outermost.  With
        // few rows (fewer workgroups than CUs) a row's time is its chain of
        // memory round trips, so the planes are loaded PG at a time (at most 8
        // vectors per thread in flight): 70B share, 40 rows, 5.7 -> 5.1 us.
        // With many rows they are loaded one plane at a time across the grid,
        // which the memory system serves better (768 rows: 14.7 against
        // 15.4 us grouped).  The additions keep the plane order either way.
        // The planes are dead once read, so they take non-temporal loads (768
        // rows: the step 2.292 -> 2.285 ms, the down projections 1 us faster).
        constexpr int PG = VPT >= 8 ? 1 : 8 / VPT;
        const int pg = M <= kNormGroupMaxRows ? PG : 1;
        f32x4 acc[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int s0 = 0; s0 < splits; s0 += pg) {
            f32x4 pv[PG][VPT];
#pragma unroll
            for (int j = 0; j < PG; ++j) {
                const bool in = j < pg && s0 + j < splits;
                const f32x4* p4 = reinterpret_cast<const f32x4*>(part + (size_t)(s0 + j) * split_stride + off);
#pragma unroll
                for (int v = 0; v < VPT; ++v) {
                    const int c = tid + v * THREADS;
                    pv[j][v] = (in && c < n4) ? __builtin_nontemporal_load(p4 + c)
                                              : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int j = 0; j < PG; ++j) {
                if (j < pg && s0 + j < splits) {
#pragma unroll
                    for (int v = 0; v < VPT; ++v) {
                        if (s0 + j == 0) acc[v] = pv[j][v];
                        else acc[v] += pv[j][v];
                    }
                }
            }
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) h[v] += acc[v];
    }
    if constexpr (kMoe) {
        f32x4 y[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) y[v] = f32x4{0.f, 0.f, 0.f, 0.f};
        // slots in groups of JG, so that at most 16 vectors are in flight
        constexpr int JG = VPT >= 16 ? 1 : 16 / VPT;
#pragma unroll 1
        for (int j0 = 0; j0 < fold.k; j0 += JG) {
#pragma unroll
            for (int jj = 0; jj < JG; ++jj) {
                const int j = j0 + jj;
                if (j >= fold.k) break;
                const float wj = fold.wts[row * fold.k + j];
                const f32x4* yr =
                    reinterpret_cast<const f32x4*>(fold.Y + (size_t)fold.inv[row * fold.k + j] * d);
#pragma unroll
                for (int v = 0; v < VPT; ++v) {
                    const int c = tid + v * THREADS;
                    if (c < n4) y[v] += wj * yr[c];
                }
            }
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) h[v] += y[v];
    }
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        ss += h[v].x * h[v].x;
        ss += h[v].y * h[v].y;
        ss += h[v].z * h[v].z;
        ss += h[v].w * h[v].w;
    }
    if (hout != src || splits > 0 || kMoe) {
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
        const f32x4 gv = kHoldGain ? g[kHoldGain ? v : 0] : g4[c];
        const f32x4 y = {h[v].x * inv_rms * gv.x, h[v].y * inv_rms * gv.y,
                         h[v].z * inv_rms * gv.z, h[v].w * inv_rms * gv.w};
        if constexpr (kBf16) {
            uint2 packed;
            packed.x = pack_bf16x2(y.x, y.y);
            packed.y = pack_bf16x2(y.z, y.w);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(act) + act_off(c)) = packed;
        } else {
            reinterpret_cast<f32x4*>(static_cast<float*>(act) + off)[c] = y;
        }
    }
}

template <bool kBf16, bool kMoe>
hipError_t launch_norm_dtype(const float* src, float* hout, const float* part, int splits,
                             size_t stride, const float* gain, void* act, int M, int d, float eps,
                             int act_tiled, const MoeFold& fold, hipStream_t stream,
                             const ProfScope& prof) {
    const int n4 = d / 4;
    const int rows = act_tiled ? (M + 15) / 16 * 16 : M;
#define SV_NORM(VPT, T)                                                                   \
    SV_LAUNCH(prof, (rmsnorm_kernel<kBf16, kMoe, VPT, T>), rows, T, stream, src, hout, part, \
              splits, stride, gain, act, M, d, eps, act_tiled, fold)
    // rows of up to 4096: 512 threads of two float4 each, so four rows' workgroups
    // share a CU and the whole large batch is resident at once (768 rows with
    // four split planes: 17.0 -> 14.5 us; 5 rows: unchanged).  Wider rows keep
    // 1024 threads (8192: 6.1 us against 7.6 with 512 threads of four).
    if (n4 <= 256) SV_NORM(1, 256);
    else if (n4 <= 1024) SV_NORM(2, 512);
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
    const MoeFold none{};
    return bf16 ? launch_norm_dtype<true, false>(src, hout, part, splits, stride, gain, act, M, d,
                                                 eps, act_tiled, none, stream, prof)
                : launch_norm_dtype<false, false>(src, hout, part, splits, stride, gain, act, M, d,
                                                  eps, act_tiled, none, stream, prof);
}

hipError_t launch_rmsnorm_moe(float* h, const MoeFold& fold, const float* gain, void* act, int M,
                              int d, float eps, int act_tiled, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    if (fold.k < 1 || fold.k > kMoeFoldMaxK || (act_tiled && d % 32)) return hipErrorInvalidValue;
    const double bytes = (double)M * d * (4.0 + 4.0 * fold.k + 4.0 + 2.0);
    ProfScope prof("rmsnorm_moe", stream, bytes, 0.0);
    return launch_norm_dtype<true, true>(h, h, nullptr, 0, 0, gain, act, M, d, eps, act_tiled,
                                         fold, stream, prof);
}

}  // namespace sv
