// bf16 MFMA matmuls out[m, n] = sum_k act[m, k] * W[n, k] on gfx950 matrix
// cores, for the verification forward at B*(K+1) = 1..128 rows per pass.
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
// another, so a wave loads MF / RF activation bytes per weight byte.  One
// fragment per wave suits up to 8 rows; from 9 rows four fragments per wave
// share each activation load, and eight where the grid still fills the chip
// (the LM head at 17..64 rows, wide projections at 17..48: skinny_wide).  Up
// to 8 rows the activations are row-major (rows past M cost nothing); from 9
// rows they come in the operand layout, where each activation load is one
// contiguous KiB.
//
// Weights come either row-major or packed in the tiled layout of pack.hip,
// where each 16 x 32 operand block is one contiguous KiB in lane order (one
// wave load = one contiguous KiB; measured about 1.4x the row-major rate).
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Fixed-order sum of a workgroup's NKS k slices through LDS (`red`, NKS x NR
// x MF x 64 x 16 bytes), one weight fragment of every row group at a time,
// and the epilogue.  Each wave stores its accumulators lane-major (one
// 16-byte write per lane and fragment); each task then sums the NKS copies of
// one lane's four outputs (16-byte reads, no bank conflicts) and writes four
// consecutive outputs n0..n0+3 of one row m: the lane's rows of the MFMA
// result tile.  Fragment rf of row group rr holds outputs n = 16 ((blk NR +
// rr) RF + rf) + 0..15.
template <int MF, int RF, int NR, int NKS, int EPI, bool kActT>
__device__ __forceinline__ void reduce_store(const f32x4v (&acc)[RF][MF],
                                             f32x4v (*red)[NR][MF][kWave], int ks, int rg,
                                             int lane, int blk, int M, int N,
                                             void* __restrict__ out, size_t split_stride) {
    constexpr int NWK = NR * NKS;
    float* plane = static_cast<float*>(out) + (size_t)blockIdx.y * split_stride;
    // rows start 16-byte aligned (8 for bf16 outputs)
    const bool vec = (N & 3) == 0 && ((uintptr_t)out & (EPI == kEpiSilu ? 7 : 15)) == 0;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        if (rf) __syncthreads();        // the previous fragment's readers are done
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) red[ks][rg][mf][lane] = acc[rf][mf];
        __syncthreads();
        constexpr int kTasks = NR * MF * kWave;
        for (int e = threadIdx.x; e < kTasks; e += NWK * kWave) {
            const int l = e % kWave;
            const int mf = (e / kWave) % MF;
            const int rr = e / (kWave * MF);
            const int n0 = ((blk * NR + rr) * RF + rf) * 16 + 4 * (l >> 4);
            const int m = mf * 16 + (l & 15);
            if (n0 >= N || m >= M) continue;
            f32x4v v = red[0][rr][mf][l];
#pragma unroll
            for (int w = 1; w < NKS; ++w) v += red[w][rr][mf][l];
            const size_t o = (size_t)m * N + n0;
            if constexpr (EPI == kEpiSilu) {
                // the next projection's activations, row-major or in the
                // operand layout (N % 32 == 0: n0..n0+3 are 8 contiguous bytes
                // of one block)
                uint16_t* dst = static_cast<uint16_t*>(out) +
                                (kActT ? ((size_t)(m >> 4) * (N >> 5) + (n0 >> 5)) * 512 +
                                             ((m & 15) + 16 * ((n0 & 31) >> 3)) * 8 + (n0 & 7)
                                       : o);
                if (kActT || (vec && n0 + 3 < N)) {
                    uint2 pk;
                    pk.x = pack_bf16x2(silu(v[0]), silu(v[1]));
                    pk.y = pack_bf16x2(silu(v[2]), silu(v[3]));
                    *reinterpret_cast<uint2*>(dst) = pk;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n0 + r < N) dst[r] = (uint16_t)f32_to_bf16(silu(v[r]));
                }
                continue;
            }
            float* dst = EPI == kEpiResidual && split_stride ? plane + o : static_cast<float*>(out) + o;
            if (vec && n0 + 3 < N) {
                if constexpr (EPI == kEpiResidual)
                    if (!split_stride) v += *reinterpret_cast<const f32x4v*>(dst);   // one owner per element
                *reinterpret_cast<f32x4v*>(dst) = v;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (n0 + r >= N) break;
                    if constexpr (EPI == kEpiResidual)
                        if (!split_stride) { dst[r] += v[r]; continue; }
                    dst[r] = v[r];
                }
            }
        }
    }
}

template <int MF, int RF, int NR, int NKS, int U, int EPI, bool kTiled, bool kActT>
__global__ __launch_bounds__(NR * NKS * kWave) void mfma_skinny_kernel(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ act, int M, int N, int K,
    int steps_per_split, void* __restrict__ out, size_t split_stride) {
    static_assert(NKS >= 2, "the k slices are reduced through LDS");
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
    const int fb0 = __builtin_amdgcn_readfirstlane((blockIdx.x * NR + rg) * RF);

    // weight operand of step s for fragment rf.  Tiled: the wave's fragments
    // are contiguous (S KiB each) from the wave-uniform base wbase, so a load
    // needs only a 32-bit lane offset; fragments past N read as zeros.
    // Row-major (one fragment): wrow + 32 * s, this lane's row.
    const char* wbase = reinterpret_cast<const char*>(W + (size_t)fb0 * S * 512);
    bool wval[RF];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) wval[rf] = fb0 + rf < nblk;
    const uint16_t* wrow = W + (size_t)min(fb0 * 16 + r16, N - 1) * K + 8 * g;
    // activation operand of step s for fragment mf.  Row-major: arow[mf] +
    // 32 * s, this lane's row; rows past M read as zeros.  Operand layout: the
    // KiB of row block mf at step s lies (mf * S + s) KiB into the pass (the
    // pass base and a 32-bit lane offset); its rows past M are padding whose
    // outputs are dropped.
    const uint16_t* arow[kActT ? 1 : MF];
    bool aval[MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
        if constexpr (kActT) {
            aval[mf] = mf * 16 < M;
        } else {
            const int m = mf * 16 + r16;
            aval[mf] = m < M;
            arow[mf] = act + (size_t)min(m, M - 1) * K + 8 * g;
        }
    }
    const char* abase = reinterpret_cast<const char*>(act);
    // Operand layout: each wave walks its slice in a rotated order, starting
    // (blockIdx.x / 8) steps in.  Workgroup i runs on XCD i % 8, so the
    // workgroups of one XCD then read different activation blocks at any
    // moment instead of all fetching the same KiB from one L2 channel
    // (8B-shaped up projection at 64 rows: 29.4 -> 24.6 us for the loop).
    const int slen = max(s1 - s0, 1);
    const int rot = kActT ? (int)((blockIdx.x >> 3) % (unsigned)slen) : 0;

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
            int ps = ss;                 // the k step both operands load
            if constexpr (kActT) {
                const int t = ss - s0 + rot;
                ps = s0 + (t >= slen ? t - slen : t);
            }
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
                x[u][mf] = (in && aval[mf])
                               ? *reinterpret_cast<const bf16x8*>(
                                     kActT ? abase + (uint32_t)(lane * 16 + (mf * S + ps) * 1024)
                                           : reinterpret_cast<const char*>(arow[mf] + 32 * ps))
                               : zero8;
#pragma unroll
            for (int rf = 0; rf < RF; ++rf)
                w[u][rf] = (in && wval[rf])
                               ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(
                                     kTiled ? wbase + (uint32_t)(lane * 16 + (rf * S + ps) * 1024)
                                            : reinterpret_cast<const char*>(wrow + 32 * ps)))
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

    __shared__ f32x4v red[NKS][NR][MF][kWave];
    reduce_store<MF, RF, NR, NKS, EPI, kActT>(acc, red, ks, rg, lane, blockIdx.x, M, N, out,
                                              split_stride);
}

template <int MF, int RF, int NR, int NKS, int U, int EPI, bool kActT = false>
hipError_t launch_shape(const MatmulArgs& a, const uint16_t* act, void* out, int Mc, int ksg,
                        size_t stride, hipStream_t stream) {
    const int rows = 16 * RF * NR;
    const dim3 grid((a.N + rows - 1) / rows, ksg);
    const int S = a.K / 32;
    const int sps = (S + ksg - 1) / ksg;
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    ProfScope prof(a.name, stream, matmul_bytes(a, Mc), 2.0 * Mc * (double)a.N * a.K);
    if (a.tiled) {
        SV_LAUNCH(prof, (mfma_skinny_kernel<MF, RF, NR, NKS, U, EPI, true, kActT>), grid,
                  NR * NKS * kWave, stream, W, act, Mc, a.N, a.K, sps, out, stride);
    } else if constexpr (RF == 1 && !kActT) {
        SV_LAUNCH(prof, (mfma_skinny_kernel<MF, RF, NR, NKS, U, EPI, false, false>), grid,
                  NR * NKS * kWave, stream, W, act, Mc, a.N, a.K, sps, out, stride);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// 17..48 rows of a wide projection (operand-layout activations): eight
// weight fragments per wave halve the activation loads per weight byte, when
// the grid still fills the chip.  Up projection (no K split): N >= 24576
// rows, 192+ workgroups.  Down projection: a K split that gives 256
// workgroups of 128 rows must still leave every wave 16+ steps.  Measured on
// the 70B-layer share at 40 rows: up 88 -> 79 us, down 83 -> 79 us; with
// 112 workgroups (8B-shaped up) or 7 steps per wave (8B-shaped down) eight
// fragments were 40% and 7% slower.
constexpr int kWideMinRows = 17, kWideMaxRows = 48;

// K split of a wide down projection (0: not wide)
int wide_down_splits(int N, int K) {
    const long long wg = (N + 127) / 128;
    int ksg = 1;
    while (wg * ksg < 256 && ksg < 8) ksg *= 2;
    return wg * ksg >= 256 && (K / 32) / (ksg * 8) >= 16 ? ksg : 0;
}

bool skinny_wide(int M, int N, int K, int epi) {
    if (M < kWideMinRows || M > kWideMaxRows) return false;
    if (epi == kEpiSilu) return N >= 24576;
    if (epi == kEpiResidual) return wide_down_splits(N, K) > 0;
    return false;
}

template <int MF, int EPI>
hipError_t launch_mf(const MatmulArgs& a, const uint16_t* act, void* out, int Mc, int ksg,
                     size_t stride, hipStream_t stream) {
    if (a.act_tiled) {
        // activations in the operand layout (9..128 rows per pass): each
        // activation load is one contiguous KiB.  Four fragments per wave and
        // eight k slices (two-step buffers up to 64 rows, one above); eight
        // fragments per wave for the LM head at 17..64 rows and for wide
        // projections at 17..48 (skinny_wide).
        if (!a.tiled) return hipErrorInvalidValue;
        if constexpr (EPI != kEpiStore && MF >= 2 && MF <= 3) {
            if (skinny_wide(a.M, a.N, a.K, EPI))
                return launch_shape<MF, 8, 1, 8, 1, EPI, true>(a, act, out, Mc, ksg, stride, stream);
        }
        if constexpr (EPI == kEpiStore && MF >= 2 && MF <= 4)
            return launch_shape<MF, 8, 1, 8, 1, EPI, true>(a, act, out, Mc, ksg, stride, stream);
        return launch_shape<MF, 4, 1, 8, (MF <= 4 ? 2 : 1), EPI, true>(a, act, out, Mc, ksg, stride,
                                                                        stream);
    }
    if constexpr (MF > 4) {
        return hipErrorInvalidValue;     // row-major activations: passes of at most 64 rows
    } else {
        // row-major activations: up to 8 rows on tiled weights, any pass on
        // row-major weights (one fragment per wave, 8 k slices, four-step
        // buffers).  The up projection's short reduction (d) runs 16 slices of
        // two-step buffers: 3% faster on the 8B shape, where the down
        // projection (K = ffn) and the head are not.
        if (a.tiled && Mc > 8) return hipErrorInvalidValue;
        if (EPI == kEpiSilu && MF == 1 && a.tiled)
            return launch_shape<1, 1, 1, 16, 2, EPI>(a, act, out, Mc, ksg, stride, stream);
        return launch_shape<MF, 1, 1, 8, 4, EPI>(a, act, out, Mc, ksg, stride, stream);
    }
}

template <int EPI>
hipError_t launch_skinny_epi(const MatmulArgs& a, hipStream_t stream) {
    const size_t out_es = EPI == kEpiSilu ? 2 : 4;
    // down projection with a K split: `splits` partial planes of [M, N]
    const bool planes = EPI == kEpiResidual && a.splits > 0;
    const int ksg = planes ? a.splits : 1;
    const size_t stride = planes ? (size_t)a.M * a.N : 0;
    // passes of 64 rows (row-major activations) or 128 (operand layout); a
    // pass starts on a 16-row block, so both layouts offset it by mb * K
    // elements (activations) and mb * N (outputs)
    const int pass = a.act_tiled ? 128 : 64;
    for (int mb = 0; mb < a.M; mb += pass) {
        const int Mc = a.M - mb < pass ? a.M - mb : pass;
        const uint16_t* act = static_cast<const uint16_t*>(a.act) + (size_t)mb * a.K;
        void* out = static_cast<char*>(a.out) + (size_t)mb * a.N * out_es;
        hipError_t e;
        switch ((Mc + 15) / 16) {
            case 1: e = launch_mf<1, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 2: e = launch_mf<2, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 3: e = launch_mf<3, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 4: e = launch_mf<4, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 5: e = launch_mf<5, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 6: e = launch_mf<6, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            case 7: e = launch_mf<7, EPI>(a, act, out, Mc, ksg, stride, stream); break;
            default: e = launch_mf<8, EPI>(a, act, out, Mc, ksg, stride, stream); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int skinny_splits(int M, int N, int K, int tiled, int act_tiled) {
    // 17+ rows run four or eight fragments per wave, so a d-row down
    // projection has few workgroups: split K until the grid fills 256 CUs
    // (>= 16 steps of 32 per split half, so every k slice keeps a few steps)
    if (!tiled || (M <= 16 && !act_tiled)) return 0;
    if (act_tiled && skinny_wide(M, N, K, kEpiResidual)) {
        const int ksg = wide_down_splits(N, K);
        return ksg > 1 ? ksg : 0;
    }
    const long long wg = (N + (act_tiled ? 63 : 127)) / (act_tiled ? 64 : 128);
    int ksg = 1;
    while (wg * ksg < 256 && ksg < 8 && (K / 32) / (ksg * 2) >= 16) ksg *= 2;
    return ksg > 1 ? ksg : 0;
}

hipError_t launch_mfma_skinny(const MatmulArgs& a, hipStream_t stream) {
    if (!a.bf16 || a.K % 32) return hipErrorInvalidValue;
    if (a.act_tiled && (!a.tiled || (a.epi == kEpiSilu && a.N % 32))) return hipErrorInvalidValue;
    switch (a.epi) {
        case kEpiSilu: return launch_skinny_epi<kEpiSilu>(a, stream);
        case kEpiResidual: return launch_skinny_epi<kEpiResidual>(a, stream);
        case kEpiStore: return launch_skinny_epi<kEpiStore>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sv
