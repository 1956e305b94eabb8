// Internal launchers of the verification-step kernels.  Host code only sees
// these declarations; every launcher enqueues on `stream` and returns the
// launch status (hipGetLastError after the launch).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Epilogue of a weight-streaming matmul  out[m, n] = sum_k act[m, k] * W[n, k].
enum Epi : int {
    kEpiSilu = 0,      // act_out[m, n] = round_act(silu(acc))         (up projection)
    kEpiResidual = 1,  // h[m, n] += acc  (fp32; one owner per element)  (down projection)
    kEpiStore = 2,     // f32_out[m, n] = acc                          (LM head)
};

struct MatmulArgs {
    const void* W;        // [N, K] weights (bf16 bits or fp32)
    const void* act;      // [M, K] activations, same dtype as W
    int M, N, K;
    int epi;
    void* out;            // act_out (kEpiSilu), h (kEpiResidual) or f32_out (kEpiStore)
    int bf16;             // 1: bf16 weights/activations, 0: fp32
    int tiled;            // 1: W in the MFMA-tiled layout of pack.hip (bf16 only)
    int act_tiled;        // 1: `act` (and the kEpiSilu output) in the operand layout of
                          // the tiled weights, rows padded to 16 (MFMA kernels,
                          // tiled weights only)
    int splits;           // kEpiResidual on the MFMA kernels: K split count (0 = add
                          // into h); `out` then holds `splits` fp32 partial
                          // planes [M, N] that the next RMSNorm folds in
    const char* name;     // timing label (null: launch_matmul names it by kernel and epilogue)
};

// bf16 weights: elements of the MFMA-tiled copy of a [rows, cols] matrix
// (rows padded to a multiple of 16), and the packing launch for `count`
// consecutive row-major matrices.
size_t tiled_elems(int rows, int cols);
hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int rows, int cols, int count,
                       hipStream_t stream);

// Kernel families a matmul can run on.
enum MatmulKind : int {
    kGemvValu = 0,        // VALU dot products, M <= 8 per launch (m-chunks above)
    kMfmaSkinny = 1,      // bf16 MFMA, weights streamed straight to registers
    kMfmaTiled = 2,       // bf16 MFMA, LDS-staged blocks for large M
};

hipError_t launch_matmul(const MatmulArgs& a, int kind, hipStream_t stream);
// Algorithmic bytes of one launch of `a` over `rows` of its activations.
double matmul_bytes(const MatmulArgs& a, int rows);

// RMSNorm of each row:  act = round_act(h / sqrt(mean(h^2) + eps) * gain)
// with h = src + part[0] + ... + part[splits-1] (split-K planes of [M, d],
// none when splits == 0); h is written to hout when hout != src or partials
// were folded (the first block copies the caller's hidden states into the
// residual stream).  act_tiled (bf16): act in the operand layout of the tiled
// weights, rows padded to a multiple of 16 with zeros.
hipError_t launch_rmsnorm(const float* src, float* hout, const float* part, int splits,
                          const float* gain, void* act, int M, int d, float eps, int bf16,
                          int act_tiled, hipStream_t stream);

// Weighted expert outputs of a mixture-of-experts block, folded into the
// residual stream by the next RMSNorm: h[t] += sum_j wts[t k + j] *
// Y[inv[t k + j]], j = 0 .. k - 1 in rank order (Y [M k, d] fp32).
constexpr int kMoeFoldMaxK = 8;
struct MoeFold {
    const float* Y = nullptr;
    const float* wts = nullptr;
    const int32_t* inv = nullptr;
    int k = 0;
};
hipError_t launch_rmsnorm_moe(float* h, const MoeFold& fold, const float* gain, void* act, int M,
                              int d, float eps, int act_tiled, hipStream_t stream);

// Kernel family and activation layout by row count (bf16, tiled weights),
// measured on the 8B-shaped stack:
//  - the projections stream their weights up to kTiledMinRows - 1 rows per
//    pass and reuse them from LDS from kTiledMinRows on (LDS-staged GEMM);
//    the LM head moves to the GEMM from kHeadTiledMinRows (forward at 96 /
//    128 rows: 0.624 / 0.662 ms against 0.635 / 0.680 with a streamed head;
//    even at 80);
//  - from kActTiledMinRows rows the activations are in the operand layout
//    (one contiguous KiB per 16 rows x 32 k) for both families; below it they
//    are row-major, where rows past M cost nothing (forward at 9 / 16 rows:
//    0.429 / 0.434 vs 0.454 / 0.491 ms row-major; at 5 rows 0.421 vs 0.398).
constexpr int kTiledMinRows = 129;
constexpr int kHeadTiledMinRows = 65;
constexpr int kActTiledMinRows = 9;

// Split count of the LDS-staged GEMM's K range for an [M, N, K] product
// (so that the tile grid fills the chip).
int tiled_splits(int M, int N, int K);
// Split count of the streaming MFMA kernel's down projection (0: no split).
int skinny_splits(int M, int N, int K, int tiled, int act_tiled);

// Softmax statistics at temperature T (1/T = inv_t), per chunk of
// stats_chunks(V) chunks of each row: chunk max and sum of exp((z - max) / T)
// into pv/ps [rows, nchunk]; at T = 0 the chunk max and argmax (lowest id on
// ties) into pv/pi.  Rows 0..n_t-1 come from `target`, n_t.. from `draft`.
int stats_chunks(int V);
hipError_t launch_row_stats(const float* target, const float* draft, int n_t, int n_d, int V,
                            float inv_t, int greedy, float* pv, float* ps, int* pi,
                            hipStream_t stream, float* copy = nullptr, size_t copy_stride = 0);

// Accept / resample / bonus for B requests, folding the chunk statistics
// written by launch_row_stats.  `scratch` holds accept_meta_floats(B, V)
// floats (per-chunk draw sums and per-request draw parameters).
size_t accept_meta_floats(int B, int V);
hipError_t launch_accept(const float* target, const float* draft, const int32_t* tokens, int B,
                         int K, int V, float inv_t, int greedy, uint64_t seed, uint32_t step,
                         const float* pv, const float* ps, const int* pi, float* scratch,
                         int32_t* out_tokens, int32_t* accept_len, float* p_at, float* q_at,
                         hipStream_t stream);

// One token per row of logits [B, V]: the bonus-token draw of a verification
// with no draft positions (inverse CDF of softmax(z / T) in ascending ids;
// argmax, lowest id on ties, at T = 0), its uniform from Philox counter
// (b, slot, 2, step).  Token b goes to tokens[b * out_stride].  pv/ps/pi are
// launch_row_stats' statistics of the B rows; scratch holds
// accept_meta_floats(B, V) floats.
hipError_t launch_sample(const float* logits, int B, int V, float inv_t, int greedy,
                         uint64_t seed, uint32_t step, int slot, const float* pv, const float* ps,
                         const int* pi, float* scratch, int32_t* tokens, int out_stride,
                         hipStream_t stream);

// Per-launch timing hook (implemented by the host layer).  When profiling is
// on, a scope hands out a pair of events that the launch records at the
// dispatch's own start and end (hipExtLaunchKernelGGL), so the measured time
// is the kernel's execution, not the gaps around it; otherwise both are null
// and the launch is an ordinary one.  One scope per kernel launch.
struct ProfScope {
    ProfScope(const char* name, hipStream_t s, double bytes, double flops);
    hipEvent_t ev0 = nullptr;
    hipEvent_t ev1 = nullptr;
};

// Launch `kernel` (parenthesise template-ids) under a timing scope.
#define SV_LAUNCH(prof, kernel, grid, block, stream, ...)                                  \
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, (stream), (prof).ev0, (prof).ev1, \
                          0, __VA_ARGS__)

}  // namespace sv
