// LDS-staged bf16 GEMM on gfx950's 32x32x16 matrix-core instruction, for the
// verification forward at large B*(K+1) (NVIDIA co-design post, "Draft length
// and performance of linear layers": GEMM-M grows to M(1+D) and crosses from
// memory- to compute-bound, so the weights must be reused from on-chip
// memory across many activation rows).
//
// out^T tile [BN weight rows x BM activation rows] per workgroup of WN x WM
// waves; wave (wn, wm) owns FN x FM 32 x 32 output blocks.  Weights and
// activations are stored in the 16 x 32 operand-block layout (pack.hip; the
// RMSNorm and the SiLU epilogue write activations that way).  Each k step of
// 32, the waves copy the tile's operands from global memory straight into an
// LDS stage with buffer_load_dwordx4 ... lds, choosing each lane's 16-byte
// piece so that every 32-row x 16-k operand of v_mfma_f32_32x32x16_bf16
// lands as one contiguous KiB in lane order: lane l holds row l % 32, k group
// 2 t + l / 32 of the step's 32-wide block (t = 0, 1 the two halves), which
// lives in 16-row block l / 16 % 2 of the pair at position (l % 16) +
// 16 (2 t + l / 32).  Operand reads from LDS are then one contiguous KiB per
// wave (no bank conflicts), and the copy of one operand reads four 256-byte
// runs of global memory.  A copy is addressed by a scalar buffer resource, a
// fixed 32-bit lane offset and a scalar step offset: with one wave per SIMD
// every cycle spent issuing a copy is a cycle the matrix pipe waits, and this
// form issues with no vector address arithmetic (the head at 768 rows:
// 821 -> 712 us against 64-bit per-lane addresses).
//
// Pipelining: NS stages in a ring, NS steps of copies in flight.  Within a
// step a wave reads the second half's operands while the first half's MFMAs
// run, then waits for the next step's copies (vmcnt), passes one bare
// workgroup barrier (after which every wave has read the step it leaves, so
// its slot is refilled at once), and issues that refill and the next step's
// first-half reads while the second half's MFMAs run.  One barrier per 32 k.
// With one wave per SIMD, any stall on issuing a copy or an LDS read idles
// the matrix pipe, so every copy and read is placed between two MFMAs.
//
// The K range can be split; split results go to fp32 partial planes that
// the following RMSNorm folds in (in split order, so results are
// deterministic).  Tile order: workgroup i runs on XCD i % 8, so tiles are
// renumbered to give every XCD a contiguous run, activation tile fastest:
// the tiles that share one weight panel run together on one XCD and reuse it
// from that XCD's L2.  The K split is the slowest index, so an XCD's run
// stays within one split and reads only that split's share of the
// activations (768-row down projection, 4 splits: 79.4 -> 78.3 us).
#include "common.hpp"
#include "kernels.hpp"

namespace sv {

namespace {

typedef float f32x16v __attribute__((ext_vector_type(16)));

// Third word of a raw buffer resource on gfx9-class parts: 32-bit data
// format, no swizzle; loads past num_records bytes read zero.
constexpr int kBufferFlags = 0x00020000;

// One 16-byte piece per lane from a buffer over [base, base + bytes) into
// LDS (lane-contiguous at the wave-uniform `dst`): byte offset voff (per
// lane) + soff (wave-uniform).
__device__ __forceinline__ void copy_to_lds(const void* base, int bytes, lds_void* dst, uint32_t voff,
                                            int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags), dst, 16,
        voff, soff, 0, 0);
}

// compiler-level barrier: no memory access moves across it
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Scheduling pattern for one region of MF MFMAs, VM VMEM instructions and DS
// DS reads: MFMA slot i is followed by its even share of each kind.
template <int I, int MF, int VM, int DS>
__device__ __forceinline__ void interleave() {
    if constexpr (I < MF) {
        constexpr int nv = (I + 1) * VM / MF - I * VM / MF;
        constexpr int nd = (I + 1) * DS / MF - I * DS / MF;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
        if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x010, nv, 0);   // VMEM
        if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);   // DS read
        interleave<I + 1, MF, VM, DS>();
    }
}

template <int WN, int WM, int FN, int FM, int NS, int WPE, int EPI>
__global__ __launch_bounds__(WN * WM * kWave, WPE)
void mfma_gemm_kernel(const uint16_t* __restrict__ Wt, const uint16_t* __restrict__ act, int M,
                        int N, int K, int splits, int steps_per_split, void* __restrict__ out,
                        size_t split_stride) {
    constexpr int NW = WN * WM;
    constexpr int BN32 = WN * FN;                // 32-row weight blocks per tile
    constexpr int BM32 = WM * FM;                // 32-row activation blocks per tile
    constexpr int NB = BN32 + BM32;
    constexpr int CP = 2 * NB;                   // 1 KiB operand copies per stage
    // every wave issues PER_WAVE copies (so the vmcnt arithmetic is the same
    // for all); when CP does not divide, the last ones repeat copy CP - 1
    // (the same bytes to the same place)
    constexpr int PER_WAVE = (CP + NW - 1) / NW;
    static_assert(PER_WAVE * (NS - 1) < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS][CP * 512];

    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform, so everything derived from it (LDS slots, copy bases) stays
    // in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wn = wave / WM, wm = wave % WM;

    // XCD-contiguous renumbering (XCD x = i % 8 gets G/8 tiles, the first
    // G%8 XCDs one more), then activation tile fastest, weight tile next, K
    // split slowest
    const int G = gridDim.x, L = blockIdx.x;
    const int q = G / 8, r = G % 8, x = L % 8, j8 = L / 8;
    const int t = x < r ? x * (q + 1) + j8 : r * (q + 1) + (x - r) * q + j8;
    const int MT = (M + BM32 * 32 - 1) / (BM32 * 32);
    const int NT = (N + BN32 * 32 - 1) / (BN32 * 32);
    const int tm = t % MT;
    const int tn = (t / MT) % NT;
    const int split = t / (MT * NT);
    const int S = K / 32;
    const int s_begin = split * steps_per_split;
    const int nsteps = min(S, s_begin + steps_per_split) - s_begin;   // >= 1 (launcher)
    const int nblk = (N + 15) / 16;              // 16-row weight blocks present
    const int mblk = (M + 15) / 16;              // 16-row activation blocks (rows padded to 16)

    // Copies go through buffer resources over the two matrices: a 32-bit lane
    // offset (the lane's 16-row block of the pair, clamped into the matrix,
    // and its piece) plus a scalar offset per step, so issuing a copy costs
    // one scalar add for its LDS slot and no vector work.
    const int hi = (lane >> 4) & 1;
    const uint32_t piece = ((lane & 15) + 16 * (lane >> 5)) * 16;
    const int bytes_w = (int)((uint32_t)nblk * (uint32_t)S * 1024u);
    const int bytes_a = (int)((uint32_t)mblk * (uint32_t)S * 1024u);
    uint32_t coff[PER_WAVE];
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int c = min(wave + NW * i, CP - 1);
        const int half = c / NB, blk = c % NB;
        const int rb = blk < BN32 ? min(2 * (tn * BN32 + blk) + hi, nblk - 1)
                                  : min(2 * (tm * BM32 + blk - BN32) + hi, mblk - 1);
        coff[i] = ((uint32_t)rb * (uint32_t)S + (uint32_t)s_begin) * 1024u + piece + 512u * half;
    }
    auto issue = [&](int j) {
        const int st = j % NS;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int c = min(wave + NW * i, CP - 1);
            const bool w = (c % NB) < BN32;
            copy_to_lds(w ? (const void*)Wt : (const void*)act, w ? bytes_w : bytes_a,
                        (lds_void*)(&lds[st][c * 512]), coff[i], j * 1024);
        }
    };

    f32x16v acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int jj = 0; jj < FM; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;

    bf16x8 a0[FN], b0[FM], a1[FN], b1[FM];
    auto load = [&](bf16x8 (&a)[FN], bf16x8 (&b)[FM], const uint16_t* stage, int half) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
            a[i] = *reinterpret_cast<const bf16x8*>(stage + (half * NB + wn * FN + i) * 512 + lane * 8);
#pragma unroll
        for (int jj = 0; jj < FM; ++jj)
            b[jj] = *reinterpret_cast<const bf16x8*>(stage + (half * NB + BN32 + wm * FM + jj) * 512 +
                                                     lane * 8);
    };
    auto mma = [&](const bf16x8 (&a)[FN], const bf16x8 (&b)[FM]) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int jj = 0; jj < FM; ++jj)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[jj], acc[i][jj], 0, 0, 0);
    };

    // MFMAs interleaved with the step's other memory instructions (spread
    // evenly), so the single wave per SIMD keeps its matrix pipe fed while
    // copies and LDS reads wait to issue
    auto interleave_copies = [&]() { interleave<0, FN * FM, PER_WAVE, FN + FM>(); };
    auto interleave_reads = [&]() { interleave<0, FN * FM, 0, FN + FM>(); };

    // prologue: steps 0 .. NS-1 in flight (slot = step % NS)
#pragma unroll
    for (int p = 0; p < NS; ++p)
        if (p < nsteps) issue(p);
    if (nsteps >= NS) wait_vmcnt<PER_WAVE * (NS - 1)>();
    else wait_vmcnt<0>();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    load(a0, b0, lds[0], 0);

    // Step j: read its second half while the first half's MFMAs run; wait for
    // step j + 1's copies and this wave's reads of step j; one barrier (every
    // wave has read step j, so its slot takes step j + NS); then step j + NS's
    // copies and step j + 1's first-half reads while the second half's MFMAs
    // run.  Steady state (every iteration refills a slot) ...
    int j = 0;
    for (; j < nsteps - NS; ++j) {
        load(a1, b1, lds[j % NS], 1);
        mma(a0, b0);
        interleave_reads();
        // step j + 1 is done once at most the steps j + 2 .. j + NS - 1 remain
        wait_vmcnt<PER_WAVE * (NS - 2)>();
        __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0); vmcnt and expcnt unconstrained
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        issue(j + NS);
        load(a0, b0, lds[(j + 1) % NS], 0);
        mma(a1, b1);
        interleave_copies();
    }
    // ... and the last steps, with every copy already issued
    for (; j < nsteps - 1; ++j) {
        load(a1, b1, lds[j % NS], 1);
        mma(a0, b0);
        interleave_reads();
        wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        load(a0, b0, lds[(j + 1) % NS], 0);
        mma(a1, b1);
        interleave_reads();
    }
    load(a1, b1, lds[(nsteps - 1) % NS], 1);
    mma(a0, b0);
    mma(a1, b1);

    // epilogue: block (i, jj) of lane l holds columns m = mbase + l % 32 and
    // rows n = nbase + 8 (v / 4) + 4 (l / 32) + v % 4, v = 0..15
    const int mpad = mblk * 16;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        const int nb = (tn * BN32 + wn * FN + i) * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) {
            const int m = (tm * BM32 + wm * FM + jj) * 32 + (lane & 31);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nb + 8 * g;
                const f32x4 v = {acc[i][jj][4 * g], acc[i][jj][4 * g + 1], acc[i][jj][4 * g + 2],
                                 acc[i][jj][4 * g + 3]};
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
                    *reinterpret_cast<f32x4*>(dst + o0) = v;
                    continue;
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    if (n + rr < N) dst[o0 + rr] = v[rr];
            }
        }
    }
}

// Tiles (WN x WM waves of FN x FM 32-row blocks; NS stages of k = 32), all
// 256 weight rows wide:
//  T256 - 2 x 2 waves of 128 x 128 (one per SIMD, 256 accumulator registers):
//         256 activation rows, 4 stages of 32 KiB
//  T192 - 4 x 2 waves of 64 x 96 (two per SIMD, 96 accumulators): 192 rows
//         (768 rows in 4 tiles), 28 KiB stages.  More LDS reads per flop than
//         2 x 2 waves of 128 x 96, but the second wave on each SIMD issues
//         while the first waits: faster in 13 of 15 measured cases (up, down
//         and head at 256-768 rows), e.g. up 93.9 -> 89.8 us and head 760.6 ->
//         735.8 us at 768 rows.  (Eight waves of 128 x 64 on T256 lose on the
//         head: 689.8 -> 701.4 us at 768 rows.)
//  T128 - 4 x 2 waves of 64 x 64 (two per SIMD): 128 rows, 24 KiB stages;
//         against 2 x 2 waves of 128 x 64 the up projection runs 4-10% faster
//         at 144-640 rows (e.g. 72.3 -> 67.3 us at 512), down and head within
//         2% either way
//  T64  - 2 x 2 waves of 128 x 32: 64 rows, 20 KiB stages (eight waves of
//         64 x 32 gain nothing)
struct T256 { static constexpr int WN = 2, WM = 2, FN = 4, FM = 4, NS = 4, WPE = 1; static constexpr double EFF = 1.00; };
struct T192 { static constexpr int WN = 4, WM = 2, FN = 2, FM = 3, NS = 4, WPE = 1; static constexpr double EFF = 0.96; };
struct T128 { static constexpr int WN = 4, WM = 2, FN = 2, FM = 2, NS = 4, WPE = 1; static constexpr double EFF = 0.87; };
struct T64 { static constexpr int WN = 2, WM = 2, FN = 4, FM = 1, NS = 5, WPE = 1; static constexpr double EFF = 0.60; };

template <class T> constexpr int tn32() { return T::WN * T::FN * 32; }
template <class T> constexpr int tm32() { return T::WM * T::FM * 32; }
template <class T> long long tiles32(int M, int N) {
    return (long long)((N + tn32<T>() - 1) / tn32<T>()) * ((M + tm32<T>() - 1) / tm32<T>());
}

template <class T, int EPI>
hipError_t launch32(const MatmulArgs& a, int splits, hipStream_t stream) {
    const int S = a.K / 32;
    const int sps = (S + splits - 1) / splits;
    // every split must own at least one step
    if (splits < 1 || (long long)sps * (splits - 1) >= S) return hipErrorInvalidValue;
    const long long G = tiles32<T>(a.M, a.N) * splits;
    if (G > 0x7fffffff) return hipErrorInvalidValue;
    // the copies address each matrix with 32-bit byte offsets
    if ((long long)(a.N + 15) / 16 * S * 1024 >= 0x7fffffffLL ||
        (long long)(a.M + 15) / 16 * S * 1024 >= 0x7fffffffLL)
        return hipErrorInvalidValue;
    const size_t stride = (size_t)a.M * a.N;
    ProfScope prof(a.name, stream, matmul_bytes(a, a.M), 2.0 * a.M * (double)a.N * a.K);
    SV_LAUNCH(prof, (mfma_gemm_kernel<T::WN, T::WM, T::FN, T::FM, T::NS, T::WPE, EPI>), (unsigned)G,
              T::WN * T::WM * kWave, stream, static_cast<const uint16_t*>(a.W),
              static_cast<const uint16_t*>(a.act), a.M, a.N, a.K, splits, sps, a.out, stride);
    return hipGetLastError();
}

constexpr int kCUs = 256;       // one workgroup per CU (LDS and registers)
constexpr int kMaxSplits = 8;

// Relative rate of a tile (output area per unit time, per workgroup), fitted
// to every tile forced on the 8B-shaped projections and a 128256-row LM head
// at 144-768 rows (medians over the three products): 256 rows 1.00, 192 rows
// 0.96, 128 rows 0.87, 64 rows 0.60.  With these the choice is within 3% of
// the fastest tile at 31 of those 33 points (7.5% at the other two), where
// a 1/BM + 1/BN model lost 23% on the up projection at 576 rows.
template <class T> constexpr double tile_eff() { return T::EFF; }

// Cost of one tile choice: full rounds of kCUs workgroups x the k steps of
// one split x the tile's area, over its efficiency.
template <class T>
double plan_cost(int M, int N, int K, bool can_split, int& splits) {
    const long long tiles = tiles32<T>(M, N);
    const int S = K / 32;
    double best = 1e300;
    splits = 1;
    for (int sp = 1; sp <= (can_split ? kMaxSplits : 1); ++sp) {
        const int sps = (S + sp - 1) / sp;
        if ((long long)sps * (sp - 1) >= S) break;           // an empty split
        if (sp > 1 && sps < 16) break;
        const long long rounds = (tiles * sp + kCUs - 1) / kCUs;
        const double c = (double)rounds * sps * tn32<T>() * tm32<T>() / tile_eff<T>();
        if (c < best * 0.999) {
            best = c;
            splits = sp;
        }
    }
    return best;
}

enum TileId { kT256 = 0, kT192 = 1, kT128 = 2, kT64 = 3 };

int choose_tile(int M, int N, int K, bool can_split, int& splits) {
    int sp[4];
    const double c[4] = {plan_cost<T256>(M, N, K, can_split, sp[0]),
                         plan_cost<T192>(M, N, K, can_split, sp[1]),
                         plan_cost<T128>(M, N, K, can_split, sp[2]),
                         plan_cost<T64>(M, N, K, can_split, sp[3])};
    int best = 0;
    for (int i = 1; i < 4; ++i)
        if (c[i] < c[best] * 0.999) best = i;
    // measurement and test override: SPEC_VERIFY_GEMM_TILE = 256 | 192 | 128 | 64
    // (activation rows per tile)
    if (const char* e = getenv("SPEC_VERIFY_GEMM_TILE")) {
        const int rows = atoi(e);
        if (rows == 256) best = kT256;
        if (rows == 192) best = kT192;
        if (rows == 128) best = kT128;
        if (rows == 64) best = kT64;
    }
    splits = sp[best];
    return best;
}

template <int EPI>
hipError_t launch_epi32(const MatmulArgs& a, int splits, int tile, hipStream_t stream) {
    switch (tile) {
        case kT256: return launch32<T256, EPI>(a, splits, stream);
        case kT192: return launch32<T192, EPI>(a, splits, stream);
        case kT128: return launch32<T128, EPI>(a, splits, stream);
        default: return launch32<T64, EPI>(a, splits, stream);
    }
}

}  // namespace

int tiled_splits(int M, int N, int K) {
    int splits;
    choose_tile(M, N, K, true, splits);
    return splits;
}

hipError_t launch_mfma_tiled(const MatmulArgs& a, hipStream_t stream) {
    if (!a.bf16 || !a.tiled || !a.act_tiled || a.K % 32) return hipErrorInvalidValue;
    if (a.epi == kEpiSilu && a.N % 32) return hipErrorInvalidValue;
    int splits;
    const int tile = choose_tile(a.M, a.N, a.K, a.epi == kEpiResidual, splits);
    if (a.epi == kEpiResidual && splits != (a.splits > 0 ? a.splits : 1))
        return hipErrorInvalidValue;    // the caller's partial planes follow tiled_splits
    switch (a.epi) {
        case kEpiSilu: return launch_epi32<kEpiSilu>(a, 1, tile, stream);
        case kEpiResidual: return launch_epi32<kEpiResidual>(a, splits, tile, stream);
        case kEpiStore: return launch_epi32<kEpiStore>(a, 1, tile, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sv
