// Device-side helpers shared by the verification-step kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---- bf16 <-> fp32 ---------------------------------------------------------
// bf16 values travel as raw 16-bit patterns (uint16_t); two of them packed in
// a 32-bit word hold the lower-index element in the low half.
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Round fp32 to bf16, nearest-even; NaN stays NaN (quiet).  gfx950's
// v_cvt_pk_bf16_f32 does it in one instruction for two values; it matches the
// integer definition (b + 0x7fff + ((b >> 16) & 1)) >> 16, NaN -> (b >> 16) |
// 0x40, on every one of the 2^32 fp32 bit patterns (checked exhaustively on
// the GPU).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// lo in bits 15:0, hi in bits 31:16
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// ---- copies into LDS ----------------------------------------------------------
// LDS pointers for __builtin_amdgcn_global_load_lds (one 16-byte piece per
// lane, written lane-contiguously at the wave-uniform LDS address).  Those
// copies are counted on vmcnt like any vector load, and the compiler does not
// wait for them before reading the LDS they fill: the kernels wait explicitly.
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ---- activation functions ---------------------------------------------------
__device__ __forceinline__ float silu(float u) { return u / (1.0f + expf(-u)); }

// ---- wave / block reductions ------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// ---- Philox4x32-10 ------------------------------------------------------------
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): per round, words 0 and 2 are multiplied by two fixed odd constants;
// the high halves are xor-ed with words 1/3 and the round key, the low halves
// become words 1/3; the key advances by the two Weyl increments between rounds.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return c0;
}

// Acceptance uniform in (0, 1] and resampling uniform in [0, 1); both are
// multiples of 2^-24, so exact in fp32.
__device__ __forceinline__ float u_accept(uint32_t w) { return (float)((w >> 8) + 1u) * 0x1.0p-24f; }
__device__ __forceinline__ float u_resample(uint32_t w) { return (float)(w >> 8) * 0x1.0p-24f; }

}  // namespace sv
