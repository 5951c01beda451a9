// device_common.hpp -- small device helpers shared by the gfx950 kernels.
//
// The library is compiled with -ffp-contract=off: every multiply-add that is
// meant to be fused is written as fmaf(), so the quantisers' separate
// binary32 multiply and add stay separate (their codes are defined by those
// two roundings).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));   // converts with v_cvt_pk_bf16_f32 (RNE)

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// binary32 -> bfloat16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t x = __float_as_uint(f);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return ((x >> 16) & 0x8000u) | 0x7FC0u;
    return (x + 0x7FFFu + ((x >> 16) & 1u)) >> 16;
}

// binary32 -> binary16 bits via the hardware conversion (round to nearest
// even; binary16 denormals are kept by the default float mode).  The compiler
// may fuse a preceding multiply into one v_fma_mix (a single rounding, and an
// addend of +0 that turns -0 into +0), so bit-exact outputs use f32_to_f16_rne.
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    _Float16 h = (_Float16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// binary32 -> binary16 bits, round to nearest even, with integer operations
// only: the binary32 value is rounded exactly once more, whatever produced it.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
    const uint32_t x = __float_as_uint(f);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7FFFFFFFu;
    if (ax > 0x7F800000u) return sign | 0x7E00u;            // NaN
    if (ax >= 0x477FF000u) return sign | 0x7C00u;           // >= 65520 rounds to inf
    if (ax >= 0x38800000u) {                                 // binary16 normal range
        uint32_t r = ax - 0x38000000u;                       // rebias the exponent
        r += 0x0FFFu + ((r >> 13) & 1u);                     // ties to even
        return sign | (r >> 13);
    }
    const uint32_t e = ax >> 23;
    if (e < 102u) return sign;                               // below 2^-25: zero
    const uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
    const uint32_t sh = 126u - e;                            // 14..24: units of 2^-24
    uint32_t q = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1u);
    if (rem > half || (rem == half && (q & 1u))) q++;
    return sign | q;
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Sum over the 64 lanes of a wave; every lane gets the total.  Fixed
// butterfly order, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

}  // namespace q4
