// device_common.hpp -- small device helpers shared by the gfx950 kernels.
//
// The library is compiled with -ffp-contract=off: every multiply-add that is
// meant to be fused is written as fmaf(), so the quantisers' separate
// binary32 multiply and add stay separate (their codes are defined by those
// two roundings).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.hpp"   // dtype codes

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


// Reductions over a group of 8 lanes that every lane of the group ends up
// holding.  Only exact, order-free operations go through them (max, integer
// sum), so the grouping does not change any result.
//
// Q8Adjacent: aligned groups of 8 neighbouring lanes, through DPP: 0xB1 swaps
// neighbours, 0x4E swaps pairs within a quad, 0x141 (row_half_mirror) maps
// lane i of the group to lane 7 - i, in the other quad.
struct Q8Adjacent {
    template <int CTRL>
    __device__ static int dpp(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }
    __device__ static float max8(float a) {
        a = fmaxf(a, __int_as_float(dpp<0xB1>(__float_as_int(a))));
        a = fmaxf(a, __int_as_float(dpp<0x4E>(__float_as_int(a))));
        return fmaxf(a, __int_as_float(dpp<0x141>(__float_as_int(a))));
    }
    __device__ static int sum8(int a) {
        a += dpp<0xB1>(a);
        a += dpp<0x4E>(a);
        return a + dpp<0x141>(a);
    }
};

// Q8Strided: the 8 lanes of a wave that agree in lane & 7 (lanes c, c+8, ...,
// c+56): DPP row_ror:8 pairs lane i with i ^ 8 inside its row of 16, and the
// gfx950 lane swaps pair rows (i ^ 16) and wave halves (i ^ 32); a swap of a
// register with itself leaves the lane's own value in one result and its
// partner's in the other.
struct Q8Strided {
    __device__ static int x8(int v) { return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); }
    __device__ static float max8(float a) {
        a = fmaxf(a, __int_as_float(x8(__float_as_int(a))));
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        a = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
    }
    __device__ static int sum8(int a) {
        a += x8(a);
        auto r = __builtin_amdgcn_permlane16_swap((unsigned)a, (unsigned)a, false, false);
        a = (int)(r[0] + r[1]);
        auto t = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)a, false, false);
        return (int)(t[0] + t[1]);
    }
};

// Q8_1 quantisation of one 32-value block by a group of 8 lanes (all active),
// 4 values per lane: d = amax / 127 (binary32), q = round-half-away(v / d)
// via v * (1 / d), s = d * sum(q).  Returns the lane's 4 codes packed
// little-endian; d (and, with WANT_S, s) comes back as binary16 bits (round
// to nearest even), the same on all 8 lanes.  The standalone quantiser and
// the GEMV that quantises its own activation both use it, so they give the
// same bits.
//
// The two binary32 divisions it needs (amax / 127, then 1 / d8) are taken
// through binary64, in a third of the instructions of a binary32 division
// and with the same result for every binary32 input:
//  * a / 127: a binary32 quotient a/127 lies at least 2^-32 (relative) from
//    every binary32 rounding midpoint (a - 127 mid is an odd multiple of the
//    midpoint spacing), and the binary64 product a * RN(1/127) is within
//    2^-52 of it, so rounding that product to binary32 rounds the quotient;
//  * 1 / d: 1/d lies at least about 2^-48 (relative) from every binary32
//    midpoint, and the binary64 reciprocal (v_rcp_f64, within 2^-22) after
//    two Newton steps is within about 2^-52 of it.
// Both were also checked against binary32 division for every non-negative
// finite binary32 input, the reciprocal with a start 2^-22 off in either
// direction and no fused multiply-add (tests/test_q8_division_routes.py
// runs a sample of that sweep).
__device__ __forceinline__ float div127_rne(float a) { return (float)((double)a * (1.0 / 127.0)); }
__device__ __forceinline__ float rcp_rne(float d) {
    const double x = (double)d;
    double r = __builtin_amdgcn_rcp(x);
    double e = __builtin_fma(-x, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-x, r, 1.0);
    r = __builtin_fma(r, e, r);
    return (float)r;
}
template <class G, bool WANT_S>
__device__ __forceinline__ uint32_t q8_1_block(const float (&v)[4], uint32_t& d16, uint32_t& s16) {
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = G::max8(amax);
    const float dd = div127_rne(amax);                 // amax / 127
    const float id = (dd != 0.0f) ? rcp_rne(dd) : 0.0f;   // 1 / dd
    int q[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float t = v[j] * id;
        q[j] = (int)roundf(t);  // half away from zero
        sum += q[j];
    }
    d16 = f32_to_f16_rne(dd);
    if constexpr (WANT_S) {
        sum = G::sum8(sum);
        s16 = f32_to_f16_rne(dd * (float)sum);
    }
    return (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) | ((uint32_t)(q[2] & 0xFF) << 16) |
           ((uint32_t)(q[3] & 0xFF) << 24);
}

// 4 consecutive activation values (bf16 or f32) starting at element e0: the
// raw load, the conversion to binary32, and both in one.
template <int XDT>
using act4_raw_t = std::conditional_t<XDT == DT_F32, float4, u32x2_t>;

template <int XDT>
__device__ __forceinline__ act4_raw_t<XDT> load_act4_raw(const void* x, int64_t e0) {
    if constexpr (XDT == DT_F32) return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + e0);
    else return *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint16_t*>(x) + e0);
}

template <int XDT>
__device__ __forceinline__ void act4_to_f32(const act4_raw_t<XDT>& t, float (&v)[4]) {
    if constexpr (XDT == DT_F32) {
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
        v[0] = bf16_to_f32(t[0] & 0xFFFFu); v[1] = bf16_to_f32(t[0] >> 16);
        v[2] = bf16_to_f32(t[1] & 0xFFFFu); v[3] = bf16_to_f32(t[1] >> 16);
    }
}

template <int XDT>
__device__ __forceinline__ void load_act4(const void* x, int64_t e0, float (&v)[4]) {
    act4_to_f32<XDT>(load_act4_raw<XDT>(x, e0), v);
}

}  // namespace q4
