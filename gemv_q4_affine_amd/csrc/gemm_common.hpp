// gemm_common.hpp -- device helpers shared by the matrix-core GEMM kernels
// (gemm.hip: k_gemm_mfma, k_gemm_pk and the packers; gemm_big.hip: k_gemm_big):
// the raw weight block types, the shift-free nibble dequantiser, the X and
// weight tile image geometry, direct-to-LDS copies and the step barrier.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace q4 {

__device__ __forceinline__ uint32_t perm(uint32_t a, uint32_t sel) { return __builtin_amdgcn_perm(a, a, sel); }

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t h2_bits(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// binary32 -> binary16 bits (RNE), for the affine scale and bias.
__device__ __forceinline__ uint32_t f16b(float f) { return f32_to_f16(f); }

struct GemmArgs {
    const void* a;     // Q4_0 qs / affine q / dense binary16 W
    const void* b;     // Q4_0 d / affine scales
    const void* c;     // affine biases
    const void* x;
    void* y;
    int M, N, K;
    int m_tiles;       // workgroup tiles along M
    int n_tiles;       // workgroup tiles along N
    int ksplit;        // k_gemm_pk: K parts per tile (<= 1: none)
    float* part;       // k_gemm_pk with ksplit > 1: fp32 partial results [ksplit][M][N]
    const int8_t* xexp;  // k_gemm_pk: the X image's row exponents
};


// Raw weight data of one whole 32-weight block of one column.
struct BlkQ4 { u32x4_t q; uint32_t d; };
struct BlkAff { u32x4_t q; uint32_t s, b; };
struct BlkF16 { u32x4_t h[4]; };
// affine 8-bit: one lane's 32 codes (half a group), bytes 0..15 and 16..31
struct BlkAff8 { u32x4_t q[2]; uint32_t s, b; };

template <int WF> struct BlkOf;
template <> struct BlkOf<WF_Q4_0> { using T = BlkQ4; };
template <> struct BlkOf<WF_AFFINE4> { using T = BlkAff; };
template <> struct BlkOf<WF_DENSE16> { using T = BlkF16; };
template <> struct BlkOf<WF_AFFINE8> { using T = BlkAff8; };

// A block past the end of K (K = 32 mod 64) contributes zeros.
template <int WF>
__device__ __forceinline__ void zero_blk(typename BlkOf<WF>::T& r, bool keep) {
    if constexpr (WF == WF_Q4_0) {
        r.d = keep ? r.d : 0u;
    } else if constexpr (WF == WF_AFFINE4 || WF == WF_AFFINE8) {
        r.s = keep ? r.s : 0u;
        r.b = keep ? r.b : 0u;
    } else {
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) r.h[t][e] = keep ? r.h[t][e] : 0u;
    }
}

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void dma2(const void* src, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 2, 0, 0);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
#define Q4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))

// Workgroup barrier for the main loop: this wave's LDS writes are complete
// (lgkmcnt 0) and all but the newest `vm` vector-memory loads have landed,
// which covers the direct-to-LDS copies the next step reads.  Unlike
// __syncthreads() it does not wait for every outstanding load (the release
// fence there would, because a direct-to-LDS copy counts as a pending LDS
// store).  The signal fences stop the compiler from moving memory accesses
// across the barrier; they emit no instructions.
template <int VM>
__device__ __forceinline__ void step_barrier() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range (63 = no constraint)");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0070 | (VM & 0xF) | (((VM >> 4) & 3) << 14));   // lgkmcnt(0), vmcnt(VM)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int kImgRows = 128;            // rows of an image tile
constexpr int kImgTile = kImgRows * 64;  // halves of an image tile (16 KiB)

// Row r of an image tile: chunk c sits at c ^ img_swz(r).  A permutation of
// rows 0..7 and, separately, of the even and of the odd rows among 0..15.
__device__ __forceinline__ int img_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Row exponents of the X image.  The image holds x * 2^e(m) for an integer
// e(m) per row: 0 where the row's largest |x| already lies in [2^-2, 2^15),
// else the e that brings it into [2^14, 2^15), so binary16 keeps the whole
// bfloat16 range.  The GEMM epilogues multiply the fp32 results of row m by
// 2^-e(m).  Both scalings are exact.
//
// The int8 table follows the image (one byte per image row).  An epilogue
// lane (MFMA half h, lane parity p) stores rows 8q + 4h + 2t + p of every
// 32-row sub-tile (q = 0..3, t = 0..1); those 8 exponents sit together at
// byte 8 * (2h + p) of the sub-tile's 32, exponent (q, t) at byte 2q + t, so
// the lane reads them with one 8-byte load and extracts them with constant
// shifts.
__device__ __forceinline__ int xexp_pos(int m) {
    const int r = m & 31;
    const int q = r >> 3, h = (r >> 2) & 1, t = (r >> 1) & 1, p = r & 1;
    return (m & ~31) + 8 * (2 * h + p) + 2 * q + t;
}
// Exponent (q, t) of a lane's 8-byte load.
__device__ __forceinline__ int xexp_of(u32x2_t ex, int q, int t) {
    return (int)(int8_t)(uint8_t)(ex[q >> 1] >> (8 * (2 * (q & 1) + t)));
}
constexpr int kXexpMin = -113, kXexpMax = 127;   // every finite row maximum fits

// Shift-free dequantiser of the packed-X kernel.
//
// A nibble in bits 0-3 of a binary16 with exponent field 0x64 (value 1024,
// unit 1) reads as 1024+q; a nibble in bits 4-7 of a binary16 with exponent
// field 0x54 (value 64, unit 1/16) reads as 64+q.  So the four nibble pairs
// of a 32-bit word come out of word & 0x000F000F, word & 0x00F000F0 and the
// same two masks on word >> 8, each with one AND-OR, one packed subtract
// (exact) and one packed multiply (Q4_0, one rounding) or fma (affine, one
// rounding): 13 instructions per 8 weights.  The price is the order of the
// halves inside each 8-weight fragment, which the X tile in LDS copies:
//   Q4_0   (bytes carry elements b and b+16): positions hold k = 0,2,1,3,4,6,5,7
//   affine (bytes carry elements 2b, 2b+1):  positions hold k = 0,4,1,5,2,6,3,7
// The two masks live in VGPRs (NibMasks, made opaque once per kernel) so that
// each AND-OR is one v_and_or_b32 (a gfx9 VOP3 takes no literal and one SGPR).
struct NibMasks {
    uint32_t lo, hi;
    __device__ __forceinline__ static NibMasks make() {
        NibMasks m{0x000F000Fu, 0x00F000F0u};
        asm volatile("" : "+v"(m.lo), "+v"(m.hi));
        return m;
    }
};
__device__ __forceinline__ uint32_t nib_lo(uint32_t w, const NibMasks& m) { return (w & m.lo) | 0x64006400u; }   // 1024+q
__device__ __forceinline__ uint32_t nib_hi(uint32_t w, const NibMasks& m) { return (w & m.hi) | 0x54005400u; }   // 64+q

// Per-block constants of the dequantiser: Q4_0 d in both halves; affine
// scale and bias in both halves (binary16).
struct BlkConst {
    half2_t c0, c1;
};
template <int WF>
__device__ __forceinline__ BlkConst blk_const(const typename BlkOf<WF>::T& r) {
    if constexpr (WF == WF_Q4_0) {
        const half2_t dd = as_h2(__builtin_amdgcn_perm(r.d, r.d, 0x01000100u));
        return {dd, dd};
    } else {
        static_assert(WF == WF_AFFINE4 || WF == WF_AFFINE8, "quantised formats only");
        const uint32_t s16 = f16b(bf16_to_f32(r.s));
        const uint32_t b16 = f16b(bf16_to_f32(r.b));
        return {as_h2(s16 | (s16 << 16)), as_h2(b16 | (b16 << 16))};
    }
}

// The 8 weights of 32-bit word w of a block, into their fragment slots.
//  Q4_0: word w holds the low nibbles of elements 4w..4w+3 (fragment w/2,
//        pairs 2(w%2), 2(w%2)+1) and the high nibbles 16+4w.. (fragment
//        2 + w/2, same pairs).
//  affine: word w holds elements 8w..8w+7 (fragment w, all four pairs).
template <int WF>
__device__ __forceinline__ void blk_word(const typename BlkOf<WF>::T& r, const BlkConst& c, int w, const NibMasks& m,
                                         u32x4_t (&out)[4]) {
    const uint32_t word = r.q[w];
    const uint32_t sh = word >> 8;
    if constexpr (WF == WF_Q4_0) {
        const half2_t clo = as_h2(0xE408E408u);   // -1032
        const half2_t chi = as_h2(0xD480D480u);   // -72
        const int h = w >> 1, p = 2 * (w & 1);
        out[h][p + 0] = h2_bits((as_h2(nib_lo(word, m)) + clo) * c.c0);
        out[h][p + 1] = h2_bits((as_h2(nib_lo(sh, m)) + clo) * c.c0);
        out[2 + h][p + 0] = h2_bits((as_h2(nib_hi(word, m)) + chi) * c.c0);
        out[2 + h][p + 1] = h2_bits((as_h2(nib_hi(sh, m)) + chi) * c.c0);
    } else {
        const half2_t clo = as_h2(0xE400E400u);   // -1024
        const half2_t chi = as_h2(0xD400D400u);   // -64
        out[w][0] = h2_bits(__builtin_elementwise_fma(as_h2(nib_lo(word, m)) + clo, c.c0, c.c1));
        out[w][1] = h2_bits(__builtin_elementwise_fma(as_h2(nib_hi(word, m)) + chi, c.c0, c.c1));
        out[w][2] = h2_bits(__builtin_elementwise_fma(as_h2(nib_lo(sh, m)) + clo, c.c0, c.c1));
        out[w][3] = h2_bits(__builtin_elementwise_fma(as_h2(nib_hi(sh, m)) + chi, c.c0, c.c1));
    }
}

// The affine 8-bit dequantiser.  A code byte q placed under the high byte
// 0x64 reads as the binary16 1024+q (unit 1), so one v_perm_b32 makes two
// weights' 1024+q from a 32-bit word of codes and the constant 0x64646464;
// a packed subtract (exact) and a packed fma with the group's scale and bias
// (one rounding) finish them: 12 instructions per 8 weights, in element
// order (the X tile keeps its natural order).  The constant and the two
// byte selectors live in VGPRs (made opaque once per kernel).
struct Perm8 {
    uint32_t hi, sel01, sel23;
    __device__ __forceinline__ static Perm8 make() {
        Perm8 p{0x64646464u, 0x04010400u, 0x04030402u};
        asm volatile("" : "+v"(p.hi), "+v"(p.sel01), "+v"(p.sel23));
        return p;
    }
};
// Fragment f (elements 8f..8f+7 of the lane's 32 codes) into out[f].
__device__ __forceinline__ void blk_word(const BlkAff8& r, const BlkConst& c, int f, const Perm8& p,
                                         u32x4_t (&out)[4]) {
    const half2_t base = as_h2(0xE400E400u);   // -1024
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t word = r.q[f >> 1][2 * (f & 1) + h];
        const half2_t v01 = as_h2(__builtin_amdgcn_perm(p.hi, word, p.sel01)) + base;
        const half2_t v23 = as_h2(__builtin_amdgcn_perm(p.hi, word, p.sel23)) + base;
        out[f][2 * h] = h2_bits(__builtin_elementwise_fma(v01, c.c0, c.c1));
        out[f][2 * h + 1] = h2_bits(__builtin_elementwise_fma(v23, c.c0, c.c1));
    }
}

// Fragment w of a block: the nibble dequantiser (NibMasks) or the 8-bit one
// (Perm8).
template <int WF, class MK>
__device__ __forceinline__ void blk_fragment(const typename BlkOf<WF>::T& r, const BlkConst& c, int w, const MK& m,
                                             u32x4_t (&out)[4]) {
    if constexpr (WF == WF_AFFINE8) blk_word(r, c, w, m, out);
    else blk_word<WF>(r, c, w, m, out);
}
// The constants each dequantiser keeps in VGPRs.
template <int WF> struct DequantConsts { using T = NibMasks; };
template <> struct DequantConsts<WF_AFFINE8> { using T = Perm8; };

template <int WF, class MK>
__device__ __forceinline__ void blk_frags_perm(const typename BlkOf<WF>::T& r, const MK& m, u32x4_t (&out)[4]) {
    const BlkConst c = blk_const<WF>(r);
#pragma unroll
    for (int w = 0; w < 4; w++) blk_fragment<WF>(r, c, w, m, out);
}


// Weight image for k_gemm_pk: for every 256-column tile and 64-wide K step a
// contiguous 9 KiB chunk, ((nt * ksteps) + k) * kWChunk bytes in,
//   bytes    0..8191  nibble blocks, block-plane major: [blk 0..1][col 0..255][16 B]
//   bytes 8192..9215  Q4_0:   d  as binary16 [blk 0..1][col 0..255]
//                     affine: s  as bfloat16 [col 0..255], then b [col 0..255]
// Columns past N and blocks past K are zero (scale 0: the weights are 0).
// The block-plane order puts the 16-byte block reads of consecutive columns in
// consecutive LDS units (no bank conflicts), and a chunk travels as nine
// contiguous 1 KiB direct-to-LDS copies.
constexpr int kWChunk = 9216;

// Affine 8-bit weight image, the same tiling with a 17 KiB chunk:
//   bytes     0..16383  codes, plane major: [plane 0..3][col 0..255][16 B],
//                       plane 2g + h holding elements 32g + 16h .. +15 of the
//                       column's 64-code group
//   bytes 16384..17407  s as bfloat16 [col 0..255], then b [col 0..255]
// A lane that dequantises elements 32g .. 32g+31 of a column reads planes 2g
// and 2g+1: two conflict-free 16-byte reads.
constexpr int kWChunk8 = 17408;
template <int WF> constexpr int w_chunk_bytes() { return WF == WF_AFFINE8 ? kWChunk8 : kWChunk; }

}  // namespace q4
