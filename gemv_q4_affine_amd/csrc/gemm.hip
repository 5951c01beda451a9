// gemm.hip -- fused dequantise + matrix-core GEMM on gfx950.
//
//   Y[M,N] = X[M,K] . dequant(Wq)[N,K]^T,  fp32 accumulation.
//
// The prefill kernel of the pages: dequantised weight tiles are made once
// and reused across every token row of the tile, the K loop is software
// pipelined (next tiles fetched while the current one is multiplied), and the
// matrix engine does the contraction (llama.cpp PR "et-backend: Q4_0
// matrix-engine GEMM rewrite for prefill", Overview; MLX issue #4621 for the
// affine format and the dequantise-then-matmul alternative).
//
// gfx950 design
//  * Operand precision.  The MFMA runs in binary16 (v_mfma_f32_32x32x16_f16
//    and v_mfma_f32_16x16x32_f16): X (bfloat16) converts to binary16 exactly
//    in binary16's normal range, and a dequantised weight (q-8)*d is rounded
//    once to binary16 (relative error <= 2^-11).  Rounding the weights to
//    bfloat16 instead (what a bf16 MFMA would need) costs about 1.6e-3
//    relative error on top of the 1.6e-3 of the bf16 output, which together
//    exceed the 2e-3 error bar; binary16 weights stay well inside it.
//  * Weights are dequantised in registers, never written back: the nibbles
//    become binary16 1024+q (or 64+q) with one AND-OR against a binary16
//    exponent at which the nibble's unit in the last place is 1, then one
//    packed subtract and one packed multiply (Q4_0) or fma (affine) give the
//    weight, rounded once.  A weight is dequantised once per M tile of the
//    workgroup -- the "static reuse across token tiles" of the ET-SoC-1
//    rewrite.
//  * Large M (k_gemm_pk): X is converted once into a binary16 tile image that
//    direct-to-LDS copies move straight into a 4-deep LDS ring together with
//    the raw weight blocks; compute waves overlap each K step's MFMAs with the
//    next step's dequantisation, one barrier per K step.  Without a workspace
//    for the image, k_gemm_mfma converts X on the way into LDS instead.
//  * Small M (k_gemm_skinny): weights stream once from HBM at full rate and
//    the waves of a workgroup split K; M == 1 (k_gemv_x) runs the decode
//    GEMV's layout with fp32 dot2 products on bf16 / binary16 X.
//  * Each MFMA sums over 16 (or 32) K slots; the slot -> k assignment only has
//    to agree between the A and B operands, so it is chosen to match each
//    weight format's nibble order and the B loader needs no byte shuffles
//    beyond one v_perm or shift per pair.
#include <type_traits>

#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace q4 {

// ---------------------------------------------------------------------------
// Weight fragment loaders.
//
// A fragment covers one 32-column tile and one 32-wide K step (two 32x32x16
// MFMAs, s = 0, 1).  Lane l owns column j = l % 32 and lane group g = l / 32;
// in MFMA s it supplies the 8 halves for K slots 8g..8g+7, which stand for
// k = kofs(s, g) + v, v = 0..7, of the 32-wide step.  The X fragment read
// from LDS uses the same kofs.
// ---------------------------------------------------------------------------


// Two nibble codes (in bits 0-3 and 16-19 after masking) -> binary16 (q-8)*d.
__device__ __forceinline__ uint32_t q4_pair(uint32_t t, half2_t dd) {
    const half2_t v = as_h2((t & 0x000F000Fu) | 0x64006400u);      // 1024 + q
    const half2_t c = as_h2(0xE408E408u);                             // -1032
    return h2_bits((v + c) * dd);                                     // (q - 8) * d, RNE
}

struct RawQ4 {      // raw Q4_0 data of one fragment: 8 nibble bytes and the scale
    u32x2_t q;
    uint32_t d;
};

struct Frag16 {     // 8 halves for each of the two 16-wide K halves
    u32x4_t s[2];
};

// Q4_0: lane group g takes bytes 8g..8g+7 of the block: low nibbles are
// elements 8g+v (MFMA s = 0), high nibbles 16+8g+v (s = 1): kofs = 16s + 8g.
__device__ __forceinline__ Frag16 q4_0_frag(const RawQ4& r) {
    const half2_t dd = as_h2(r.d | (r.d << 16));
    Frag16 f;
#pragma unroll
    for (int w = 0; w < 2; w++) {
        const uint32_t word = r.q[w];
        const uint32_t t01 = perm(word, 0x0C010C00u);   // byte0 | byte1 << 16
        const uint32_t t23 = perm(word, 0x0C030C02u);   // byte2 | byte3 << 16
        f.s[0][2 * w + 0] = q4_pair(t01, dd);
        f.s[0][2 * w + 1] = q4_pair(t23, dd);
        f.s[1][2 * w + 0] = q4_pair(t01 >> 4, dd);
        f.s[1][2 * w + 1] = q4_pair(t23 >> 4, dd);
    }
    return f;
}

struct RawAff {     // raw affine data: 8 nibble bytes, scale and bias (bf16 bits)
    u32x2_t q;
    uint32_t s, b;
};


// Affine: byte i holds elements 2i (low) and 2i+1 (high).  Lane group g takes
// bytes 8g..8g+7 = elements 16g..16g+15: s = 0 gets 16g+v, s = 1 gets
// 16g+8+v: kofs = 16g + 8s.  Value q*s + b, one binary16 fma (one rounding).
__device__ __forceinline__ Frag16 affine_frag(const RawAff& r) {
    const uint32_t s16 = f16b(bf16_to_f32(r.s));
    const uint32_t b16 = f16b(bf16_to_f32(r.b));
    // lane 0 of a pair holds q_lo (unit 1), lane 1 holds 16*q_hi (unit 16):
    // scale the high lane by 1/16 (exact) folded into its scale.
    const half2_t sc = as_h2(s16 | (f16b(bf16_to_f32(r.s) * 0.0625f) << 16));
    const half2_t bb = as_h2(b16 | (b16 << 16));
    const half2_t c = as_h2(0xE400E400u);   // -1024
    Frag16 f;
#pragma unroll
    for (int w = 0; w < 2; w++) {
        const uint32_t word = r.q[w];
#pragma unroll
        for (int p = 0; p < 4; p++) {
            // byte p -> (low nibble in bits 0-3, high nibble kept in bits 20-23)
            const uint32_t t = perm(word, 0x0C000C00u + (uint32_t)p * 0x00010001u);
            const half2_t v = as_h2((t & 0x00F0000Fu) | 0x64006400u);   // 1024+q_lo, 1024+16 q_hi
            const half2_t q = v + c;                                     // q_lo, 16 q_hi (exact)
            const half2_t y = __builtin_elementwise_fma(q, sc, bb);     // q*s + b
            f.s[w][p] = h2_bits(y);
        }
    }
    return f;
}

// ---------------------------------------------------------------------------
// Large-M kernel: workgroup = 4 waves side by side along N; each wave owns
// NT 32-column tiles and all MT 32-row tiles of the workgroup's M range.
//
// K advances 64 per iteration (two 32-weight blocks).  In the four
// 32x32x16 MFMAs of an iteration (s = 0..3), lane (j = l % 32, g = l / 32)
// supplies elements 8s..8s+7 of block 2k+g of column j: one 128-bit load
// brings the lane its whole block, and the X fragment it pairs with is
// X[i][64k + 32g + 8s .. +8].
// ---------------------------------------------------------------------------
constexpr int kStep = 64;            // K per iteration
constexpr int kLdsStride = 72;       // halves per staged X row (64 + 8 padding)

// Two binary32 values -> packed binary16, each rounded to nearest even (the
// rounding of the X image, so that every path converts X alike).
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
    return f32_to_f16(lo) | (f32_to_f16(hi) << 16);
}

// 8 consecutive X values (bf16 or f32) -> 8 binary16 values (skinny kernel).
template <int XDT>
__device__ __forceinline__ u32x4_t load_x8(const void* x, int64_t off, bool ok) {
    u32x4_t r = {0u, 0u, 0u, 0u};
    if (!ok) return r;
    if (XDT == DT_BF16) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(x) + off);
#pragma unroll
        for (int i = 0; i < 4; i++) r[i] = cvt_pk(__uint_as_float(v[i] << 16), __uint_as_float(v[i] & 0xFFFF0000u));
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
        const float4 v0 = p[0], v1 = p[1];
        r[0] = cvt_pk(v0.x, v0.y); r[1] = cvt_pk(v0.z, v0.w);
        r[2] = cvt_pk(v1.x, v1.y); r[3] = cvt_pk(v1.z, v1.w);
    }
    return r;
}

// Raw X loads for the staging pipeline (converted later): 8 values per unit.
template <int XDT>
struct RawX8 { u32x4_t lo, hi; };   // bf16: lo only; f32: lo = values 0..3, hi = 4..7

template <int XDT>
__device__ __forceinline__ RawX8<XDT> load_x8_raw(const void* x, int64_t off) {
    RawX8<XDT> r;
    if constexpr (XDT == DT_BF16) {
        r.lo = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(x) + off);
        r.hi = r.lo;
    } else {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const float*>(x) + off);
        r.lo = p[0];
        r.hi = p[1];
    }
    return r;
}

template <int XDT>
__device__ __forceinline__ u32x4_t convert_x8(const RawX8<XDT>& v) {
    u32x4_t r;
    if constexpr (XDT == DT_BF16) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            r[i] = cvt_pk(__uint_as_float(v.lo[i] << 16), __uint_as_float(v.lo[i] & 0xFFFF0000u));
    } else {
        r[0] = cvt_pk(__uint_as_float(v.lo[0]), __uint_as_float(v.lo[1]));
        r[1] = cvt_pk(__uint_as_float(v.lo[2]), __uint_as_float(v.lo[3]));
        r[2] = cvt_pk(__uint_as_float(v.hi[0]), __uint_as_float(v.hi[1]));
        r[3] = cvt_pk(__uint_as_float(v.hi[2]), __uint_as_float(v.hi[3]));
    }
    return r;
}

__device__ __forceinline__ void store_y(void* y, int ydt, int64_t off, float v) {
    if (ydt == DT_F32) reinterpret_cast<float*>(y)[off] = v;
    else reinterpret_cast<uint16_t*>(y)[off] = (uint16_t)f32_to_bf16(v);
}


// Block kblk of column n.  Callers pass a clamped, valid (n, kblk): the load
// is unconditional so that it never waits inside a branch.
template <int WF>
__device__ __forceinline__ typename BlkOf<WF>::T load_blk(const GemmArgs& a, int n, int kblk) {
    typename BlkOf<WF>::T r;
    const int nb = a.K / 32;
    if constexpr (WF == WF_Q4_0) {
        r.q = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(a.a) + ((int64_t)n * nb + kblk) * 16));
        r.d = reinterpret_cast<const uint16_t*>(a.b)[(int64_t)n * nb + kblk];
    } else if constexpr (WF == WF_AFFINE4) {
        r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const uint8_t*>(a.a) + (int64_t)n * (a.K / 2) + (int64_t)kblk * 16));
        const int64_t gi = (int64_t)n * (a.K / 64) + (kblk >> 1);
        r.s = reinterpret_cast<const uint16_t*>(a.b)[gi];
        r.b = reinterpret_cast<const uint16_t*>(a.c)[gi];
    } else {
        const u32x4_t* w = reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const uint16_t*>(a.a) + (int64_t)n * a.K + (int64_t)kblk * 32);
#pragma unroll
        for (int t = 0; t < 4; t++) r.h[t] = w[t];
    }
    return r;
}


// Elements 8t..8t+7 of a block as 8 binary16 values, t = 0..3.
template <int WF>
__device__ __forceinline__ void blk_frags(const typename BlkOf<WF>::T& r, u32x4_t (&out)[4]) {
    if constexpr (WF == WF_Q4_0) {
        const half2_t dd = as_h2(r.d | (r.d << 16));
        // t = 0: low nibbles of bytes 0..7, t = 1: low of 8..15,
        // t = 2: high nibbles of bytes 0..7, t = 3: high of 8..15
#pragma unroll
        for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int w = 0; w < 2; w++) {
                const uint32_t word = r.q[2 * h + w];
                const uint32_t t01 = perm(word, 0x0C010C00u);
                const uint32_t t23 = perm(word, 0x0C030C02u);
                out[h][2 * w + 0] = q4_pair(t01, dd);
                out[h][2 * w + 1] = q4_pair(t23, dd);
                out[2 + h][2 * w + 0] = q4_pair(t01 >> 4, dd);
                out[2 + h][2 * w + 1] = q4_pair(t23 >> 4, dd);
            }
        }
    } else if constexpr (WF == WF_AFFINE4) {
        // element 8t+v sits in word t: byte v/2, low nibble for even v
        RawAff lo, hi;
        lo.s = hi.s = r.s;
        lo.b = hi.b = r.b;
        lo.q = u32x2_t{r.q[0], r.q[1]};
        hi.q = u32x2_t{r.q[2], r.q[3]};
        const Frag16 f0 = affine_frag(lo);   // s[0] = word 0, s[1] = word 1
        const Frag16 f1 = affine_frag(hi);
        out[0] = f0.s[0];
        out[1] = f0.s[1];
        out[2] = f1.s[0];
        out[3] = f1.s[1];
    } else {
#pragma unroll
        for (int t = 0; t < 4; t++) out[t] = r.h[t];
    }
}

// Quantised weights reach the workgroup through LDS: direct-to-LDS loads
// (global_load_lds: no registers held while in flight) copy the raw blocks
// of the workgroup's 4*NT*32 columns for one K step (2 blocks per column)
// into one of 4 slots, three steps before the step is multiplied.  Every
// load instruction reads 32 columns x 32 contiguous bytes.
constexpr int kSlots = 4;

template <int WF, int NT>
struct WStage;
// A 2-byte direct-to-LDS load puts each lane's value in a 4-byte slot (lane i
// at byte 4i, zero-extended), so the 16-bit scales occupy one dword each.
template <int NT>
struct WStage<WF_Q4_0, NT> {
    static constexpr int kCols = 4 * NT * 32;
    uint8_t q[kSlots][kCols][2][16];      // raw nibble blocks
    uint32_t d[kSlots][kCols][2];         // binary16 scales
};
template <int NT>
struct WStage<WF_AFFINE4, NT> {
    static constexpr int kCols = 4 * NT * 32;
    uint8_t q[kSlots][kCols][2][16];      // raw nibbles (2 blocks = one group)
    uint32_t s[kSlots][kCols];            // bfloat16 scale of the group
    uint32_t b[kSlots][kCols];            // bfloat16 bias of the group
};
template <int NT>
struct WStage<WF_DENSE16, NT> {
    uint32_t unused;
};


template <int WF, int MT, int NT, int XDT, int YDT>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma(const GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][MT * 32 * kLdsStride];
    constexpr bool kStaged = WF != WF_DENSE16;
    __shared__ __attribute__((aligned(16))) WStage<WF, NT> ws;
    using Blk = typename BlkOf<WF>::T;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;
    const int g = lane >> 5;

    const int wg = blockIdx.x;
    const int mt_idx = wg % a.m_tiles;
    const int nt_idx = wg / a.m_tiles;
    const int m0 = mt_idx * MT * 32;
    const int nwg0 = nt_idx * (4 * NT * 32);
    const int n0 = nwg0 + wave * NT * 32;
    const int nb = a.K / 32;
    const int nsteps = (nb + 1) / 2;                 // a last step may hold one block only

    // X staging: units of 8 values; unit u -> row u / 8, column (u % 8) * 8
    constexpr int kUnits = MT * 32 * 8;
    constexpr int kUnitsPerThread = (kUnits + 255) / 256;
    int xrow[kUnitsPerThread], xcol[kUnitsPerThread];
    int64_t xoff[kUnitsPerThread];
#pragma unroll
    for (int t = 0; t < kUnitsPerThread; t++) {
        const int u = tid + t * 256;
        xrow[t] = u >> 3;
        xcol[t] = (u & 7) * 8;
        const int m = m0 + xrow[t];
        xoff[t] = (int64_t)(m < a.M ? m : a.M - 1) * a.K;   // clamped: padded rows are never stored
    }
    // weight columns (clamped: padded columns are never stored)
    int wn[NT];
#pragma unroll
    for (int ni = 0; ni < NT; ni++) {
        const int n = n0 + ni * 32 + j;
        wn[ni] = n < a.N ? n : a.N - 1;
    }

    floatx16_t acc[MT][NT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mi][ni][v] = 0.0f;

    RawX8<XDT> xr[kUnitsPerThread];
    Blk wr[NT];
    u32x4_t bf[NT][4];

    auto load_x = [&](int k) {
#pragma unroll
        for (int t = 0; t < kUnitsPerThread; t++) {
            const int col = k * kStep + xcol[t];
            xr[t] = load_x8_raw<XDT>(a.x, xoff[t] + (col < a.K ? col : a.K - 8));
        }
    };
    // raw weights of step k (blocks 2k, 2k+1 of the workgroup's columns) -> slot k % 4
    constexpr int kCols = 4 * NT * 32;
    constexpr int kDmaQ = kCols * 2 / 256;                 // 16-byte block loads per wave
    constexpr int kDmaS = (WF == WF_Q4_0) ? kCols * 2 / 256 : 2 * kCols / 256;   // 2-byte loads per wave
    constexpr int kDmaPerStep = kStaged ? kDmaQ + kDmaS : 0;
    auto dma_step = [&](int k) {
        if constexpr (kStaged) {
            const int slot = k & (kSlots - 1);
#pragma unroll
            for (int i = 0; i < kDmaQ; i++) {
                const int q = wave * kDmaQ + i;             // 32 columns x 2 blocks
                int n = nwg0 + q * 32 + (lane >> 1);
                n = n < a.N ? n : a.N - 1;
                int blk = 2 * k + (lane & 1);
                blk = blk < nb ? blk : nb - 1;
                const uint8_t* src = (WF == WF_Q4_0)
                    ? reinterpret_cast<const uint8_t*>(a.a) + ((int64_t)n * nb + blk) * 16
                    : reinterpret_cast<const uint8_t*>(a.a) + (int64_t)n * (a.K / 2) + (int64_t)blk * 16;
                dma16(src, &ws.q[slot][q * 32][0][0]);
            }
            if constexpr (WF == WF_Q4_0) {
#pragma unroll
                for (int i = 0; i < kDmaS; i++) {
                    const int q = wave * kDmaS + i;         // 64 scale entries
                    int n = nwg0 + q * 32 + (lane >> 1);
                    n = n < a.N ? n : a.N - 1;
                    int blk = 2 * k + (lane & 1);
                    blk = blk < nb ? blk : nb - 1;
                    dma2(reinterpret_cast<const uint16_t*>(a.b) + (int64_t)n * nb + blk, &ws.d[slot][q * 32][0]);
                }
            } else {
                const int ng = a.K / 64;
                int gi = k < ng ? k : ng - 1;
#pragma unroll
                for (int i = 0; i < kDmaS / 2; i++) {
                    const int q = wave * (kDmaS / 2) + i;   // 64 columns
                    int n = nwg0 + q * 64 + lane;
                    n = n < a.N ? n : a.N - 1;
                    dma2(reinterpret_cast<const uint16_t*>(a.b) + (int64_t)n * ng + gi, &ws.s[slot][q * 64]);
                    dma2(reinterpret_cast<const uint16_t*>(a.c) + (int64_t)n * ng + gi, &ws.b[slot][q * 64]);
                }
            }
        }
    };
    // registers for the weights of step k: from the LDS slot, or from global (dense)
    auto fetch_w = [&](int k) {
        if constexpr (kStaged) {
            const int slot = k & (kSlots - 1);
#pragma unroll
            for (int ni = 0; ni < NT; ni++) {
                const int cw = wave * NT * 32 + ni * 32 + j;
                wr[ni].q = *reinterpret_cast<const u32x4_t*>(&ws.q[slot][cw][g][0]);
                if constexpr (WF == WF_Q4_0) {
                    wr[ni].d = ws.d[slot][cw][g] & 0xFFFFu;
                } else {
                    wr[ni].s = ws.s[slot][cw] & 0xFFFFu;
                    wr[ni].b = ws.b[slot][cw] & 0xFFFFu;
                }
            }
        } else {
            const int kblk = 2 * k + g;
#pragma unroll
            for (int ni = 0; ni < NT; ni++) wr[ni] = load_blk<WF>(a, wn[ni], kblk < nb ? kblk : nb - 1);
        }
    };
    auto stage_step = [&](int k, int dst) {
#pragma unroll
        for (int t = 0; t < kUnitsPerThread; t++) {
            if (tid + t * 256 < kUnits) {
                u32x4_t v = convert_x8<XDT>(xr[t]);
                const bool ok = k * kStep + xcol[t] < a.K;
#pragma unroll
                for (int e = 0; e < 4; e++) v[e] = ok ? v[e] : 0u;
                *reinterpret_cast<u32x4_t*>(&lds[dst][xrow[t] * kLdsStride + xcol[t]]) = v;
            }
        }
        if constexpr (kStaged) fetch_w(k);
        const bool bok = 2 * k + g < nb;
#pragma unroll
        for (int ni = 0; ni < NT; ni++) {
            zero_blk<WF>(wr[ni], bok);
            blk_frags<WF>(wr[ni], bf[ni]);
        }
    };
    auto mfmas = [&](int k) {
        const uint16_t* la = lds[k & 1];
#pragma unroll
        for (int s = 0; s < 4; s++) {
#pragma unroll
            for (int mi = 0; mi < MT; mi++) {
                const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&la[(mi * 32 + j) * kLdsStride + 32 * g + 8 * s]);
                const half8_t ah = __builtin_bit_cast(half8_t, av);
#pragma unroll
                for (int ni = 0; ni < NT; ni++)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        ah, __builtin_bit_cast(half8_t, bf[ni][s]), acc[mi][ni], 0, 0, 0);
            }
        }
    };

    // prologue: raw weights of steps 0 and 1 requested and step 0 staged; then
    // step 1's X and step 2's weights go in flight in the same order as in
    // the main loop (X, then weights), so that the loop's waits are exact
    dma_step(0);
    if (nsteps > 1) dma_step(1);
    load_x(0);
    if constexpr (!kStaged) fetch_w(0);
    Q4_WAIT_VMCNT(0);
    __syncthreads();
    stage_step(0, 0);
    if (nsteps > 1) {
        load_x(1);
        if constexpr (!kStaged) fetch_w(1);
    }
    if (nsteps > 2) dma_step(2);
    __syncthreads();

    // main loop: every iteration requests the raw weights of step k+3
    int k = 0;
    for (; k + 3 < nsteps; k++) {
        mfmas(k);
        stage_step(k + 1, (k + 1) & 1);               // X loaded during the previous iteration
        load_x(k + 2);                                // the next X goes in flight
        if constexpr (!kStaged) fetch_w(k + 2);
        dma_step(k + 3);
        // step k+2's weights (requested one iteration ago) must have landed:
        // only this iteration's X loads and weight requests may be in flight
        if constexpr (kStaged) step_barrier<kUnitsPerThread + kDmaPerStep>();
        else __syncthreads();
    }
    // last iterations: nothing left to request
    for (; k < nsteps; k++) {
        mfmas(k);
        if (k + 1 < nsteps) stage_step(k + 1, (k + 1) & 1);
        if (k + 2 < nsteps) {
            load_x(k + 2);
            if constexpr (!kStaged) fetch_w(k + 2);
        }
        __syncthreads();
    }

    // epilogue: lane holds column j of each tile, rows 8*(v/4) + 4*g + v%4
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++) {
            const int n = n0 + ni * 32 + j;
            if (n >= a.N) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int m = m0 + mi * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                if (m < a.M) store_y(a.y, YDT, (int64_t)m * a.N + n, acc[mi][ni][v]);
            }
        }
}

// ---------------------------------------------------------------------------
// Packed-X large-M kernel.
//
// X is first converted once to a binary16 "LDS image" (k_pack_x): for each
// 128-row M tile and 64-wide K step a 16 KiB tile laid out exactly as the
// GEMM keeps it in LDS.  Inside a tile row r (128 bytes) stores its 16-byte
// chunk c (k = 8c..8c+7) at chunk position c ^ img_swz(r) -- an XOR swizzle
// that puts the 128-bit fragment reads of 8 consecutive rows (one 128-byte
// bank sweep) and of 16 consecutive rows (256 bytes) in distinct banks
// without padding -- and the halves of a chunk follow the fragment order of
// blk_frags_perm.  Rows past M and steps past K are zero.  The GEMM then never
// converts X: its producer waves only issue direct-to-LDS copies.
//
// Persistent workgroups of 8 waves, one per CU, each running a stream of
// 128 x 256 output tiles:
//  * waves 0-3 (consumers) own NT 32-column tiles each and all MT 32-row tiles
//    of the current output tile; per K step they run the MFMAs of step k while
//    dequantising the weights of step k+1 into registers, interleaved
//    instruction by instruction (one basic block per step);
//  * waves 4-7 (producers, one per SIMD) copy the X tile and the raw weight
//    blocks (and scales) of step k+3 into a 4-deep LDS ring with
//    direct-to-LDS loads and, before each barrier, wait until step k+2 has
//    landed.  They issue no other memory operation, so the count in that
//    wait is exact.  Their stream runs on across tile boundaries.
// One barrier per K step.  At the end of each tile the consumers write the
// output straight from the accumulators (pairs of columns per store) and
// go on with the next tile, whose first steps are already in LDS.
// ---------------------------------------------------------------------------
// Ring depth: steps k..k+3 resident (100 KiB; 132 KiB with the 17 KiB affine
// 8-bit chunks); producers request step k + depth - 1 during step k.  A
// 6-deep ring was slower: the slot of step k (k mod 6) costs address
// arithmetic on every LDS read of the compute waves, k mod 4 almost none.
template <int WF> constexpr int pk_slots() { return 4; }
constexpr int kPkProducers = 4;          // producer waves, one per SIMD
// X -> image (see above), one workgroup of 256 threads per image row.  The
// workgroup first finds the row's largest |x|.  A row whose largest lies in
// [2^-2, 2^15) is converted as it is (e = 0: the same bits as a direct
// conversion); any other row is scaled by 2^e, e = 14 - floor(log2 max), so
// its largest lands in [2^14, 2^15) (a zero or non-finite maximum keeps
// e = 0).  Then the row's chunks are written as binary16 of x * 2^e, rounded
// to nearest even, and e to the exponent table.  For bfloat16 X of a scaled
// row every value within 2^-31 of the row's largest converts exactly.  Rows
// past M and steps past K are zero.
// Workgroup blk of the packer (image row blk); wave_max: 4 floats of LDS.
template <int WF, int XDT>
__device__ __forceinline__ void pack_x_body(int blk, float* wave_max, const void* __restrict__ x,
                                            uint16_t* __restrict__ img, int8_t* __restrict__ xexp, int M, int K,
                                            int ksteps) {
    constexpr int kBatch = 2;                   // chunks per thread held in registers (K <= 4096 in one batch)
    using Raw = RawX8<XDT>;
    const int m = blk;
    const int tid = threadIdx.x;
    const int nch = ksteps * 8;                 // 16-byte chunks of an image row
    const int kch = m < M ? K / 8 : 0;          // chunks holding X (K % 32 == 0)
    const int64_t xoff = (int64_t)m * K;
    auto absmax = [](const Raw& v, float mx) {
        if constexpr (XDT == DT_BF16) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(v.lo[i] << 16)), fabsf(__uint_as_float(v.lo[i] & 0xFFFF0000u))));
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(v.lo[i])), fabsf(__uint_as_float(v.hi[i]))));
        }
        return mx;
    };
    // pass 1: the row's largest |x|
    Raw keep[kBatch];
    float mx = 0.0f;
    for (int c0 = 0; c0 < kch; c0 += 256 * kBatch) {
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            const int c = c0 + b * 256 + tid;
            if (c < kch) keep[b] = load_x8_raw<XDT>(x, xoff + (int64_t)c * 8);
        }
#pragma unroll
        for (int b = 0; b < kBatch; b++)
            if (c0 + b * 256 + tid < kch) mx = absmax(keep[b], mx);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((tid & 63) == 0) wave_max[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    int e = 0;
    if (mx > 0.0f && mx <= 3.4028234663852886e38f) {
        e = 14 - (__builtin_amdgcn_frexp_expf(mx) - 1);        // 14 - floor(log2(mx))
        if (e >= 0 && e <= 16) e = 0;                           // largest in [2^-2, 2^15): as it is
        e = e < kXexpMin ? kXexpMin : (e > kXexpMax ? kXexpMax : e);
    }
    // pass 2: binary16 of x * 2^e into the image (a row of one batch is still
    // in registers; longer rows are read again)
    const int r = m & (kImgRows - 1);
    const int64_t tile0 = (int64_t)(m / kImgRows) * ksteps;
    const bool one_batch = kch <= 256 * kBatch;
    for (int c0 = 0; c0 < nch; c0 += 256 * kBatch) {
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            const int c = c0 + b * 256 + tid;
            if (c >= nch) break;
            u32x4_t o = {0u, 0u, 0u, 0u};
            if (c < kch) {
                const Raw v = one_batch ? keep[b] : load_x8_raw<XDT>(x, xoff + (int64_t)c * 8);
                float f[8];
                if constexpr (XDT == DT_BF16) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        f[2 * i] = __uint_as_float(v.lo[i] << 16);
                        f[2 * i + 1] = __uint_as_float(v.lo[i] & 0xFFFF0000u);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        f[i] = __uint_as_float(v.lo[i]);
                        f[4 + i] = __uint_as_float(v.hi[i]);
                    }
                }
                // position p of the chunk holds k = perm[p]
                // (Q4_0, affine 4-bit, affine 8-bit: element order)
                constexpr int kPerm[3][8] = {{0, 2, 1, 3, 4, 6, 5, 7}, {0, 4, 1, 5, 2, 6, 3, 7}, {0, 1, 2, 3, 4, 5, 6, 7}};
                constexpr int kP = WF == WF_Q4_0 ? 0 : WF == WF_AFFINE4 ? 1 : 2;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int p0 = kPerm[kP][2 * i];
                    const int p1 = kPerm[kP][2 * i + 1];
                    o[i] = f32_to_f16(ldexpf(f[p0], e)) | (f32_to_f16(ldexpf(f[p1], e)) << 16);
                }
            }
            const int64_t t = (tile0 + (c >> 3)) * (kImgTile / 8) + r * 8 + ((c & 7) ^ img_swz(r));
            *reinterpret_cast<u32x4_t*>(img + t * 8) = o;
        }
    }
    if (tid == 0) xexp[xexp_pos(m)] = (int8_t)e;
}

template <int WF, int XDT>
__global__ __launch_bounds__(256) void k_pack_x(const void* __restrict__ x, uint16_t* __restrict__ img,
                                                int8_t* __restrict__ xexp, int M, int K, int ksteps) {
    __shared__ float wave_max[4];
    pack_x_body<WF, XDT>(blockIdx.x, wave_max, x, img, xexp, M, K, ksteps);
}


// planar weights -> image, one workgroup per (256-column tile, 4 K steps).
// Loads go row by row (8 lanes read a row's 128 contiguous bytes of nibble
// blocks) into an LDS tile swizzled by row; stores go plane by plane (each
// thread writes one column's 16-byte block), so both sides are coalesced.
// Workgroup blk of the packer; lq: 32 KiB of LDS, [column][8 blocks], block
// slot b ^ (column & 7).
template <int WF>
__device__ __forceinline__ void pack_w_body(int blk, u32x4_t* lq, const uint8_t* __restrict__ wq,
                                            const uint16_t* __restrict__ wsc, const uint16_t* __restrict__ wbias,
                                            uint8_t* __restrict__ img, int N, int K, int ksteps) {
    const int tid = threadIdx.x;
    const int kq = (ksteps + 3) / 4;
    const int grp = blk % kq;
    const int nt = blk / kq;
    const int nb = K / 32;
    // nibble blocks 8*grp .. 8*grp+7 of the tile's columns
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int u = tid + 256 * i;
        const int row = u >> 3, b8 = u & 7;
        const int n = nt * 256 + row;
        const int b = grp * 8 + b8;
        u32x4_t q = {0u, 0u, 0u, 0u};
        if (n < N && b < nb) {
            if constexpr (WF == WF_Q4_0) q = *reinterpret_cast<const u32x4_t*>(wq + ((int64_t)n * nb + b) * 16);
            else q = *reinterpret_cast<const u32x4_t*>(wq + (int64_t)n * (K / 2) + (int64_t)b * 16);
        }
        lq[row * 8 + (b8 ^ (row & 7))] = q;
    }
    // this thread's column's scales (Q4_0: 8 blocks; affine: 4 groups), as
    // one vector load when K is a multiple of 256 (the run is then whole and
    // aligned), else one by one
    const int n = nt * 256 + tid;
    uint16_t sc[8] = {0, 0, 0, 0, 0, 0, 0, 0}, bi[4] = {0, 0, 0, 0};
    const bool whole = (K % 256) == 0;
    if constexpr (WF == WF_Q4_0) {
        if (n < N) {
            if (whole) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wsc + (int64_t)n * nb + grp * 8);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    sc[2 * i] = (uint16_t)(v[i] & 0xFFFFu);
                    sc[2 * i + 1] = (uint16_t)(v[i] >> 16);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++)
                    if (grp * 8 + i < nb) sc[i] = wsc[(int64_t)n * nb + grp * 8 + i];
            }
        }
    } else {
        const int ngr = K / 64;
        if (n < N) {
            if (whole) {
                const u32x2_t vs = *reinterpret_cast<const u32x2_t*>(wsc + (int64_t)n * ngr + grp * 4);
                const u32x2_t vb = *reinterpret_cast<const u32x2_t*>(wbias + (int64_t)n * ngr + grp * 4);
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    sc[2 * i] = (uint16_t)(vs[i] & 0xFFFFu);
                    sc[2 * i + 1] = (uint16_t)(vs[i] >> 16);
                    bi[2 * i] = (uint16_t)(vb[i] & 0xFFFFu);
                    bi[2 * i + 1] = (uint16_t)(vb[i] >> 16);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (grp * 4 + i < ngr) {
                        sc[i] = wsc[(int64_t)n * ngr + grp * 4 + i];
                        bi[i] = wbias[(int64_t)n * ngr + grp * 4 + i];
                    }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const int k = grp * 4 + st;
        if (k >= ksteps) break;
        uint8_t* chunk = img + ((int64_t)nt * ksteps + k) * kWChunk;
#pragma unroll
        for (int blk = 0; blk < 2; blk++) {
            const int b8 = 2 * st + blk;
            *reinterpret_cast<u32x4_t*>(chunk + (blk * 256 + tid) * 16) = lq[tid * 8 + (b8 ^ (tid & 7))];
            if constexpr (WF == WF_Q4_0) reinterpret_cast<uint16_t*>(chunk + 8192)[blk * 256 + tid] = sc[b8];
        }
        if constexpr (WF == WF_AFFINE4) {
            reinterpret_cast<uint16_t*>(chunk + 8192)[tid] = sc[st];
            reinterpret_cast<uint16_t*>(chunk + 8704)[tid] = bi[st];
        }
    }
}

template <int WF>
__global__ __launch_bounds__(256) void k_pack_w(const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsc,
                                                const uint16_t* __restrict__ wbias, uint8_t* __restrict__ img,
                                                int N, int K, int ksteps) {
    __shared__ u32x4_t lq[256 * 8];
    pack_w_body<WF>(blockIdx.x, lq, wq, wsc, wbias, img, N, K, ksteps);
}

// Affine 8-bit codes [N][K] with group-64 scales and biases [N][K/64] ->
// image, one workgroup per (256-column tile, 2 K steps).  Loads go row by
// row (8 lanes read a row's 128 contiguous code bytes, two groups) into an
// LDS tile swizzled by row; stores go plane by plane (each thread writes one
// column's 16 bytes), so both sides are coalesced.  Columns past N get zero
// codes, scales and biases.
// lq: 32 KiB of LDS, [column][8 chunks], chunk slot c ^ (column & 7).
__device__ __forceinline__ void pack_w8_body(int blk, u32x4_t* lq, const uint8_t* __restrict__ wq,
                                             const uint16_t* __restrict__ wsc, const uint16_t* __restrict__ wbias,
                                             uint8_t* __restrict__ img, int N, int K, int ksteps) {
    const int tid = threadIdx.x;
    const int kq = (ksteps + 1) / 2;
    const int grp = blk % kq;
    const int nt = blk / kq;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int u = tid + 256 * i;
        const int row = u >> 3, c = u & 7;     // 16-byte chunk c of the row's 128 bytes
        const int n = nt * 256 + row;
        const int64_t kb = (int64_t)grp * 128 + c * 16;
        u32x4_t q = {0u, 0u, 0u, 0u};
        if (n < N && kb < K) q = *reinterpret_cast<const u32x4_t*>(wq + (int64_t)n * K + kb);
        lq[row * 8 + (c ^ (row & 7))] = q;
    }
    const int n = nt * 256 + tid;
    const int ngr = K / 64;
    uint16_t sc[2] = {0, 0}, bi[2] = {0, 0};
#pragma unroll
    for (int st = 0; st < 2; st++)
        if (n < N && grp * 2 + st < ngr) {
            sc[st] = wsc[(int64_t)n * ngr + grp * 2 + st];
            bi[st] = wbias[(int64_t)n * ngr + grp * 2 + st];
        }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 2; st++) {
        const int k = grp * 2 + st;
        if (k >= ksteps) break;
        uint8_t* chunk = img + ((int64_t)nt * ksteps + k) * kWChunk8;
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const int c = 4 * st + p;          // elements 16p .. 16p+15 of group k
            *reinterpret_cast<u32x4_t*>(chunk + (p * 256 + tid) * 16) = lq[tid * 8 + (c ^ (tid & 7))];
        }
        reinterpret_cast<uint16_t*>(chunk + 16384)[tid] = sc[st];
        reinterpret_cast<uint16_t*>(chunk + 16896)[tid] = bi[st];
    }
}

__global__ __launch_bounds__(256) void k_pack_w8(const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wsc,
                                                 const uint16_t* __restrict__ wbias, uint8_t* __restrict__ img, int N,
                                                 int K, int ksteps) {
    __shared__ u32x4_t lq[256 * 8];
    pack_w8_body(blockIdx.x, lq, wq, wsc, wbias, img, N, K, ksteps);
}

// Workgroups per weight image: 4-bit formats one per (256-column tile, 4 K
// steps), affine 8-bit one per (256-column tile, 2 K steps).
template <int WF>
constexpr int pack_w_steps() { return WF == WF_AFFINE8 ? 2 : 4; }

// Both images of a per-call GEMM in one launch (they are independent HBM
// streams; one launch saves the second launch and its ramp): workgroups
// 0 .. nx-1 pack X rows, the rest the weight image.
template <int WF, int XDT>
__global__ __launch_bounds__(256) void k_pack_xw(int nx, const void* __restrict__ x, uint16_t* __restrict__ ximg,
                                                 int8_t* __restrict__ xexp, int M, const uint8_t* __restrict__ wq,
                                                 const uint16_t* __restrict__ wsc, const uint16_t* __restrict__ wbias,
                                                 uint8_t* __restrict__ wimg, int N, int K, int ksteps) {
    __shared__ u32x4_t lq[256 * 8];
    const int b = blockIdx.x;
    if (b < nx) {
        pack_x_body<WF, XDT>(b, reinterpret_cast<float*>(lq), x, ximg, xexp, M, K, ksteps);
    } else {
        if constexpr (WF == WF_AFFINE8) pack_w8_body(b - nx, lq, wq, wsc, wbias, wimg, N, K, ksteps);
        else pack_w_body<WF>(b - nx, lq, wq, wsc, wbias, wimg, N, K, ksteps);
    }
}

// One ring slot: the X tile (16 KiB) and the weight chunk (9 KiB; affine
// 8-bit 17 KiB) of a step.
template <int WF>
struct PkSlot {
    uint16_t x[kImgTile];
    uint8_t w[w_chunk_bytes<WF>()];
};
template <int WF>
struct PkLds {
    PkSlot<WF> slot[pk_slots<WF>()];
};

template <int WF, int YDT, bool SPLIT>
__global__ __launch_bounds__(256 + 64 * kPkProducers, 1) void k_gemm_pk(const GemmArgs a) {
    static_assert(WF == WF_Q4_0 || WF == WF_AFFINE4 || WF == WF_AFFINE8, "quantised weights only");
    constexpr int MT = 4, NT = 2;
    constexpr int kCols = 4 * NT * 32;
    constexpr int kRows = MT * 32;
    static_assert(kRows == kImgRows && kCols == 256, "tile shape");
    constexpr int kSlots = pk_slots<WF>();
    __shared__ __attribute__((aligned(16))) PkLds<WF> lds;
    using Blk = typename BlkOf<WF>::T;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Persistent: workgroup b runs the work units b, b + G, b + 2G, ...
    // (G = gridDim.x) as one stream of K steps: global step s is step s % ust
    // of the workgroup's unit s / ust.  Unit u is part u % ksplit (K steps
    // p*ust .. p*ust + ust - 1) of tile u / ksplit; tile t covers rows
    // (t % m_tiles) * 128 and columns (t / m_tiles) * 256.  With ksplit > 1
    // each part writes its fp32 tile to the partial buffer, and a second
    // kernel sums the parts in order.
    const int G = gridDim.x;
    const int ksplit = SPLIT ? a.ksplit : 1;        // a compile-time 1 without a split
    const int nunits = a.m_tiles * a.n_tiles * ksplit;
    const int my_units = (nunits - (int)blockIdx.x + G - 1) / G;
    const int nb = a.K / 32;
    const int nsteps = (nb + 1) / 2;                 // K steps of a tile
    const int ust = nsteps / ksplit;                 // of a unit (ksplit divides nsteps)
    const int S = my_units * ust;
    auto unit_of = [&](int i) { return (int)blockIdx.x + i * G; };
    auto tile_m0 = [&](int i) { return unit_of(i) / ksplit % a.m_tiles * kRows; };
    auto tile_n0 = [&](int i) { return unit_of(i) / ksplit / a.m_tiles * kCols; };
    auto part_of = [&](int i) { return unit_of(i) % ksplit; };

    if (wave < 4) {
        // ------------------------------ consumer ------------------------------
        const int j = lane & 31;
        const int g = lane >> 5;
        floatx16_t acc[MT][NT];
#pragma unroll
        for (int mi = 0; mi < MT; mi++)
#pragma unroll
            for (int ni = 0; ni < NT; ni++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[mi][ni][v] = 0.0f;
        u32x4_t bfA[NT][4], bfB[NT][4];
        using Consts = typename DequantConsts<WF>::T;
        const Consts masks = Consts::make();

        // raw weight blocks of step k from its ring slot
        auto read_w = [&](int k, Blk (&r)[NT]) {
            const uint8_t* wb = lds.slot[k % kSlots].w;
#pragma unroll
            for (int ni = 0; ni < NT; ni++) {
                const int cw = wave * NT * 32 + ni * 32 + j;
                if constexpr (WF == WF_AFFINE8) {
                    r[ni].q[0] = *reinterpret_cast<const u32x4_t*>(wb + ((2 * g) * 256 + cw) * 16);
                    r[ni].q[1] = *reinterpret_cast<const u32x4_t*>(wb + ((2 * g + 1) * 256 + cw) * 16);
                    r[ni].s = reinterpret_cast<const uint16_t*>(wb + 16384)[cw];
                    r[ni].b = reinterpret_cast<const uint16_t*>(wb + 16896)[cw];
                } else if constexpr (WF == WF_Q4_0) {
                    r[ni].q = *reinterpret_cast<const u32x4_t*>(wb + (g * 256 + cw) * 16);
                    r[ni].d = reinterpret_cast<const uint16_t*>(wb + 8192)[g * 256 + cw];
                } else {
                    r[ni].q = *reinterpret_cast<const u32x4_t*>(wb + (g * 256 + cw) * 16);
                    r[ni].s = reinterpret_cast<const uint16_t*>(wb + 8192)[cw];
                    r[ni].b = reinterpret_cast<const uint16_t*>(wb + 8704)[cw];
                }
            }
        };
        // blocks past the end of K (K = 32 mod 64) have a zero scale in the
        // weight image (and zero X in the X image)
        auto dequant = [&](int k, Blk (&r)[NT], u32x4_t (&bf)[NT][4]) {
            const bool bok = 2 * k + g < nb;
#pragma unroll
            for (int ni = 0; ni < NT; ni++) {
                zero_blk<WF>(r[ni], bok);
                blk_frags_perm<WF>(r[ni], masks, bf[ni]);
            }
        };
        // X fragment (mi, s) of this lane: row mi*32 + j, chunk 4g + s
        // (kofs = 32g + 8s), swizzled by the row
        int aofs[4];
#pragma unroll
        for (int s = 0; s < 4; s++) aofs[s] = j * 64 + (((4 * g + s) ^ img_swz(j)) * 8);   // rows mi*32 + j
        auto read_a = [&](int k, int s, u32x4_t (&av)[MT]) {
            const uint16_t* la = lds.slot[k % kSlots].x;
#pragma unroll
            for (int mi = 0; mi < MT; mi++)
                av[mi] = *reinterpret_cast<const u32x4_t*>(&la[mi * 32 * 64 + aofs[s]]);
        };
        // MFMA (mi, ni) of K slice s; `first` selects (0, 0), else the others
        auto mfma_slice = [&](int s, const u32x4_t (&av)[MT], const u32x4_t (&bf)[NT][4], bool first) {
#pragma unroll
            for (int mi = 0; mi < MT; mi++)
#pragma unroll
                for (int ni = 0; ni < NT; ni++)
                    if ((mi == 0 && ni == 0) == first)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(half8_t, av[mi]), __builtin_bit_cast(half8_t, bf[ni][s]),
                            acc[mi][ni], 0, 0, 0);
        };
        // Instruction order inside one segment: the first MFMA (its operands
        // were loaded during the previous segment), the segment's LDS reads,
        // then each remaining MFMA followed by up to `valu` vector
        // instructions.  The compiler waits for all outstanding LDS reads at
        // the first MFMA (it does not count LDS returns as ordered here), so
        // the reads issued after it get a whole segment to land.
        auto segment_order = [&](auto nreads, auto valu) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, decltype(nreads)::value, 0);
#pragma unroll
            for (int i = 1; i < MT * NT; i++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, decltype(valu)::value, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        constexpr int kWReads = NT * (WF == WF_Q4_0 ? 2 : WF == WF_AFFINE4 ? 3 : 4);
        // One K step in four segments (K slices s = 0..3) fenced by
        // sched_barrier, so that every LDS read is issued one segment ahead of
        // its use: the slice s+1 X fragments during slice s, the next step's
        // slice 0 during slice 3 (that tile landed one barrier ago), and the
        // raw weights of step k+1 in segment 0.  The dequantisation is spread
        // evenly, two 32-bit words of raw weights (a quarter of a step's) per
        // segment, so that each segment issues about four VALU instructions
        // per MFMA, what one wave hides under its MFMAs:
        //   segment 0: words 2-3 of block 1 of step k (kept in `rb` from the
        //              previous step): this step's slices that come from them
        //              are used in segments 1-3
        //   segment 1: words 0-1 of block 0 of step k+1
        //   segment 2: words 0-1 of block 1 of step k+1
        //   segment 3: words 2-3 of block 0 of step k+1
        // Word w of a block feeds fragments w/2 and 2 + w/2 (Q4_0) or w
        // (affine 4-bit and 8-bit), so every fragment of step k+1 that slice 0
        // needs is complete at the end of step k.  `a0` holds this step's slice
        // 0 on entry and the next step's on return; `rb` holds block 1 of step
        // k on entry and of step k+1 on return.  k is the global step; the next
        // one may start the next tile.  Past the last step the k+1 slots hold
        // older data that is never used.
        auto body = [&](int k, u32x4_t (&cur)[NT][4], u32x4_t (&nxt)[NT][4], u32x4_t (&a0)[MT], Blk& rb) {
            Blk r[NT];
            u32x4_t a1[MT], a2[MT], a3[MT];
            mfma_slice(0, a0, cur, true);
            read_a(k, 1, a1);
            read_w(k + 1, r);
            mfma_slice(0, a0, cur, false);
            {
                const BlkConst cb = blk_const<WF>(rb);
                blk_fragment<WF>(rb, cb, 2, masks, cur[1]);
                blk_fragment<WF>(rb, cb, 3, masks, cur[1]);
            }
            segment_order(std::integral_constant<int, kWReads + MT>{}, std::integral_constant<int, 4>{});

            mfma_slice(1, a1, cur, true);
            read_a(k, 2, a2);
            mfma_slice(1, a1, cur, false);
            const BlkConst c0 = blk_const<WF>(r[0]);
            blk_fragment<WF>(r[0], c0, 0, masks, nxt[0]);
            blk_fragment<WF>(r[0], c0, 1, masks, nxt[0]);
            segment_order(std::integral_constant<int, MT>{}, std::integral_constant<int, 4>{});

            mfma_slice(2, a2, cur, true);
            read_a(k, 3, a3);
            mfma_slice(2, a2, cur, false);
            const BlkConst c1 = blk_const<WF>(r[1]);
            blk_fragment<WF>(r[1], c1, 0, masks, nxt[1]);
            blk_fragment<WF>(r[1], c1, 1, masks, nxt[1]);
            segment_order(std::integral_constant<int, MT>{}, std::integral_constant<int, 4>{});

            mfma_slice(3, a3, cur, true);
            read_a(k + 1, 0, a0);
            mfma_slice(3, a3, cur, false);
            blk_fragment<WF>(r[0], c0, 2, masks, nxt[0]);
            blk_fragment<WF>(r[0], c0, 3, masks, nxt[0]);
            segment_order(std::integral_constant<int, MT>{}, std::integral_constant<int, 4>{});
            // the fragments must be complete here: without this the compiler
            // may sink their dequantisation past the barrier into the next step
#pragma unroll
            for (int ni = 0; ni < NT; ni++)
#pragma unroll
                for (int t = 0; t < 4; t++) asm volatile("" : "+v"(nxt[ni][t]));
            rb = r[1];
        };
        static_assert(NT == 2, "the dequantisation split assumes two blocks per step");

        // Epilogue of local tile i, straight from the accumulators (lane:
        // column j, rows 8*(v/4) + 4*g + v%4).  A DPP swap of neighbouring
        // lanes hands each lane two adjacent columns of one row -- the even
        // lane row r, the odd lane row r+1 -- so every store writes a pair
        // (two bf16 in 4 bytes, or two f32 in 8).  No LDS is involved: the
        // stores drain while the next tile's MFMAs run.  Then the accumulators
        // restart.
        const bool odd = (lane & 1) != 0;
        const bool pair_ok = (a.N & 1) == 0;                  // pair stores stay aligned
        auto swap_pair = [](float v) {
            return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
        };
        // A tile that lies wholly inside Y (with N even) takes a path with no
        // bounds test: every pair store is in bounds and aligned, and each
        // lane's stores advance by fixed multiples of N from one base address.
        auto store_tile = [&](int i, auto whole_c) {
            constexpr bool kWhole = decltype(whole_c)::value;
            const int m0 = tile_m0(i);
            const int nw0 = tile_n0(i) + wave * NT * 32;
#pragma unroll
            for (int mi = 0; mi < MT; mi++) {
                // the row exponents of sub-tile mi: its 32 bytes through the
                // scalar cache (a uniform address), then this lane's 8
                using const_u32 = __attribute__((address_space(4))) const uint32_t;
                const const_u32* sp = (const const_u32*)(a.xexp + m0 + mi * 32);
                uint32_t w[8];
#pragma unroll
                for (int t = 0; t < 8; t++) w[t] = sp[t];
                const int c = 2 * g + (odd ? 1 : 0);
                u32x2_t ex;
                ex[0] = c == 0 ? w[0] : c == 1 ? w[2] : c == 2 ? w[4] : w[6];
                ex[1] = c == 0 ? w[1] : c == 1 ? w[3] : c == 2 ? w[5] : w[7];
                const int r0 = m0 + mi * 32 + 4 * g + (odd ? 1 : 0);
#pragma unroll
                for (int ni = 0; ni < NT; ni++) {
                    const int col = nw0 + ni * 32 + (j & ~1);    // even column of the pair
                    const int64_t base = (int64_t)r0 * a.N + col;
#pragma unroll
                    for (int v = 0; v < 16; v += 2) {
                        const float a0v = acc[mi][ni][v], a1v = acc[mi][ni][v + 1];
                        const float d0 = swap_pair(a0v), d1 = swap_pair(a1v);
                        // row r of the X image was scaled by 2^e(r)
                        const int ue = -xexp_of(ex, v >> 2, (v >> 1) & 1);
                        const float lo = ldexpf(odd ? d1 : a0v, ue);   // column col
                        const float hi = ldexpf(odd ? a1v : d0, ue);   // column col + 1
                        const int dr = 8 * (v >> 2) + (v & 3);
                        const int row = r0 + dr;
                        if (!kWhole && (row >= a.M || col >= a.N)) continue;
                        const int64_t off = base + (int64_t)dr * a.N;
                        const bool pair = kWhole || (pair_ok && col + 1 < a.N);
                        if constexpr (SPLIT) {
                            float* yp = a.part + (int64_t)part_of(i) * a.M * a.N + off;
                            if (pair) {
                                *reinterpret_cast<f32x2_t*>(yp) = f32x2_t{lo, hi};
                            } else {
                                yp[0] = lo;
                                if (col + 1 < a.N) yp[1] = hi;
                            }
                        } else if constexpr (YDT == DT_BF16) {
                            uint16_t* yp = reinterpret_cast<uint16_t*>(a.y) + off;
                            if (pair) {
                                const f32x2_t f = {lo, hi};
                                *reinterpret_cast<uint32_t*>(yp) =
                                    __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
                            } else {
                                yp[0] = (uint16_t)f32_to_bf16(lo);
                                if (col + 1 < a.N) yp[1] = (uint16_t)f32_to_bf16(hi);
                            }
                        } else {
                            float* yp = reinterpret_cast<float*>(a.y) + off;
                            if (pair) {
                                *reinterpret_cast<f32x2_t*>(yp) = f32x2_t{lo, hi};
                            } else {
                                yp[0] = lo;
                                if (col + 1 < a.N) yp[1] = hi;
                            }
                        }
                    }
                }
            }
        };
        auto epilogue = [&](int i) {
            const bool whole = tile_m0(i) + kRows <= a.M && tile_n0(i) + kCols <= a.N && pair_ok;
            if (whole) store_tile(i, std::true_type{});
            else store_tile(i, std::false_type{});
#pragma unroll
            for (int mi = 0; mi < MT; mi++)
#pragma unroll
                for (int ni = 0; ni < NT; ni++)
#pragma unroll
                    for (int v = 0; v < 16; v++) acc[mi][ni][v] = 0.0f;
        };

        step_barrier<63>();                    // prologue: steps 0 and 1 landed
        u32x4_t a0[MT];
        Blk rb;
        {
            Blk r[NT];
            read_w(0, r);
            dequant(0, r, bfA);
            read_a(0, 0, a0);
            rb = r[1];
        }
        // kl: local index of the current step in its unit, ti: local unit
        int kl = 0, ti = 0;
        auto end_step = [&]() {
            if (kl + 1 == ust) {
                epilogue(ti);
                ti++;
                kl = 0;
            } else {
                kl++;
            }
        };
        // no condition inside a step's block of MFMAs: a conditional use of the
        // next step's fragments would let the compiler sink their
        // dequantisation out of the block it is meant to overlap
        int k = 0;
        for (; k + 1 < S; k += 2) {
            body(k, bfA, bfB, a0, rb);
            step_barrier<63>();
            end_step();
            body(k + 1, bfB, bfA, a0, rb);
            step_barrier<63>();
            end_step();
        }
        if (k < S) {
            body(k, bfA, bfB, a0, rb);
            step_barrier<63>();
            end_step();
        }
    } else {
        // ------------------------------ producer ------------------------------
        // kPkProducers waves; per step each copies its share of the X tile
        // (1 KiB copies), of the weight blocks (32 columns x 2 blocks per copy)
        // and of the scales.
        const int pw = wave - 4;
        // per step 25 copies of 1 KiB (16 of X, 9 of weights; affine 8-bit 33:
        // 17 of weights); wave pw takes copies pw, pw + 4, ...
        constexpr int kWBytes = w_chunk_bytes<WF>();
        constexpr int kCopies = 16 + kWBytes / 1024;
        static_assert(kWBytes % 1024 == 0, "whole 1 KiB copies");
        const int my_copies = (kCopies - pw + kPkProducers - 1) / kPkProducers;
        // the next step to request: global index rs = ri * ust + rk
        int rs = 0, ri = 0, rk = 0;
        auto copy_next = [&]() {
            PkSlot<WF>& sl = lds.slot[rs % kSlots];
            const int mt_idx = tile_m0(ri) / kRows;
            const int nt_idx = tile_n0(ri) / kCols;
            const int kg = part_of(ri) * ust + rk;      // K step within the tile
            const uint8_t* xs = reinterpret_cast<const uint8_t*>(a.x) + ((int64_t)mt_idx * nsteps + kg) * (kImgTile * 2);
            const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(a.a) + ((int64_t)nt_idx * nsteps + kg) * kWBytes;
#pragma unroll
            for (int i = 0; i < (kCopies + kPkProducers - 1) / kPkProducers; i++) {
                const int c = pw + kPkProducers * i;
                if (c < 16) dma16(xs + c * 1024 + lane * 16, reinterpret_cast<uint8_t*>(sl.x) + c * 1024);
                else if (c < kCopies) dma16(wsrc + (c - 16) * 1024 + lane * 16, sl.w + (c - 16) * 1024);
            }
            rs++;
            if (++rk == ust) {
                rk = 0;
                ri++;
            }
        };
        // prologue: steps 0 .. kAhead-1 requested, steps 0 and 1 landed.
        // Steps k+3 .. k+kAhead may stay in flight: kAhead - 2 steps of this
        // wave's copies (one step: 7 or 6 copies; affine 8-bit 9 or 8).
        constexpr int kAhead = kSlots - 1;
        constexpr int kMaxC = (kCopies + kPkProducers - 1) / kPkProducers, kMinC = kCopies / kPkProducers;
        static_assert(kAhead >= 3 && (kAhead - 2) * kMaxC < 64, "wait counts below");
        auto wait_step = [&]() {
            if (my_copies == kMaxC) step_barrier<(kAhead - 2) * kMaxC>();
            else step_barrier<(kAhead - 2) * kMinC>();
        };
        for (int i = 0; i < kAhead; i++)
            if (i < S) copy_next();
        if (S >= kAhead) wait_step();
        else step_barrier<0>();
        // during step k: request step k+kAhead, then make sure step k+2 has landed
        for (int k = 0; k < S; k++) {
            if (k + kAhead < S) {
                copy_next();
                wait_step();
            } else {
                step_barrier<0>();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Skinny kernel (small M): weights streamed once at HBM rate.
//
// Workgroup = kSkWaves waves on the same 16*NT columns, splitting K by chunks
// of 4 blocks (the K-splitting of the ET-SoC-1 rewrite) and summing their
// partial tiles through LDS in a fixed order.  MFMA 16x16x32: lane l owns
// column j = l % 16 and lane group g = l / 16, and loads one whole 32-weight
// block -- block 4c+g of chunk c -- with one 128-bit load; in MFMA t
// (t = 0..3) it supplies elements 8t..8t+7 of that block, and the X fragment
// it pairs with is X[i][32 (4c+g) + 8t .. +8].  Every lane scales by its own
// block's d.  Bandwidth comes from memory-level parallelism: every load is
// unconditional (clamped addresses; a block past the end of K gets a zero
// scale, rows past M are computed and dropped), and the next chunk's weights
// and X fragments are in flight while the current chunk is multiplied.
// ---------------------------------------------------------------------------
constexpr int kSkWaves = 8;

struct SkinnyRawQ4 { u32x4_t q; uint32_t d; };
struct SkinnyRawAff { u32x4_t q; uint32_t s, b; };

template <int WF>
struct SkRaw;
template <> struct SkRaw<WF_Q4_0> { SkinnyRawQ4 r; };
template <> struct SkRaw<WF_AFFINE4> { SkinnyRawAff r; };
template <> struct SkRaw<WF_DENSE16> { u32x4_t h[4]; };

// Raw data of block kblk of column n (both valid): one 128-bit load of the
// nibbles (16 for dense binary16) and the scales.
template <int WF>
__device__ __forceinline__ SkRaw<WF> sk_load(const GemmArgs& a, int n, int kblk) {
    SkRaw<WF> r;
    const int nb = a.K / 32;
    if constexpr (WF == WF_Q4_0) {
        r.r.q = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(a.a) + ((int64_t)n * nb + kblk) * 16));
        r.r.d = reinterpret_cast<const uint16_t*>(a.b)[(int64_t)n * nb + kblk];
    } else if constexpr (WF == WF_AFFINE4) {
        r.r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const uint8_t*>(a.a) + (int64_t)n * (a.K / 2) + (int64_t)kblk * 16));
        const int64_t gi = (int64_t)n * (a.K / 64) + (kblk >> 1);
        r.r.s = reinterpret_cast<const uint16_t*>(a.b)[gi];
        r.r.b = reinterpret_cast<const uint16_t*>(a.c)[gi];
    } else {
        const u32x4_t* w = reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const uint16_t*>(a.a) + (int64_t)n * a.K + (int64_t)kblk * 32);
#pragma unroll
        for (int t = 0; t < 4; t++) r.h[t] = __builtin_nontemporal_load(w + t);
    }
    return r;
}

// A block that must not contribute: zero scale (quantised) or zero weights.
template <int WF>
__device__ __forceinline__ void sk_zero(SkRaw<WF>& r, bool keep) {
    if constexpr (WF == WF_Q4_0) {
        r.r.d = keep ? r.r.d : 0u;
    } else if constexpr (WF == WF_AFFINE4) {
        r.r.s = keep ? r.r.s : 0u;
        r.r.b = keep ? r.r.b : 0u;
    } else {
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) r.h[t][e] = keep ? r.h[t][e] : 0u;
    }
}

// Elements 8t..8t+7 of the lane's block as 8 binary16 values, t = 0..3.
template <int WF>
__device__ __forceinline__ void sk_frag(const SkRaw<WF>& r, u32x4_t (&out)[4]) {
    if constexpr (WF == WF_Q4_0) {
        const half2_t dd = as_h2(r.r.d | (r.r.d << 16));
        // t = 0: low nibbles of bytes 0..7, t = 1: low of 8..15,
        // t = 2: high nibbles of bytes 0..7, t = 3: high of 8..15
#pragma unroll
        for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int w = 0; w < 2; w++) {
                const uint32_t word = r.r.q[2 * h + w];
                const uint32_t t01 = perm(word, 0x0C010C00u);
                const uint32_t t23 = perm(word, 0x0C030C02u);
                out[h][2 * w + 0] = q4_pair(t01, dd);
                out[h][2 * w + 1] = q4_pair(t23, dd);
                out[2 + h][2 * w + 0] = q4_pair(t01 >> 4, dd);
                out[2 + h][2 * w + 1] = q4_pair(t23 >> 4, dd);
            }
        }
    } else if constexpr (WF == WF_AFFINE4) {
        // element 8t+v sits in word t: byte v/2, low nibble for even v
        RawAff lo, hi;
        lo.s = hi.s = r.r.s;
        lo.b = hi.b = r.r.b;
        lo.q = u32x2_t{r.r.q[0], r.r.q[1]};
        hi.q = u32x2_t{r.r.q[2], r.r.q[3]};
        const Frag16 f0 = affine_frag(lo);   // s[0] = word 0, s[1] = word 1
        const Frag16 f1 = affine_frag(hi);
        out[0] = f0.s[0];
        out[1] = f0.s[1];
        out[2] = f1.s[0];
        out[3] = f1.s[1];
    } else {
#pragma unroll
        for (int t = 0; t < 4; t++) out[t] = r.h[t];
    }
}

template <int WF, int MT, int NT, int XDT, int YDT>
__global__ __launch_bounds__(64 * kSkWaves) void k_gemm_skinny(const GemmArgs a) {
    __shared__ float red[kSkWaves - 1][MT * 16 * NT * 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * (NT * 16);
    const int nb = a.K / 32;
    const int nchunks = (nb + 3) / 4;

    // clamped columns and rows (never stored when out of range)
    int ncl[NT];
    bool nok[NT];
#pragma unroll
    for (int ni = 0; ni < NT; ni++) {
        const int n = n0 + ni * 16 + j;
        nok[ni] = n < a.N;
        ncl[ni] = nok[ni] ? n : a.N - 1;
    }
    int64_t xrow[MT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++) {
        const int m = mi * 16 + j;
        xrow[mi] = (int64_t)(m < a.M ? m : a.M - 1) * a.K;
    }

    struct Stage {
        SkRaw<WF> w[NT];
        RawX8<XDT> x[MT][4];
        bool kok;
    };
    auto load = [&](int c, Stage& st) {
        const int kblk = c * 4 + g;
        st.kok = kblk < nb;
        const int kb = st.kok ? kblk : nb - 1;
#pragma unroll
        for (int ni = 0; ni < NT; ni++) st.w[ni] = sk_load<WF>(a, ncl[ni], kb);
#pragma unroll
        for (int mi = 0; mi < MT; mi++)
#pragma unroll
            for (int t = 0; t < 4; t++) st.x[mi][t] = load_x8_raw<XDT>(a.x, xrow[mi] + (int64_t)kb * 32 + 8 * t);
    };

    floatx4_t acc[MT][NT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++) acc[mi][ni] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](Stage& st) {
        u32x4_t xa[MT][4];
#pragma unroll
        for (int mi = 0; mi < MT; mi++)
#pragma unroll
            for (int t = 0; t < 4; t++) xa[mi][t] = convert_x8<XDT>(st.x[mi][t]);
#pragma unroll
        for (int ni = 0; ni < NT; ni++) {
            sk_zero<WF>(st.w[ni], st.kok && nok[ni]);
            u32x4_t bfr[4];
            sk_frag<WF>(st.w[ni], bfr);
#pragma unroll
            for (int t = 0; t < 4; t++)
#pragma unroll
                for (int mi = 0; mi < MT; mi++)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(half8_t, xa[mi][t]), __builtin_bit_cast(half8_t, bfr[t]), acc[mi][ni], 0, 0,
                        0);
        }
    };

    if (wave < nchunks) {
        // chunks wave, wave + W, ...: the next one loads while this one
        // multiplies; two stages with fixed roles (no register copies, which
        // would wait for the loads in flight).  A load past the end repeats
        // the last chunk and is never used.
        Stage s0, s1;
        load(wave, s0);
        for (int c = wave;;) {
            const int c1 = c + kSkWaves;
            load(c1 < nchunks ? c1 : c, s1);
            __builtin_amdgcn_sched_barrier(0);     // the next chunk's loads go out before this chunk's math
            compute(s0);
            if (c1 >= nchunks) break;
            const int c2 = c1 + kSkWaves;
            load(c2 < nchunks ? c2 : c1, s0);
            __builtin_amdgcn_sched_barrier(0);
            compute(s1);
            if (c2 >= nchunks) break;
            c = c2;
        }
    }

    // fixed-order reduction over the K-splitting waves: w0 + w1 + ...;
    // lane holds column j, rows 4*g + v of each 16x16 tile
    if (wave > 0) {
#pragma unroll
        for (int mi = 0; mi < MT; mi++)
#pragma unroll
            for (int ni = 0; ni < NT; ni++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    red[wave - 1][((mi * 16 + 4 * g + v) * NT + ni) * 16 + j] = acc[mi][ni][v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int mi = 0; mi < MT; mi++)
#pragma unroll
            for (int ni = 0; ni < NT; ni++) {
                const int n = n0 + ni * 16 + j;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const int r = mi * 16 + 4 * g + v;
                    const int idx = (r * NT + ni) * 16 + j;
                    float t = acc[mi][ni][v];
#pragma unroll
                    for (int w = 0; w < kSkWaves - 1; w++) t += red[w][idx];
                    if (n < a.N && r < a.M) store_y(a.y, YDT, (int64_t)r * a.N + n, t);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel (2 <= M <= 32, bf16 X, Q4_0 or affine): X is used as it is
// and the weights are never rounded.
//
// The bf16 MFMA 16x16x32 takes bf16 X directly and each weight as the exact
// bf16 value 128 + q (the nibble ANDed into the mantissa of 128.0, whose unit
// is 1).  One MFMA covers exactly one 32-weight block of 16 columns, so its
// result is per block and is scaled afterwards in fp32:
//   Q4_0:    y += d * (sum x (128 + q) - 136 sum x)            = d * sum x (q - 8)
//   affine:  y += s * (sum x (128 + q) - 128 sum x) + b * sum x  per group of 64
// The -136 sum x (-128 sum x) term is the MFMA's accumulator input: itself an
// MFMA of X against a constant operand, so it arrives in the output layout
// and serves every column tile.  Products are exact and sums fp32, so the
// result differs from the exact one by fp32 accumulation and the output
// rounding only.
//
// Workgroup: 8 waves on the same NT*16 columns (MT 16-row tiles).  K runs in
// slices of 32/MT blocks; in each slice wave w multiplies blocks 4w/MT ..
// (the waves split K).  A workgroup needs all of X and its columns are
// consecutive rows of the weight planes, so each slice of X, of the weights
// and of the scales is read with whole contiguous wave loads (1 KiB per
// load) and stored to LDS, where every lane reads its MFMA operands: lane
// 16g + j takes dword g of its block of column j (Q4_0: elements 4g..4g+3
// and 16+4g..16+4g+3; affine: 8g..8g+7).  A dword's nibbles pair up as
// (byte 0, byte 2) and (byte 1, byte 3); the X fragment is permuted into the
// same order.  A weight column of a slice takes 4 (mod 64) dwords of LDS, so
// the 64 lanes read distinct banks.  A slice's X, weights and scales are
// loaded together, two slices ahead, into a ring of register stages and
// stored to LDS (double-buffered) the step before they are used: loads
// complete in issue order, so any other split would make the earliest wait
// for everything issued before it.  One barrier per slice.  The partial
// tiles meet in LDS at the end and are summed in wave order, so results are
// deterministic.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int kSmWaves = 8;
constexpr int kSmMaxM = 32;

// Eight weights of dword w as bf16 128 + q, in the pair order (byte 0,
// byte 2), (byte 1, byte 3) of the low nibbles, then of the high nibbles.
__device__ __forceinline__ bf16x8_t sm_weights(uint32_t w, uint32_t mask) {
    const uint32_t magic = 0x43004300u;    // bf16 (128, 128)
    u32x4_t b;
    b[0] = (w & mask) | magic;
    b[1] = ((w >> 8) & mask) | magic;
    b[2] = ((w >> 4) & mask) | magic;
    b[3] = ((w >> 12) & mask) | magic;
    return __builtin_bit_cast(bf16x8_t, b);
}

// X fragment for the weight order above.  Q4_0: lo = x[4g..4g+3],
// hi = x[16+4g..16+4g+3] of the block; affine: x[8g..8g+7].
template <int WF>
struct SmX;
template <> struct SmX<WF_Q4_0> { u32x2_t lo, hi; };
template <> struct SmX<WF_AFFINE4> { u32x4_t v; };

template <int WF>
__device__ __forceinline__ bf16x8_t sm_xfrag(const SmX<WF>& x) {
    u32x4_t r;
    if constexpr (WF == WF_Q4_0) {
        // bytes: (0,2) pairs elements (4g, 4g+2), (1,3) pairs (4g+1, 4g+3)
        r[0] = __builtin_amdgcn_perm(x.lo[1], x.lo[0], 0x05040100u);
        r[1] = __builtin_amdgcn_perm(x.lo[1], x.lo[0], 0x07060302u);
        r[2] = __builtin_amdgcn_perm(x.hi[1], x.hi[0], 0x05040100u);
        r[3] = __builtin_amdgcn_perm(x.hi[1], x.hi[0], 0x07060302u);
    } else {
        // byte i of a dword holds elements 2i (low) and 2i+1 (high): the
        // pairs are (0,4), (2,6), (1,5), (3,7)
        r[0] = __builtin_amdgcn_perm(x.v[2], x.v[0], 0x05040100u);
        r[1] = __builtin_amdgcn_perm(x.v[3], x.v[1], 0x05040100u);
        r[2] = __builtin_amdgcn_perm(x.v[2], x.v[0], 0x07060302u);
        r[3] = __builtin_amdgcn_perm(x.v[3], x.v[1], 0x07060302u);
    }
    return __builtin_bit_cast(bf16x8_t, r);
}

template <int WF, int MT, int NT, int YDT, int XP, bool ONE>
__global__ __launch_bounds__(64 * kSmWaves, 1) void k_gemm_small(const GemmArgs a) {
    static_assert(WF == WF_Q4_0 || WF == WF_AFFINE4, "quantised weights only");
    static_assert(MT == 1 || MT == 2, "one or two row tiles");
    constexpr int kThreads = 64 * kSmWaves;
    constexpr int kRows = MT * 16;
    constexpr int kSliceBlk = 32 / MT;                    // blocks per K slice
    constexpr int kBpw = kSliceBlk / kSmWaves;            // blocks per wave per slice
    constexpr int kRowH = kSliceBlk * 32 + 8;             // X row of a slice, bf16 (16 B pad)
    constexpr int kXBufH = kRows * kRowH;
    constexpr int kUnitsRow = kSliceBlk * 4;              // 16-byte X units per row of a slice
    static_assert(XP * kThreads / kUnitsRow <= kRows, "X rows copied fit the slice buffer");
    constexpr int kCols = NT * 16;
    constexpr int kColB = kSliceBlk * 16 + 16;            // weight column of a slice, bytes
    static_assert(kColB / 4 % 64 == 4, "bank spread of the weight reads");
    constexpr int kWBufB = kCols * kColB;
    constexpr int kWTot = kCols * kSliceBlk;              // 16-byte weight units per slice
    constexpr int kWU = (kWTot + kThreads - 1) / kThreads;
    static_assert(kWTot % 64 == 0, "whole waves per weight pass");
    constexpr int kGs = kSliceBlk / 2;                    // affine groups per slice
    constexpr int kNsc = WF == WF_Q4_0 ? kCols * kSliceBlk : kCols * kGs;   // scales per plane
    static_assert(kNsc % 64 == 0, "whole waves per scale pass");
    constexpr int kSU = (kNsc + kThreads - 1) / kThreads;
    constexpr int kSBufH = (WF == WF_Q4_0 ? 1 : 2) * kNsc;
    constexpr int kTile = MT * NT * 4 * 64;               // partial values per wave
    constexpr int kXBytes = 2 * kXBufH * 2;
    constexpr int kBytes = kXBytes + 2 * kWBufB + 2 * kSBufH * 2;
    constexpr int kRedBytes = kSmWaves * kTile * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kBytes > kRedBytes ? kBytes : kRedBytes];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                   // [2][kRows][kRowH]
    uint8_t* wsm = smem + kXBytes;                                       // [2][kCols][kColB]
    uint16_t* ssm = reinterpret_cast<uint16_t*>(smem + kXBytes + 2 * kWBufB);   // [2][planes][kNsc]
    float* red = reinterpret_cast<float*>(smem);                         // after the last slice

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * kCols;
    const int nb = a.K / 32;
    const int ng = a.K / 64;
    const int nslices = (nb + kSliceBlk - 1) / kSliceBlk;
    const uint16_t* xg = reinterpret_cast<const uint16_t*>(a.x);
    // LDS rows of the A fragments, clamped (rows past M are computed, never stored)
    int xrow[MT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++) xrow[mi] = (mi * 16 + j < a.M ? mi * 16 + j : a.M - 1) * kRowH;

    // ---- one slice: X, weights and scales (a record of the ring) ----
    // X: unit u = tid + 512 i, XP passes over rows 0 .. XP*512/kUnitsRow - 1
    // (>= M); rows past M re-read row M-1 and a unit past K reads another
    // unit of its row (slices past the end re-read the last one), so every
    // load is valid and unconditional; a unit past K is stored as zeros, so
    // blocks past K (and whole slices past the end) contribute nothing
    // whatever their scale.  Weights: unit u is block u % kSliceBlk of column
    // u / kSliceBlk; columns past N re-read column N-1, blocks past K block
    // nb-1.  No select or branch sits next to a load: either makes the
    // compiler wait for every load in flight.
    struct Rec {
        u32x4_t x[XP];
        u32x4_t w[kWU];
        uint16_t s0[kSU];       // Q4_0 d; affine s
        uint16_t s1[kSU];       // affine b
    };
    auto rec_load = [&](int sl, Rec& st) {
        const int slc = sl < nslices ? sl : nslices - 1;
#pragma unroll
        for (int i = 0; i < XP; i++) {
            const int u = tid + i * kThreads;
            const int row = u / kUnitsRow, cu = u % kUnitsRow;
            const int k = slc * kSliceBlk * 32 + cu * 8;
            st.x[i] = *reinterpret_cast<const u32x4_t*>(xg + (int64_t)(row < a.M ? row : a.M - 1) * a.K +
                                                        (k < a.K ? k : k % a.K));
        }
#pragma unroll
        for (int i = 0; i < kWU; i++) {
            const int u = tid + i * kThreads;
            if (kWTot % kThreads == 0 || u < kWTot) {       // whole waves: a uniform condition
                const int c = u / kSliceBlk, b = u % kSliceBlk;
                const int64_t n = n0 + c < a.N ? n0 + c : a.N - 1;
                const int kb = slc * kSliceBlk + b;
                const int kbc = kb < nb ? kb : nb - 1;
                if constexpr (WF == WF_Q4_0)
                    st.w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                        reinterpret_cast<const uint8_t*>(a.a) + (n * nb + kbc) * 16));
                else
                    st.w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                        reinterpret_cast<const uint8_t*>(a.a) + n * (a.K / 2) + (int64_t)kbc * 16));
            }
        }
#pragma unroll
        for (int i = 0; i < kSU; i++) {
            const int u = tid + i * kThreads;
            if (kNsc % kThreads == 0 || u < kNsc) {
                if constexpr (WF == WF_Q4_0) {
                    const int c = u / kSliceBlk, b = u % kSliceBlk;
                    const int64_t n = n0 + c < a.N ? n0 + c : a.N - 1;
                    const int kb = slc * kSliceBlk + b;
                    st.s0[i] = reinterpret_cast<const uint16_t*>(a.b)[n * nb + (kb < nb ? kb : nb - 1)];
                } else {
                    const int c = u / kGs, gr = u % kGs;
                    const int64_t n = n0 + c < a.N ? n0 + c : a.N - 1;
                    const int gi = slc * kGs + gr;
                    const int64_t off = n * ng + (gi < ng ? gi : ng - 1);
                    st.s0[i] = reinterpret_cast<const uint16_t*>(a.b)[off];
                    st.s1[i] = reinterpret_cast<const uint16_t*>(a.c)[off];
                }
            }
        }
    };
    auto rec_store = [&](int sl, const Rec& st) {
        uint16_t* xb = xs + (sl & 1) * kXBufH;
#pragma unroll
        for (int i = 0; i < XP; i++) {
            const int u = tid + i * kThreads;
            const int row = u / kUnitsRow, cu = u % kUnitsRow;
            const int k = sl * kSliceBlk * 32 + cu * 8;
            const u32x4_t v = k < a.K ? st.x[i] : u32x4_t{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4_t*>(xb + row * kRowH + cu * 8) = v;
        }
        uint8_t* wb = wsm + (sl & 1) * kWBufB;
#pragma unroll
        for (int i = 0; i < kWU; i++) {
            const int u = tid + i * kThreads;
            if (kWTot % kThreads == 0 || u < kWTot)
                *reinterpret_cast<u32x4_t*>(wb + (u / kSliceBlk) * kColB + (u % kSliceBlk) * 16) = st.w[i];
        }
        uint16_t* sb = ssm + (sl & 1) * kSBufH;
#pragma unroll
        for (int i = 0; i < kSU; i++) {
            const int u = tid + i * kThreads;
            if (kNsc % kThreads == 0 || u < kNsc) {
                sb[u] = st.s0[i];
                if constexpr (WF == WF_AFFINE4) sb[kNsc + u] = st.s1[i];
            }
        }
    };

    floatx4_t acc[MT][NT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++) acc[mi][ni] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t mask = 0x000F000Fu;
    asm volatile("" : "+v"(mask));           // a VGPR operand: one v_and_or_b32 per pair
    const floatx4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

    // operands of block kBpw*wave + t of slice sl
    auto x_frag = [&](int sl, int t, int mi) {
        const uint16_t* p = xs + (sl & 1) * kXBufH + xrow[mi] + (kBpw * wave + t) * 32;
        SmX<WF> x;
        if constexpr (WF == WF_Q4_0) {
            x.lo = *reinterpret_cast<const u32x2_t*>(p + 4 * g);
            x.hi = *reinterpret_cast<const u32x2_t*>(p + 16 + 4 * g);
        } else {
            x.v = *reinterpret_cast<const u32x4_t*>(p + 8 * g);
        }
        return sm_xfrag<WF>(x);
    };
    auto w_word = [&](int sl, int ni, int t) {
        return *reinterpret_cast<const uint32_t*>(wsm + (sl & 1) * kWBufB + (ni * 16 + j) * kColB +
                                                  (kBpw * wave + t) * 16 + 4 * g);
    };

    auto compute = [&](int sl) {
        const uint16_t* sb = ssm + (sl & 1) * kSBufH;
        if constexpr (WF == WF_Q4_0) {
            const bf16x8_t neg136 = __builtin_bit_cast(bf16x8_t, u32x4_t{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
#pragma unroll
            for (int t = 0; t < kBpw; t++) {
                bf16x8_t xa[MT];
                floatx4_t c0[MT];
#pragma unroll
                for (int mi = 0; mi < MT; mi++) {
                    xa[mi] = x_frag(sl, t, mi);
                    c0[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mi], neg136, zero4, 0, 0, 0);
                }
#pragma unroll
                for (int ni = 0; ni < NT; ni++) {
                    const bf16x8_t wb = sm_weights(w_word(sl, ni, t), mask);
                    const float d = f16_to_f32(sb[(ni * 16 + j) * kSliceBlk + kBpw * wave + t]);
#pragma unroll
                    for (int mi = 0; mi < MT; mi++) {
                        const floatx4_t dv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mi], wb, c0[mi], 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; v++) acc[mi][ni][v] = __builtin_fmaf(d, dv[v], acc[mi][ni][v]);
                    }
                }
            }
        } else {
            const bf16x8_t neg128 = __builtin_bit_cast(bf16x8_t, u32x4_t{0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u});
#pragma unroll
            for (int h = 0; h < kBpw / 2; h++) {       // this wave's groups of 64
                bf16x8_t xa0[MT], xa1[MT];
                floatx4_t cs[MT];                      // -128 * (sum of x over the group)
#pragma unroll
                for (int mi = 0; mi < MT; mi++) {
                    xa0[mi] = x_frag(sl, 2 * h, mi);
                    xa1[mi] = x_frag(sl, 2 * h + 1, mi);
                    cs[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        xa1[mi], neg128, __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa0[mi], neg128, zero4, 0, 0, 0), 0, 0, 0);
                }
#pragma unroll
                for (int ni = 0; ni < NT; ni++) {
                    const int si = (ni * 16 + j) * kGs + (kBpw / 2) * wave + h;
                    const float sv = bf16_to_f32(sb[si]);
                    const float bq = bf16_to_f32(sb[kNsc + si]) * -0.0078125f;   // b / -128 (exact)
                    const bf16x8_t w0 = sm_weights(w_word(sl, ni, 2 * h), mask);
                    const bf16x8_t w1 = sm_weights(w_word(sl, ni, 2 * h + 1), mask);
#pragma unroll
                    for (int mi = 0; mi < MT; mi++) {
                        const floatx4_t dv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            xa1[mi], w1, __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa0[mi], w0, cs[mi], 0, 0, 0), 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; v++) {
                            acc[mi][ni][v] = __builtin_fmaf(sv, dv[v], acc[mi][ni][v]);
                            acc[mi][ni][v] = __builtin_fmaf(bq, cs[mi][v], acc[mi][ni][v]);
                        }
                    }
                }
            }
        }
    };

    // Step sl multiplies slice sl from LDS, stores slice sl+1 from its ring
    // slot into the other LDS buffers and refills the slot with slice
    // sl+1+kRing.  Phases are fenced so that no work on loaded values (and
    // so no wait) moves between them.  The slice count is padded to a
    // multiple of kRing; in the last ring nothing is refilled.  ONE (one or
    // two slices): all of them load at once, so there is no loop; with a
    // loop the ring holds two (four would spill).
    constexpr int kRing = ONE ? 4 : 2;
    const int nsteps = (nslices + kRing - 1) / kRing * kRing;
    Rec ring[kRing];           // slot r holds slices r, r + kRing, ...
    auto step = [&](int sl, auto last, auto r) {
        constexpr bool kLast = decltype(last)::value;
        constexpr int kR = decltype(r)::value;
        constexpr int kNext = (kR + 1) % kRing;
        __builtin_amdgcn_sched_barrier(0);
        compute(sl);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!kLast || kR < kRing - 1) rec_store(sl + 1, ring[kNext]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!kLast) rec_load(sl + 1 + kRing, ring[kNext]);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    auto group = [&](int sl0, auto last) {
        step(sl0 + 0, last, std::integral_constant<int, 0>{});
        step(sl0 + 1, last, std::integral_constant<int, 1>{});
        if constexpr (kRing == 4) {
            step(sl0 + 2, last, std::integral_constant<int, 2>{});
            step(sl0 + 3, last, std::integral_constant<int, 3>{});
        }
    };
#pragma unroll
    for (int r = 0; r < kRing; r++) rec_load(r, ring[r]);
    rec_store(0, ring[0]);
    if constexpr (!ONE) rec_load(kRing, ring[0]);
    __syncthreads();
    if constexpr (ONE) {
        group(0, std::true_type{});
    } else {
        // the first ring is peeled: straight from the prologue its wait
        // counts would otherwise be merged with the loop's
        group(0, std::false_type{});
        for (int sl = kRing; sl < nsteps - kRing; sl += kRing) group(sl, std::false_type{});
        group(nsteps - kRing, std::true_type{});
    }

    // partial tiles to LDS (free after the last barrier); every thread then
    // sums some outputs over the waves in order (lane holds column j, rows
    // 4g + v of each 16x16 tile)
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
#pragma unroll
            for (int v = 0; v < 4; v++) red[wave * kTile + ((mi * NT + ni) * 4 + v) * 64 + lane] = acc[mi][ni][v];
    __syncthreads();
    for (int i = tid; i < kTile; i += kThreads) {
        float t = red[i];
#pragma unroll
        for (int w = 1; w < kSmWaves; w++) t += red[w * kTile + i];
        const int l = i & 63;
        const int v = (i >> 6) & 3;
        const int tile = i >> 8;                  // mi * NT + ni
        const int mi = tile / NT, ni = tile % NT;
        const int r = mi * 16 + 4 * (l >> 4) + v;
        const int n = n0 + ni * 16 + (l & 15);
        if (r < a.M && n < a.N) store_y(a.y, YDT, (int64_t)r * a.N + n, t);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int WF, int MT, int NT, int XDT, int YDT>
static void launch_mfma_t(GemmArgs ga, hipStream_t s) {
    ga.m_tiles = (ga.M + MT * 32 - 1) / (MT * 32);
    ga.n_tiles = (ga.N + 4 * NT * 32 - 1) / (4 * NT * 32);
    const dim3 grid((unsigned)(ga.m_tiles * ga.n_tiles)), block(256);
    hipLaunchKernelGGL((k_gemm_mfma<WF, MT, NT, XDT, YDT>), grid, block, 0, s, ga);
}

template <int WF, int XDT, int YDT>
static void launch_mfma_m(GemmArgs ga, hipStream_t s) {
    // fewer rows per tile at moderate M keeps the grid above the CU count
    if (ga.M <= 32) launch_mfma_t<WF, 1, 2, XDT, YDT>(ga, s);
    else if (ga.M <= 1024) launch_mfma_t<WF, 2, 2, XDT, YDT>(ga, s);
    else launch_mfma_t<WF, 4, 2, XDT, YDT>(ga, s);
}

template <int WF>
static void launch_mfma_w(GemmArgs ga, int xdt, int ydt, hipStream_t s) {
    if (xdt == DT_BF16) {
        if (ydt == DT_BF16) launch_mfma_m<WF, DT_BF16, DT_BF16>(ga, s);
        else launch_mfma_m<WF, DT_BF16, DT_F32>(ga, s);
    } else {
        if (ydt == DT_BF16) launch_mfma_m<WF, DT_F32, DT_BF16>(ga, s);
        else launch_mfma_m<WF, DT_F32, DT_F32>(ga, s);
    }
}

hipError_t launch_gemm_mfma(int wfmt, const void* a, const void* b, const void* c, const void* x, int xdt, void* y,
                            int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    GemmArgs ga{};
    ga.a = a; ga.b = b; ga.c = c; ga.x = x; ga.y = y;
    ga.M = (int)M; ga.N = (int)N; ga.K = (int)K;
    if (wfmt == WF_Q4_0) launch_mfma_w<WF_Q4_0>(ga, xdt, ydt, s);
    else if (wfmt == WF_AFFINE4) launch_mfma_w<WF_AFFINE4>(ga, xdt, ydt, s);
    else launch_mfma_w<WF_DENSE16>(ga, xdt, ydt, s);
    return hipGetLastError();
}

// The binary16 tiles, then one exponent byte per image row.
static int64_t x_tiles_bytes(int64_t M, int64_t K) {
    return (M + kImgRows - 1) / kImgRows * ((K + 63) / 64) * (int64_t)kImgTile * 2;
}

int64_t x_image_bytes(int64_t M, int64_t K) {
    return x_tiles_bytes(M, K) + (M + kImgRows - 1) / kImgRows * kImgRows;
}

const int8_t* x_image_exponents(const void* ximg, int64_t M, int64_t K) {
    return static_cast<const int8_t*>(ximg) + x_tiles_bytes(M, K);
}

int64_t weight_image_bytes(int64_t N, int64_t K) { return (N + 255) / 256 * ((K + 63) / 64) * (int64_t)kWChunk; }

int64_t packed_x_bytes(int64_t M, int64_t N, int64_t K) {
    return x_image_bytes(M, K) + weight_image_bytes(N, K) + splitk_bytes(M, N, K);
}

template <int WF, int XDT>
static void launch_pack_t(const GemmArgs& ga, uint16_t* img, hipStream_t s) {
    const int ksteps = (ga.K + 63) / 64;
    const dim3 grid((unsigned)(ga.m_tiles * kImgRows)), block(256);
    int8_t* xexp = const_cast<int8_t*>(x_image_exponents(img, ga.M, ga.K));
    hipLaunchKernelGGL((k_pack_x<WF, XDT>), grid, block, 0, s, ga.x, img, xexp, ga.M, ga.K, ksteps);
}

template <int WF>
static void launch_pack_w_t(const void* a, const void* b, const void* c, int N, int K, uint8_t* wimg, hipStream_t s) {
    const int n_tiles = (N + 255) / 256;
    const int ksteps = (K + 63) / 64;
    const dim3 grid((unsigned)(n_tiles * ((ksteps + 3) / 4))), block(256);
    hipLaunchKernelGGL((k_pack_w<WF>), grid, block, 0, s, static_cast<const uint8_t*>(a),
                       static_cast<const uint16_t*>(b), static_cast<const uint16_t*>(c), wimg, N, K, ksteps);
}

// The weight planes a per-call GEMM packs into its weight image.
struct WPack {
    const void* a;      // Q4_0 qs / affine codes
    const void* b;      // Q4_0 d / affine scales
    const void* c;      // affine biases
    uint8_t* wimg;
};

// Y = the sum of the ksplit fp32 partial results, in part order; 4 outputs
// per thread.
template <int YDT>
__global__ __launch_bounds__(256) void k_splitk_sum(const float* __restrict__ part, int ksplit, int64_t mn,
                                                     void* __restrict__ y) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= mn) return;
    if (e + 4 <= mn && (mn & 3) == 0) {        // every part's 4 values 16-byte aligned
        floatx4_t t = *reinterpret_cast<const floatx4_t*>(part + e);
        for (int p = 1; p < ksplit; p++) t += *reinterpret_cast<const floatx4_t*>(part + (int64_t)p * mn + e);
        if constexpr (YDT == DT_BF16) {
            const f32x2_t lo = {t[0], t[1]}, hi = {t[2], t[3]};
            const u32x2_t v = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                               __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t))};
            *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(y) + e) = v;
        } else {
            *reinterpret_cast<floatx4_t*>(reinterpret_cast<float*>(y) + e) = t;
        }
    } else {
        const int64_t end = e + 4 < mn ? e + 4 : mn;   // this thread's 4 outputs only
        for (int64_t i = e; i < end; i++) {
            float t = part[i];
            for (int p = 1; p < ksplit; p++) t += part[(int64_t)p * mn + i];
            store_y(y, YDT, i, t);
        }
    }
}

// K parts per tile of k_gemm_pk: split only when fewer than half the CUs
// would get a tile, into the most parts that divide the tile's K steps,
// leave at least 4 of them per part and keep the parts within the CU count.
static int splitk_parts(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + kImgRows - 1) / kImgRows) * ((N + 255) / 256);
    const int64_t nsteps = (K + 63) / 64;
    const int64_t cus = current_cu_count();
    if (tiles * 2 > cus) return 1;
    int best = 1;
    for (int d = 2; d <= 16; d++)
        if (nsteps % d == 0 && nsteps / d >= 4 && tiles * d <= cus) best = d;
    return best;
}

// The split-K partial results after the two images (none where the 256 x
// 256-tile kernel runs: it never splits K).
int64_t splitk_bytes(int64_t M, int64_t N, int64_t K) {
    if (use_big_tiles(M, N, K)) return 0;
    const int d = splitk_parts(M, N, K);
    return d > 1 ? (int64_t)d * M * N * 4 : 0;
}

template <int WF, int XDT>
static void launch_pack_xw_t(const GemmArgs& ga, uint16_t* ximg, const WPack& wp, hipStream_t s) {
    const int ksteps = (ga.K + 63) / 64;
    const int nx = ga.m_tiles * kImgRows;
    const int nw = ga.n_tiles * ((ksteps + pack_w_steps<WF>() - 1) / pack_w_steps<WF>());
    int8_t* xexp = const_cast<int8_t*>(x_image_exponents(ximg, ga.M, ga.K));
    hipLaunchKernelGGL((k_pack_xw<WF, XDT>), dim3((unsigned)(nx + nw)), dim3(256), 0, s, nx, ga.x, ximg, xexp, ga.M,
                       static_cast<const uint8_t*>(wp.a), static_cast<const uint16_t*>(wp.b),
                       static_cast<const uint16_t*>(wp.c), wp.wimg, ga.N, ga.K, ksteps);
}

// X image into ximg, then the GEMM on it and the weight image ga.a; with a
// partial buffer (splitk_bytes(M, N, K) bytes, or nullptr) small tile counts
// are split along K.  With wp the weight image is packed too (into wp->wimg,
// which ga.a points at), in the same launch as the X image.
template <int WF>
static void launch_on_images(GemmArgs ga, int xdt, int ydt, uint16_t* ximg, float* part, hipStream_t s,
                             const WPack* wp = nullptr) {
    ga.m_tiles = (ga.M + kImgRows - 1) / kImgRows;
    ga.n_tiles = (ga.N + 255) / 256;
    if constexpr (WF != WF_AFFINE8) {
        if (use_big_tiles(ga.M, ga.N, ga.K)) {
            // 256 x 256 tiles (at least one per CU): no K split, no partials
            if (wp != nullptr) launch_pack_w_t<WF>(wp->a, wp->b, wp->c, ga.N, ga.K, wp->wimg, s);
            if (xdt == DT_BF16) launch_pack_t<WF, DT_BF16>(ga, ximg, s);
            else launch_pack_t<WF, DT_F32>(ga, ximg, s);
            launch_gemm_big(WF, ga.a, ximg, ga.y, ydt, ga.M, ga.N, ga.K, s);
            return;
        }
    }
    if (wp != nullptr) {
        if (xdt == DT_BF16) launch_pack_xw_t<WF, DT_BF16>(ga, ximg, *wp, s);
        else launch_pack_xw_t<WF, DT_F32>(ga, ximg, *wp, s);
    } else {
        if (xdt == DT_BF16) launch_pack_t<WF, DT_BF16>(ga, ximg, s);
        else launch_pack_t<WF, DT_F32>(ga, ximg, s);
    }
    ga.x = ximg;
    ga.xexp = x_image_exponents(ximg, ga.M, ga.K);
    ga.ksplit = part != nullptr ? splitk_parts(ga.M, ga.N, ga.K) : 1;
    ga.part = part;
    const int cus = current_cu_count();
    const int units = ga.m_tiles * ga.n_tiles * ga.ksplit;
    const dim3 grid((unsigned)(units < cus ? units : cus)), block(256 + 64 * kPkProducers);
    if (ga.ksplit > 1) {
        if (ydt == DT_BF16) hipLaunchKernelGGL((k_gemm_pk<WF, DT_BF16, true>), grid, block, 0, s, ga);
        else hipLaunchKernelGGL((k_gemm_pk<WF, DT_F32, true>), grid, block, 0, s, ga);
    } else {
        if (ydt == DT_BF16) hipLaunchKernelGGL((k_gemm_pk<WF, DT_BF16, false>), grid, block, 0, s, ga);
        else hipLaunchKernelGGL((k_gemm_pk<WF, DT_F32, false>), grid, block, 0, s, ga);
    }
    if (ga.ksplit > 1) {
        const int64_t mn = (int64_t)ga.M * ga.N;
        const dim3 g2((unsigned)((mn / 4 + 1 + 255) / 256)), b2(256);
        if (ydt == DT_BF16) hipLaunchKernelGGL((k_splitk_sum<DT_BF16>), g2, b2, 0, s, part, ga.ksplit, mn, ga.y);
        else hipLaunchKernelGGL((k_splitk_sum<DT_F32>), g2, b2, 0, s, part, ga.ksplit, mn, ga.y);
    }
}

hipError_t launch_pack_weight_image(int wfmt, const void* a, const void* b, const void* c, int64_t N, int64_t K,
                                    void* wimg, hipStream_t s) {
    if (wfmt == WF_Q4_0) {
        launch_pack_w_t<WF_Q4_0>(a, b, c, (int)N, (int)K, static_cast<uint8_t*>(wimg), s);
    } else if (wfmt == WF_AFFINE4) {
        launch_pack_w_t<WF_AFFINE4>(a, b, c, (int)N, (int)K, static_cast<uint8_t*>(wimg), s);
    } else if (wfmt == WF_AFFINE8) {
        if (K % 64 != 0) return hipErrorInvalidValue;
        const int ksteps = (int)(K / 64);
        const int n_tiles = (int)((N + 255) / 256);
        hipLaunchKernelGGL(k_pack_w8, dim3((unsigned)(n_tiles * ((ksteps + 1) / 2))), dim3(256), 0, s,
                           static_cast<const uint8_t*>(a), static_cast<const uint16_t*>(b),
                           static_cast<const uint16_t*>(c), static_cast<uint8_t*>(wimg), (int)N, (int)K, ksteps);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_image(int wfmt, const void* wimg, const void* x, int xdt, void* y, int ydt, int64_t M,
                             int64_t N, int64_t K, void* ximg, float* part, hipStream_t s) {
    GemmArgs ga{};
    ga.a = wimg; ga.x = x; ga.y = y;
    ga.M = (int)M; ga.N = (int)N; ga.K = (int)K;
    if (wfmt == WF_Q4_0) launch_on_images<WF_Q4_0>(ga, xdt, ydt, static_cast<uint16_t*>(ximg), part, s);
    else if (wfmt == WF_AFFINE4) launch_on_images<WF_AFFINE4>(ga, xdt, ydt, static_cast<uint16_t*>(ximg), part, s);
    else if (wfmt == WF_AFFINE8) launch_on_images<WF_AFFINE8>(ga, xdt, ydt, static_cast<uint16_t*>(ximg), part, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// Affine 8-bit on the same kernel: the weight image (17 KiB chunks), then
// the X image (element order) and the GEMM; one workspace as below.
int64_t weight_image8_bytes(int64_t N, int64_t K) { return (N + 255) / 256 * ((K + 63) / 64) * (int64_t)kWChunk8; }

int64_t affine8_packed_bytes(int64_t M, int64_t N, int64_t K) {
    const int d = splitk_parts(M, N, K);
    return x_image_bytes(M, K) + weight_image8_bytes(N, K) + (d > 1 ? (int64_t)d * M * N * 4 : 0);
}

hipError_t launch_affine8_gemm_packed(const uint8_t* wq, const uint16_t* scales, const uint16_t* biases, const void* x,
                                      int xdt, void* y, int ydt, int64_t M, int64_t N, int64_t K, void* img, bool split,
                                      hipStream_t s) {
    uint8_t* wimg = static_cast<uint8_t*>(img) + x_image_bytes(M, K);
    float* part = reinterpret_cast<float*>(wimg + weight_image8_bytes(N, K));
    GemmArgs ga{};
    ga.a = wimg; ga.x = x; ga.y = y;
    ga.M = (int)M; ga.N = (int)N; ga.K = (int)K;
    const WPack wp{wq, scales, biases, wimg};
    launch_on_images<WF_AFFINE8>(ga, xdt, ydt, static_cast<uint16_t*>(img),
                                 split && splitk_parts(M, N, K) > 1 ? part : nullptr, s, &wp);
    return hipGetLastError();
}

// One workspace: the X image, the weight image, then (with `split`) the
// split-K partial results when the tile count calls for them.
hipError_t launch_gemm_packed(int wfmt, const void* a, const void* b, const void* c, const void* x, int xdt, void* y,
                              int ydt, int64_t M, int64_t N, int64_t K, void* img, bool split, hipStream_t s) {
    if (wfmt != WF_Q4_0 && wfmt != WF_AFFINE4) return hipErrorInvalidValue;
    uint8_t* wimg = static_cast<uint8_t*>(img) + x_image_bytes(M, K);
    float* part = split && splitk_bytes(M, N, K) > 0 ? reinterpret_cast<float*>(wimg + weight_image_bytes(N, K))
                                                     : nullptr;
    GemmArgs ga{};
    ga.a = wimg; ga.x = x; ga.y = y;
    ga.M = (int)M; ga.N = (int)N; ga.K = (int)K;
    const WPack wp{a, b, c, wimg};
    if (wfmt == WF_Q4_0) launch_on_images<WF_Q4_0>(ga, xdt, ydt, static_cast<uint16_t*>(img), part, s, &wp);
    else launch_on_images<WF_AFFINE4>(ga, xdt, ydt, static_cast<uint16_t*>(img), part, s, &wp);
    return hipGetLastError();
}

template <int WF, int MT, int NT, int XDT, int YDT>
static void launch_skinny_t(GemmArgs ga, hipStream_t s) {
    const dim3 grid((unsigned)((ga.N + NT * 16 - 1) / (NT * 16))), block(64 * kSkWaves);
    hipLaunchKernelGGL((k_gemm_skinny<WF, MT, NT, XDT, YDT>), grid, block, 0, s, ga);
}

template <int WF, int XDT, int YDT>
static void launch_skinny_m(GemmArgs ga, hipStream_t s) {
    if (ga.M <= 16) launch_skinny_t<WF, 1, 2, XDT, YDT>(ga, s);
    else if (ga.M <= 32) launch_skinny_t<WF, 2, 2, XDT, YDT>(ga, s);
    else launch_skinny_t<WF, 4, 1, XDT, YDT>(ga, s);
}

template <int WF>
static void launch_skinny_w(GemmArgs ga, int xdt, int ydt, hipStream_t s) {
    if (xdt == DT_BF16) {
        if (ydt == DT_BF16) launch_skinny_m<WF, DT_BF16, DT_BF16>(ga, s);
        else launch_skinny_m<WF, DT_BF16, DT_F32>(ga, s);
    } else {
        if (ydt == DT_BF16) launch_skinny_m<WF, DT_F32, DT_BF16>(ga, s);
        else launch_skinny_m<WF, DT_F32, DT_F32>(ga, s);
    }
}

// ---------------------------------------------------------------------------
// Vector kernel for M == 1 on bf16 / f32 activations (the MFMA skinny kernel
// is faster from M = 2 on).
//
// The layout of the decode GEMV: lane l of wave w owns 32-weight block
// column 8w + (l & 7) (and every 8*NW-th after it) and RI rows r0 + (l >> 3)
// + 8i; one 128-bit load brings a row's block.  The dots run two products at a
// time in fp32 (v_dot2_f32_bf16 on bf16 X, v_dot2_f32_f16 on f32 X rounded to
// binary16): each nibble pair becomes the 16-bit pair (B+q, B+q') with one
// AND-OR against the exponent of B (bf16 128 or binary16 1024, where a
// nibble's unit is 1), exact, so a block row's sum of (B+q)*x minus B times
// the column's sum of x gives sum q*x (exact products, fp32 sums).  Q4_0 then
// takes (q-8)*d per block, affine s*sum q*x + b*sum x per group.  The X pairs
// are permuted once per column to match the nibble pairs and serve all RI
// rows.  Partial sums meet in a fixed order (an 8-lane butterfly, then waves
// in order through LDS), so results are deterministic.
// ---------------------------------------------------------------------------
template <int XDT>
struct VecDot {
    // magic exponent and value: bf16 128.0 / binary16 1024.0
    static constexpr uint32_t kMagic = XDT == DT_BF16 ? 0x43004300u : 0x64006400u;
    static constexpr float kBase = XDT == DT_BF16 ? 128.0f : 1024.0f;
    static constexpr uint32_t kOne = XDT == DT_BF16 ? 0x3F803F80u : 0x3C003C00u;   // (1, 1)
    __device__ static float dot(uint32_t a, uint32_t b, float c) {
        if constexpr (XDT == DT_BF16)
            return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                                   false);
        else
            return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
    }
};

constexpr int kVecMaxWaves = 16;

// M == 1 on bf16 X keeps to 64 VGPRs (8 waves per SIMD, 2 workgroups per
// CU); larger M and f32 X take 512-thread workgroups and more registers.
template <int WF, int M, int RI, int XDT, int YDT>
__global__ __launch_bounds__(M == 1 ? 1024 : 512) __attribute__((amdgpu_waves_per_eu(M == 1 && XDT == DT_BF16 ? 8 : 1)))
void k_gemv_x(const GemmArgs a) {
    static_assert(WF == WF_Q4_0 || WF == WF_AFFINE4, "quantised weights only");
    using D = VecDot<XDT == DT_BF16 ? DT_BF16 : DT_F16>;
    __shared__ float red[kVecMaxWaves][8 * RI * M];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int bl = w * 8 + (lane & 7);
    const int rl = lane >> 3;
    const int stride = nw * 8;
    const int nb = a.K / 32;
    const int r0 = blockIdx.x * 8 * RI;

    // rows past N read row 0 (valid memory) and are never written
    const uint8_t* rq[RI];
    const uint16_t* rs[RI];
    const uint16_t* rb[RI];
#pragma unroll
    for (int i = 0; i < RI; i++) {
        const int R = r0 + rl + 8 * i;
        const int n = R < a.N ? R : 0;
        rq[i] = static_cast<const uint8_t*>(a.a) + (int64_t)n * nb * 16;
        if constexpr (WF == WF_Q4_0) {
            rs[i] = static_cast<const uint16_t*>(a.b) + (int64_t)n * nb;
            rb[i] = nullptr;
        } else {
            rs[i] = static_cast<const uint16_t*>(a.b) + (int64_t)n * (nb / 2);
            rb[i] = static_cast<const uint16_t*>(a.c) + (int64_t)n * (nb / 2);
        }
    }
    float acc[RI][M];
#pragma unroll
    for (int i = 0; i < RI; i++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[i][m] = 0.0f;

    for (int c = bl; c < nb; c += stride) {
        // X of column c, as 16 words of two 16-bit values (elements 2j, 2j+1)
        uint32_t xw[M][16];
#pragma unroll
        for (int m = 0; m < M; m++) {
            if constexpr (XDT == DT_BF16) {
                const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(
                    static_cast<const uint16_t*>(a.x) + (int64_t)m * a.K + (int64_t)c * 32);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const u32x4_t v = xp[q];
#pragma unroll
                    for (int t = 0; t < 4; t++) xw[m][4 * q + t] = v[t];
                }
            } else {
                const float4* xp = reinterpret_cast<const float4*>(
                    static_cast<const float*>(a.x) + (int64_t)m * a.K + (int64_t)c * 32);
#pragma unroll
                for (int q = 0; q < 8; q++) {
                    const float4 v = xp[q];
                    xw[m][2 * q] = f32_to_f16(v.x) | (f32_to_f16(v.y) << 16);
                    xw[m][2 * q + 1] = f32_to_f16(v.z) | (f32_to_f16(v.w) << 16);
                }
            }
        }
        u32x4_t wq[RI];
        uint32_t sc[RI], bi[RI];
#pragma unroll
        for (int i = 0; i < RI; i++) {
            wq[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(rq[i] + (int64_t)c * 16));
            if constexpr (WF == WF_Q4_0) {
                sc[i] = rs[i][c];
                bi[i] = 0;
            } else {
                sc[i] = rs[i][c >> 1];
                bi[i] = rb[i][c >> 1];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // X pairs in the order of the nibble pairs of word t: slots 0-3 =
        // low nibbles of bytes (0, 2), of bytes (1, 3), high nibbles of bytes
        // (0, 2), of bytes (1, 3)
        auto lo2 = [](uint32_t p, uint32_t q) { return (p & 0xFFFFu) | (q << 16); };
        auto hi2 = [](uint32_t p, uint32_t q) { return (p >> 16) | (q & 0xFFFF0000u); };
        uint32_t xp[M][16];
        float sx[M];
#pragma unroll
        for (int m = 0; m < M; m++) {
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if constexpr (WF == WF_Q4_0) {      // byte b: elements b and b + 16
                    xp[m][4 * t + 0] = lo2(xw[m][2 * t], xw[m][2 * t + 1]);
                    xp[m][4 * t + 1] = hi2(xw[m][2 * t], xw[m][2 * t + 1]);
                    xp[m][4 * t + 2] = lo2(xw[m][8 + 2 * t], xw[m][9 + 2 * t]);
                    xp[m][4 * t + 3] = hi2(xw[m][8 + 2 * t], xw[m][9 + 2 * t]);
                } else {                             // byte b: elements 2b and 2b + 1
                    xp[m][4 * t + 0] = lo2(xw[m][4 * t], xw[m][4 * t + 2]);
                    xp[m][4 * t + 1] = lo2(xw[m][4 * t + 1], xw[m][4 * t + 3]);
                    xp[m][4 * t + 2] = hi2(xw[m][4 * t], xw[m][4 * t + 2]);
                    xp[m][4 * t + 3] = hi2(xw[m][4 * t + 1], xw[m][4 * t + 3]);
                }
            }
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; j++) s = D::dot(xw[m][j], D::kOne, s);
            sx[m] = s;
        }
        const float off = D::kBase + (WF == WF_Q4_0 ? 8.0f : 0.0f);
#pragma unroll
        for (int i = 0; i < RI; i++) {
            uint32_t wp[16];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t v = wq[i][t];
                wp[4 * t + 0] = (v & 0x000F000Fu) | D::kMagic;
                wp[4 * t + 1] = ((v >> 8) & 0x000F000Fu) | D::kMagic;
                wp[4 * t + 2] = ((v >> 4) & 0x000F000Fu) | D::kMagic;
                wp[4 * t + 3] = ((v >> 12) & 0x000F000Fu) | D::kMagic;
            }
            float scale, bias;
            if constexpr (WF == WF_Q4_0) {
                scale = f16_to_f32(sc[i]);
                bias = 0.0f;
            } else {
                scale = bf16_to_f32(sc[i]);
                bias = bf16_to_f32(bi[i]);
            }
#pragma unroll
            for (int m = 0; m < M; m++) {
                float d = 0.0f;
#pragma unroll
                for (int j = 0; j < 16; j++) d = D::dot(wp[j], xp[m][j], d);
                const float t = fmaf(-off, sx[m], d);          // sum of (q - 8) x, or q x
                acc[i][m] = fmaf(scale, t, acc[i][m]);
                if constexpr (WF == WF_AFFINE4) acc[i][m] = fmaf(bias, sx[m], acc[i][m]);
            }
        }
    }

    auto sum8 = [](float v) {
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
        return v;
    };
#pragma unroll
    for (int i = 0; i < RI; i++)
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float v = sum8(acc[i][m]);
            if ((lane & 7) == 0) red[w][(i * 8 + rl) * M + m] = v;
        }
    __syncthreads();
    for (int t = threadIdx.x; t < 8 * RI * M; t += blockDim.x) {
        const int m = t % M;
        const int slot = t / M;
        const int R = r0 + (slot & 7) + 8 * (slot >> 3);
        if (R >= a.N) continue;
        float v = red[0][t];
        for (int ww = 1; ww < nw; ww++) v += red[ww][t];
        const int64_t off = (int64_t)m * a.N + R;
        if constexpr (YDT == DT_BF16) reinterpret_cast<uint16_t*>(a.y)[off] = (uint16_t)f32_to_bf16(v);
        else reinterpret_cast<float*>(a.y)[off] = v;
    }
}

template <int WF, int M, int XDT, int YDT>
static void launch_vec_m(const GemmArgs& ga, hipStream_t s) {
    const int nb = ga.K / 32;
    const int maxw = M == 1 ? kVecMaxWaves : kVecMaxWaves / 2;
    const int nw = nb < 8 ? 1 : ((nb + 7) / 8 > maxw ? maxw : (nb + 7) / 8);
    // rows per lane: enough workgroups for 32 resident waves per CU at most
    const int64_t slots = (int64_t)current_cu_count() * 32 / nw;
    int64_t ri = (ga.N + 8 * slots - 1) / (8 * slots);
    const int cap = M == 1 && XDT == DT_BF16 ? 2 : 1;
    ri = ri < 1 ? 1 : (ri > cap ? cap : ri);
    const dim3 block(nw * 64);
    const dim3 grid((unsigned)((ga.N + 8 * ri - 1) / (8 * ri)));
    if constexpr (M == 1 && XDT == DT_BF16) {
        if (ri == 2) { hipLaunchKernelGGL((k_gemv_x<WF, M, 2, XDT, YDT>), grid, block, 0, s, ga); return; }
    }
    hipLaunchKernelGGL((k_gemv_x<WF, M, 1, XDT, YDT>), grid, block, 0, s, ga);
}

template <int WF, int XDT, int YDT>
static void launch_vec_t(const GemmArgs& ga, hipStream_t s) {
    switch (ga.M) {
        case 1: launch_vec_m<WF, 1, XDT, YDT>(ga, s); break;
        case 2: launch_vec_m<WF, 2, XDT, YDT>(ga, s); break;
        case 3: launch_vec_m<WF, 3, XDT, YDT>(ga, s); break;
        default: launch_vec_m<WF, 4, XDT, YDT>(ga, s); break;
    }
}

template <int WF>
static void launch_vec_w(const GemmArgs& ga, int xdt, int ydt, hipStream_t s) {
    if (xdt == DT_BF16) {
        if (ydt == DT_BF16) launch_vec_t<WF, DT_BF16, DT_BF16>(ga, s);
        else launch_vec_t<WF, DT_BF16, DT_F32>(ga, s);
    } else {
        if (ydt == DT_BF16) launch_vec_t<WF, DT_F32, DT_BF16>(ga, s);
        else launch_vec_t<WF, DT_F32, DT_F32>(ga, s);
    }
}

template <int WF, int MT, int NT, int YDT, int XP>
static void launch_small_t(GemmArgs ga, hipStream_t s) {
    const dim3 grid((unsigned)((ga.N + NT * 16 - 1) / (NT * 16))), block(64 * kSmWaves);
    const int slice_blk = 32 / MT;
    const int nslices = (ga.K / 32 + slice_blk - 1) / slice_blk;
    // everything at once only for one or two slices: with more requested
    // together, HBM returns all of a workgroup's slices late and together,
    // and no arithmetic overlaps the loads (two slices in flight keep HBM
    // busy: 4-6% faster at K = 4096, M = 2..16)
    if (nslices <= 2) hipLaunchKernelGGL((k_gemm_small<WF, MT, NT, YDT, XP, true>), grid, block, 0, s, ga);
    else hipLaunchKernelGGL((k_gemm_small<WF, MT, NT, YDT, XP, false>), grid, block, 0, s, ga);
}

// The widest column group (NT tiles of 16) that still gives every CU a
// workgroup; NT = 1 when none does.
template <int WF, int MT, int YDT, int XP>
static void launch_small_n(GemmArgs ga, hipStream_t s) {
    const int64_t cus = current_cu_count();
    if ((ga.N + 47) / 48 >= cus) launch_small_t<WF, MT, 3, YDT, XP>(ga, s);
    else if ((ga.N + 31) / 32 >= cus) launch_small_t<WF, MT, 2, YDT, XP>(ga, s);
    else launch_small_t<WF, MT, 1, YDT, XP>(ga, s);
}

// Rows: one 16-row tile up to M = 16 (X copy passes of 4 rows), two up to
// 32 (passes of 8 rows).
template <int WF, int YDT>
static void launch_small_m(GemmArgs ga, hipStream_t s) {
    if (ga.M <= 4) launch_small_n<WF, 1, YDT, 1>(ga, s);
    else if (ga.M <= 8) launch_small_n<WF, 1, YDT, 2>(ga, s);
    else if (ga.M <= 16) launch_small_n<WF, 1, YDT, 4>(ga, s);
    else launch_small_n<WF, 2, YDT, 4>(ga, s);
}

template <int WF>
static void launch_small_w(GemmArgs ga, int ydt, hipStream_t s) {
    if (ydt == DT_BF16) launch_small_m<WF, DT_BF16>(ga, s);
    else launch_small_m<WF, DT_F32>(ga, s);
}

constexpr int kSmChunkMaxM = 128;   // most rows the skinny path takes as row chunks
constexpr int kVecMaxM = 1;   // the skinny path's vector kernel serves M == 1 (the small-M kernel beyond)

hipError_t launch_gemm_skinny(int wfmt, const void* a, const void* b, const void* c, const void* x, int xdt, void* y,
                              int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const bool chunks = xdt == DT_BF16 && M > kSmMaxM && (wfmt == WF_Q4_0 || wfmt == WF_AFFINE4);
    if (M > (chunks ? kSmChunkMaxM : 64)) return hipErrorInvalidValue;
    GemmArgs ga{};
    ga.a = a; ga.b = b; ga.c = c; ga.x = x; ga.y = y;
    ga.M = (int)M; ga.N = (int)N; ga.K = (int)K;
    const bool small = xdt == DT_BF16 && M > kVecMaxM && M <= kSmMaxM;
    if (chunks) {
        // more rows than the small-M kernel takes: row chunks of at most
        // kSmMaxM, each run as a call of that many rows would run (a last
        // single row on the vector kernel) and each streaming the weights
        // again (up to 64 rows that beats the matrix-core GEMM with its
        // per-call images)
        const int ysz = ydt == DT_BF16 ? 2 : 4;
        for (int64_t r = 0; r < M; r += kSmMaxM) {
            GemmArgs gc = ga;
            gc.M = (int)(M - r < kSmMaxM ? M - r : kSmMaxM);
            gc.x = static_cast<const uint16_t*>(x) + r * K;
            gc.y = static_cast<uint8_t*>(y) + r * N * ysz;
            if (gc.M <= kVecMaxM) {
                if (wfmt == WF_Q4_0) launch_vec_w<WF_Q4_0>(gc, xdt, ydt, s);
                else launch_vec_w<WF_AFFINE4>(gc, xdt, ydt, s);
            } else {
                if (wfmt == WF_Q4_0) launch_small_w<WF_Q4_0>(gc, ydt, s);
                else launch_small_w<WF_AFFINE4>(gc, ydt, s);
            }
        }
        return hipGetLastError();
    }
    if (M <= kVecMaxM && wfmt == WF_Q4_0) launch_vec_w<WF_Q4_0>(ga, xdt, ydt, s);
    else if (M <= kVecMaxM && wfmt == WF_AFFINE4) launch_vec_w<WF_AFFINE4>(ga, xdt, ydt, s);
    else if (small && wfmt == WF_Q4_0) launch_small_w<WF_Q4_0>(ga, ydt, s);
    else if (small && wfmt == WF_AFFINE4) launch_small_w<WF_AFFINE4>(ga, ydt, s);
    else if (wfmt == WF_Q4_0) launch_skinny_w<WF_Q4_0>(ga, xdt, ydt, s);
    else if (wfmt == WF_AFFINE4) launch_skinny_w<WF_AFFINE4>(ga, xdt, ydt, s);
    else launch_skinny_w<WF_DENSE16>(ga, xdt, ydt, s);
    return hipGetLastError();
}

}  // namespace q4
