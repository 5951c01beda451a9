// quant.hip -- quantisers and dequantisers for gfx950.
//
// Q4_0 (GGUF block; the format of llama.cpp PR "et-backend: Q4_0
// matrix-engine GEMM rewrite for prefill", Overview), Q8_1 activations (the
// q4_0 x q8_1 decode kernels of "2026-05-06 Q4 sync-after focused repro",
// Important source touch points) and affine 4-bit group-64 (MLX issue #4621,
// Repro: quantize / dequantize with group_size=64, bits=4).
//
// These kernels are bandwidth-bound and off the per-token hot path except
// q8_1_quantize_act (once per token, latency-bound).  Every code they emit is
// decided in binary32 with separate multiply and add (the library is built
// with -ffp-contract=off), IEEE division and round-to-nearest-even
// conversions, so the planes are bit-exact.
#include "device_common.hpp"
#include "kernels.hpp"

namespace q4 {

// ---------------------------------------------------------------------------
// Q4_0 quantisation: one thread per 32-weight block.
// ---------------------------------------------------------------------------
template <int WDT>
__global__ __launch_bounds__(256) void k_q4_quantize(const void* __restrict__ w, int64_t nblocks,
                                                     uint8_t* __restrict__ qs, uint16_t* __restrict__ d) {
    for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * blockDim.x) {
        float v[32];
        if (WDT == DT_F32) {
            const float4* p = reinterpret_cast<const float4*>(w) + blk * 8;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                float4 t = p[i];
                v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
            }
        } else {
            const u32x4_t* p = reinterpret_cast<const u32x4_t*>(w) + blk * 4;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                u32x4_t t = p[i];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    v[8 * i + 2 * j] = bf16_to_f32(t[j] & 0xFFFFu);
                    v[8 * i + 2 * j + 1] = bf16_to_f32(t[j] >> 16);
                }
            }
        }
        // first element of largest magnitude, with its sign
        float amax = 0.0f, maxv = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; j++) {
            float a = fabsf(v[j]);
            if (a > amax) { amax = a; maxv = v[j]; }
        }
        const float dd = maxv / -8.0f;
        const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
        uint32_t code[32];
#pragma unroll
        for (int j = 0; j < 32; j++) {
            float t = v[j] * id;     // binary32 multiply ...
            float u = t + 8.5f;      // ... then add (not fused)
            int c = (int)u;          // u >= 0.5, so truncation is floor
            code[j] = (uint32_t)(c < 15 ? c : 15);
        }
        u32x4_t out;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                uint32_t byte = code[4 * i + j] | (code[4 * i + j + 16] << 4);
                word |= byte << (8 * j);
            }
            out[i] = word;
        }
        reinterpret_cast<u32x4_t*>(qs)[blk] = out;
        d[blk] = (uint16_t)f32_to_f16_rne(dd);
    }
}

// ---------------------------------------------------------------------------
// Q8_1 quantisation: 8 lanes per 32-element block, 4 elements per lane.
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(256) void k_q8_1_quantize(const void* __restrict__ x, int64_t nblocks,
                                                       int8_t* __restrict__ qs, uint16_t* __restrict__ ds) {
    const int sub = threadIdx.x & 7;  // lane within the block's group of 8
    for (int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3; base < nblocks;
         base += ((int64_t)gridDim.x * blockDim.x) >> 3) {
        const int64_t e0 = base * 32 + sub * 4;
        float v[4];
        load_act4<XDT>(x, e0, v);
        uint32_t d16, s16;
        const uint32_t word = q8_1_block<Q8Adjacent, true>(v, d16, s16);
        *reinterpret_cast<uint32_t*>(qs + e0) = word;
        if (sub == 0) reinterpret_cast<uint32_t*>(ds)[base] = d16 | (s16 << 16);
    }
}

// ---------------------------------------------------------------------------
// Affine 4-bit quantisation: one thread per group of 64 weights.
// ---------------------------------------------------------------------------
template <int WDT>
__global__ __launch_bounds__(256) void k_affine4_quantize(const void* __restrict__ w, int64_t ngroups,
                                                          uint8_t* __restrict__ wq, uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ biases) {
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < ngroups;
         g += (int64_t)gridDim.x * blockDim.x) {
        float v[64];
        if (WDT == DT_F32) {
            const float4* p = reinterpret_cast<const float4*>(w) + g * 16;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                float4 t = p[i];
                // weights are first rounded to bfloat16
                v[4 * i] = bf16_to_f32(f32_to_bf16(t.x));
                v[4 * i + 1] = bf16_to_f32(f32_to_bf16(t.y));
                v[4 * i + 2] = bf16_to_f32(f32_to_bf16(t.z));
                v[4 * i + 3] = bf16_to_f32(f32_to_bf16(t.w));
            }
        } else {
            const u32x4_t* p = reinterpret_cast<const u32x4_t*>(w) + g * 8;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                u32x4_t t = p[i];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    v[8 * i + 2 * j] = bf16_to_f32(t[j] & 0xFFFFu);
                    v[8 * i + 2 * j + 1] = bf16_to_f32(t[j] >> 16);
                }
            }
        }
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int j = 1; j < 64; j++) {
            mn = fminf(mn, v[j]);
            mx = fmaxf(mx, v[j]);
        }
        mn = mn + 0.0f;  // a zero extreme is taken as +0
        mx = mx + 0.0f;
        const float s32 = (mx - mn) / 15.0f;
        const uint32_t sb = f32_to_bf16(s32);
        const uint32_t bb = f32_to_bf16(mn);
        const float s = bf16_to_f32(sb), b = bf16_to_f32(bb);
        u32x4_t out[2];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                uint32_t c = 0;
                if (s != 0.0f) {
                    float r = (v[8 * i + j] - b) / s;
                    float f = floorf(r + 0.5f);
                    f = fminf(fmaxf(f, 0.0f), 15.0f);
                    c = (uint32_t)f;
                }
                word |= c << (4 * j);  // element 2i in the low nibble of byte i
            }
            out[i >> 2][i & 3] = word;
        }
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(wq + g * 32);
        dst[0] = out[0];
        dst[1] = out[1];
        scales[g] = (uint16_t)sb;
        biases[g] = (uint16_t)bb;
    }
}

// ---------------------------------------------------------------------------
// Dequantisers to dense binary16 / bfloat16 / binary32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_out(float v, int odt) {
    return odt == DT_F16 ? f32_to_f16_rne(v) : f32_to_bf16(v);
}

// Each 32-weight block (Q4_0) or half group (affine) is written by 4 lanes,
// 8 consecutive outputs each, so that the lanes of a wave store one
// contiguous run (1 KiB of binary16 per store instruction).
template <int ODT>
__device__ __forceinline__ void store8(void* out, int64_t e0, const float (&v)[8]) {
    if constexpr (ODT == DT_F32) {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e0);
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        u32x4_t t;
#pragma unroll
        for (int j = 0; j < 4; j++) t[j] = pack_out(v[2 * j], ODT) | (pack_out(v[2 * j + 1], ODT) << 16);
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + e0) = t;
    }
}

// Part p of a block holds elements 8p..8p+7: the low nibbles of bytes
// 8(p & 1)..+7 for p < 2, their high nibbles for p >= 2.
template <int ODT>
__global__ __launch_bounds__(256) void k_q4_dequantize(const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d,
                                                       int64_t nparts, void* __restrict__ out) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nparts;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t blk = t >> 2;
        const int p = (int)(t & 3);
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(qs + blk * 16 + 8 * (p & 1));
        const float dd = f16_to_f32(d[blk]);
        const int sh = 4 * (p >> 1);
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t nib = (w[i >> 2] >> (8 * (i & 3) + sh)) & 0xFu;
            v[i] = (float)((int)nib - 8) * dd;        // exact in binary32
        }
        store8<ODT>(out, t * 8, v);
    }
}

// Part p of a 32-weight half group holds elements 8p..8p+7, the nibbles of
// bytes 4p..4p+3 (element 2i in the low nibble of byte i).
template <int ODT>
__global__ __launch_bounds__(256) void k_affine4_dequantize(const uint8_t* __restrict__ wq,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ biases, int64_t nparts,
                                                            int group_shift, void* __restrict__ out) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nparts;
         t += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(wq + t * 4);
        const int64_t g = (t * 8) >> group_shift;
        const float s = bf16_to_f32(scales[g]);
        const float b = bf16_to_f32(biases[g]);
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = fmaf((float)((w >> (4 * i)) & 0xFu), s, b);  // nearest binary32 to q*s + b
        store8<ODT>(out, t * 8, v);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_for(int64_t items, int per_block) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g > (1 << 20)) g = 1 << 20;  // grid-stride loops cover the rest
    return (unsigned)(g < 1 ? 1 : g);
}

hipError_t launch_q4_quantize(const void* w, int wdt, int64_t N, int64_t K, uint8_t* qs, uint16_t* d,
                              hipStream_t s) {
    const int64_t nb = N * (K / 32);
    if (wdt == DT_F32)
        hipLaunchKernelGGL(k_q4_quantize<DT_F32>, dim3(grid_for(nb, 256)), dim3(256), 0, s, w, nb, qs, d);
    else
        hipLaunchKernelGGL(k_q4_quantize<DT_BF16>, dim3(grid_for(nb, 256)), dim3(256), 0, s, w, nb, qs, d);
    return hipGetLastError();
}

hipError_t launch_q8_1_quantize(const void* x, int xdt, int64_t M, int64_t K, int8_t* qs, uint16_t* ds,
                                hipStream_t s) {
    const int64_t nb = M * (K / 32);
    if (xdt == DT_F32)
        hipLaunchKernelGGL(k_q8_1_quantize<DT_F32>, dim3(grid_for(nb * 8, 256)), dim3(256), 0, s, x, nb, qs, ds);
    else
        hipLaunchKernelGGL(k_q8_1_quantize<DT_BF16>, dim3(grid_for(nb * 8, 256)), dim3(256), 0, s, x, nb, qs, ds);
    return hipGetLastError();
}

hipError_t launch_affine4_quantize(const void* w, int wdt, int64_t N, int64_t K, int64_t G, uint8_t* wq,
                                   uint16_t* sc, uint16_t* bi, hipStream_t s) {
    (void)G;  // group size 64 only (validated on the host)
    const int64_t ng = N * (K / 64);
    if (wdt == DT_F32)
        hipLaunchKernelGGL(k_affine4_quantize<DT_F32>, dim3(grid_for(ng, 256)), dim3(256), 0, s, w, ng, wq, sc, bi);
    else
        hipLaunchKernelGGL(k_affine4_quantize<DT_BF16>, dim3(grid_for(ng, 256)), dim3(256), 0, s, w, ng, wq, sc, bi);
    return hipGetLastError();
}

hipError_t launch_q4_dequantize(const uint8_t* qs, const uint16_t* d, int64_t N, int64_t K, void* out, int odt,
                                hipStream_t s) {
    const int64_t np = N * (K / 32) * 4;
    const dim3 g(grid_for(np, 256)), b(256);
    if (odt == DT_F16) hipLaunchKernelGGL(k_q4_dequantize<DT_F16>, g, b, 0, s, qs, d, np, out);
    else if (odt == DT_BF16) hipLaunchKernelGGL(k_q4_dequantize<DT_BF16>, g, b, 0, s, qs, d, np, out);
    else hipLaunchKernelGGL(k_q4_dequantize<DT_F32>, g, b, 0, s, qs, d, np, out);
    return hipGetLastError();
}

hipError_t launch_affine4_dequantize(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, int64_t G,
                                     int64_t N, int64_t K, void* out, int odt, hipStream_t s) {
    const int64_t np = N * (K / 8);
    const int gs = (G == 64) ? 6 : 5;
    const dim3 g(grid_for(np, 256)), b(256);
    if (odt == DT_F16) hipLaunchKernelGGL(k_affine4_dequantize<DT_F16>, g, b, 0, s, wq, sc, bi, np, gs, out);
    else if (odt == DT_BF16) hipLaunchKernelGGL(k_affine4_dequantize<DT_BF16>, g, b, 0, s, wq, sc, bi, np, gs, out);
    else hipLaunchKernelGGL(k_affine4_dequantize<DT_F32>, g, b, 0, s, wq, sc, bi, np, gs, out);
    return hipGetLastError();
}

}  // namespace q4
