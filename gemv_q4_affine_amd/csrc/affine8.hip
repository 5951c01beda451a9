// affine8.hip -- affine 8-bit group-64 weights on gfx950: quantiser,
// dequantiser and the fused small-M GEMV.
//
// Format (MLX quantize / quantized_matmul with bits=8, group_size=64: MLX
// issue #4621 "quantized_matmul takes 14-41% longer than dequantize + bf16
// matmul at prefill sizes", Repro, which runs bits 4 and 8): w_q u8 [N][K],
// byte k of a row is element k; scales and biases bf16 [N][K/64];
// w ~ q*s + b.  The quantisation rule is the min/max reading used for 4 bits
// with 255 steps.
//
// Large M goes through the dequantiser and the dense binary16 GEMM (the
// dispatch in capi.cpp): the page finds dequantise-then-matmul ahead at
// prefill sizes for both bit widths.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace q4 {

// ---------------------------------------------------------------------------
// Quantiser: one thread per group of 64 weights.
// ---------------------------------------------------------------------------
template <int WDT>
__global__ __launch_bounds__(256) void k_affine8_quantize(const void* __restrict__ w, int64_t ngroups,
                                                          uint8_t* __restrict__ wq, uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ biases) {
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < ngroups;
         g += (int64_t)gridDim.x * blockDim.x) {
        float v[64];
        if constexpr (WDT == DT_F32) {
            const float4* p = reinterpret_cast<const float4*>(w) + g * 16;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const float4 t = p[i];
                // binary32 weights are first rounded to bfloat16
                v[4 * i] = bf16_to_f32(f32_to_bf16(t.x));
                v[4 * i + 1] = bf16_to_f32(f32_to_bf16(t.y));
                v[4 * i + 2] = bf16_to_f32(f32_to_bf16(t.z));
                v[4 * i + 3] = bf16_to_f32(f32_to_bf16(t.w));
            }
        } else {
            const u32x4_t* p = reinterpret_cast<const u32x4_t*>(w) + g * 8;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const u32x4_t t = p[i];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    v[8 * i + 2 * j] = bf16_to_f32(t[j] & 0xFFFFu);
                    v[8 * i + 2 * j + 1] = bf16_to_f32(t[j] >> 16);
                }
            }
        }
        float lo = v[0], hi = v[0];
#pragma unroll
        for (int j = 1; j < 64; j++) {
            lo = fminf(lo, v[j]);
            hi = fmaxf(hi, v[j]);
        }
        lo = lo + 0.0f;  // a zero extreme is taken as +0
        hi = hi + 0.0f;
        const uint32_t sb = f32_to_bf16((hi - lo) / 255.0f);
        const uint32_t bb = f32_to_bf16(lo);
        const float s = bf16_to_f32(sb), b = bf16_to_f32(bb);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(wq + g * 64);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            u32x4_t o;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                uint32_t word = 0;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    uint32_t c = 0;
                    if (s != 0.0f) {
                        const float f = fminf(fmaxf(floorf((v[16 * i + 4 * j + e] - b) / s + 0.5f), 0.0f), 255.0f);
                        c = (uint32_t)f;
                    }
                    word |= c << (8 * e);
                }
                o[j] = word;
            }
            dst[i] = o;
        }
        scales[g] = (uint16_t)sb;
        biases[g] = (uint16_t)bb;
    }
}

// ---------------------------------------------------------------------------
// Dequantiser: 8 consecutive outputs per thread, a wave's stores contiguous.
// The binary32 value nearest q*s + b (one fma), then RNE into the output type.
// ---------------------------------------------------------------------------
template <int ODT>
__global__ __launch_bounds__(256) void k_affine8_dequantize(const uint8_t* __restrict__ wq,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ biases, int64_t nparts,
                                                            void* __restrict__ out) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nparts;
         t += (int64_t)gridDim.x * blockDim.x) {
        const u32x2_t c = *reinterpret_cast<const u32x2_t*>(wq + t * 8);
        const int64_t g = t >> 3;                       // 8 parts of 8 per group of 64
        const float s = bf16_to_f32(scales[g]);
        const float b = bf16_to_f32(biases[g]);
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = fmaf((float)((c[i >> 2] >> (8 * (i & 3))) & 0xFFu), s, b);
        if constexpr (ODT == DT_F32) {
            float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + t * 8);
            o[0] = make_float4(v[0], v[1], v[2], v[3]);
            o[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            u32x4_t o;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t lo = ODT == DT_F16 ? f32_to_f16_rne(v[2 * j]) : f32_to_bf16(v[2 * j]);
                const uint32_t hi = ODT == DT_F16 ? f32_to_f16_rne(v[2 * j + 1]) : f32_to_bf16(v[2 * j + 1]);
                o[j] = lo | (hi << 16);
            }
            *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + t * 8) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// Fused GEMV for 1 <= M <= 16 (decode and small batches).  A workgroup of 4 waves owns 8 rows;
// lane (r = l >> 3, c = l & 7) of wave w takes row r and the 16 bytes
// 128 t + 16 c .. +15 of chunks t = w, w + 4, ... (one 128-bit load, 8 rows x
// 128 contiguous bytes per instruction), U chunks in flight at a time.  Each
// weight is dequantised once in binary32 (q*s + b, one fma) and multiplied
// with the M activation rows (v_dot2_f32_bf16 on code pairs, with s and b
// applied per group, measured slower).  The 8 column lanes of a row meet in
// an XOR butterfly, the 4 waves' partials are added in wave order: the
// summation order depends on K only.
// ---------------------------------------------------------------------------
template <int XDT>
using x16_raw_t = std::conditional_t<XDT == DT_F32, float4[4], u32x4_t[2]>;

template <int XDT>
__device__ __forceinline__ void load_x16_raw(const void* x, int64_t e0, x16_raw_t<XDT>& r) {
    if constexpr (XDT == DT_F32) {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + e0);
#pragma unroll
        for (int i = 0; i < 4; i++) r[i] = p[i];
    } else {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(x) + e0);
        r[0] = p[0];
        r[1] = p[1];
    }
}

template <int XDT>
__device__ __forceinline__ float x16_at(const x16_raw_t<XDT>& r, int e) {
    if constexpr (XDT == DT_F32) {
        const float4 t = r[e >> 2];
        return (e & 3) == 0 ? t.x : (e & 3) == 1 ? t.y : (e & 3) == 2 ? t.z : t.w;
    } else {
        const uint32_t word = r[e >> 3][(e >> 1) & 3];
        return (e & 1) ? __uint_as_float(word & 0xFFFF0000u) : __uint_as_float(word << 16);
    }
}

// U chunks per iteration, all loads issued before any arithmetic.
template <int M>
constexpr int kGemv8U = M == 1 ? 4 : (M <= 4 ? 2 : 1);

// M is the row capacity; the launch has mrows <= M activation rows (rows past
// mrows repeat the last one and are not stored).
template <int M, int XDT, int YDT>
__global__ __launch_bounds__(256) void k_affine8_gemv(const uint8_t* __restrict__ wq, const uint16_t* __restrict__ sc,
                                                      const uint16_t* __restrict__ bi, const void* __restrict__ x,
                                                      void* __restrict__ y, int N, int K, int mrows) {
    constexpr int U = kGemv8U<M>;
    __shared__ float red[4][8][M];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int c = lane & 7;
    const int r = lane >> 3;
    const int row = (int)blockIdx.x * 8 + r;
    const int rr = row < N ? row : N - 1;                // rows past N read the last row, never stored
    const uint8_t* wrow = wq + (int64_t)rr * K;
    const int ng = K / 64;
    const uint16_t* srow = sc + (int64_t)rr * ng;
    const uint16_t* brow = bi + (int64_t)rr * ng;
    const int nchunks = (K + 127) / 128;
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.0f;
    for (int t0 = w; t0 < nchunks; t0 += 4 * U) {
        u32x4_t qv[U];
        uint32_t sv[U], bv[U];
        bool okv[U];
        x16_raw_t<XDT> xr[U][M];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int k0 = (t0 + 4 * u) * 128 + c * 16;
            okv[u] = k0 < K;                             // K % 64 == 0: 16 bytes wholly in or out
            const int kk = okv[u] ? k0 : 0;
            qv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wrow + kk));
            sv[u] = srow[kk >> 6];
            bv[u] = brow[kk >> 6];
#pragma unroll
            for (int m = 0; m < M; m++) load_x16_raw<XDT>(x, (int64_t)(m < mrows ? m : mrows - 1) * K + kk, xr[u][m]);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float s = okv[u] ? bf16_to_f32(sv[u]) : 0.0f;
            const float b = okv[u] ? bf16_to_f32(bv[u]) : 0.0f;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const float wv = fmaf((float)((qv[u][e >> 2] >> (8 * (e & 3))) & 0xFFu), s, b);
#pragma unroll
                for (int m = 0; m < M; m++) acc[m] = fmaf(wv, x16_at<XDT>(xr[u][m], e), acc[m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        float v = acc[m];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        if (c == 0) red[w][r][m] = v;
    }
    __syncthreads();
    if (threadIdx.x < 8 * M) {
        const int r2 = threadIdx.x / M, m = threadIdx.x % M;
        const int row2 = (int)blockIdx.x * 8 + r2;
        if (row2 < N && m < mrows) {
            const float v = ((red[0][r2][m] + red[1][r2][m]) + red[2][r2][m]) + red[3][r2][m];
            if constexpr (YDT == DT_BF16) reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + row2] = (uint16_t)f32_to_bf16(v);
            else reinterpret_cast<float*>(y)[(int64_t)m * N + row2] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel for 4 < M <= 32 on a bfloat16 activation.  Codes 0..255
// are exact in bfloat16, so v_mfma_f32_16x16x32_bf16 takes X and the raw codes
// and sums q*x exactly per product; per group g of column n the result is
// scaled in binary32: y += s[n,g] * sum_k q x + b[n,g] * sum_k x (the second
// sum an MFMA of X against ones, so it arrives in the output layout).
// A workgroup of kA8MmaWaves waves owns NT tiles of 16 weight rows (output
// columns); every wave multiplies its X fragments with all NT tiles (the sum
// of X once for all of them); the waves split the groups and add their
// tiles through LDS in wave order.  MFMA operand
// layout: lane l = 16 h + j supplies row j of X (column j of W) and the 8
// K slots 8h..8h+7; it holds the outputs of rows 4h..4h+3 of column j.  Lane
// (h, j) loads bytes 16h..16h+15 of the group for weight row j (16 rows x 64
// contiguous bytes per instruction); MFMA 0 takes its bytes 0..7, MFMA 1 its
// bytes 8..15, and the X fragments are loaded in the same K order.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 8 codes (two words) as 8 exact bfloat16 values
__device__ __forceinline__ bf16x8_t codes_bf16(uint32_t w0, uint32_t w1) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const uint32_t w = i == 0 ? w0 : w1;
        const f32x2_t lo = {(float)(w & 0xFFu), (float)((w >> 8) & 0xFFu)};
        const f32x2_t hi = {(float)((w >> 16) & 0xFFu), (float)(w >> 24)};
        r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t));
        r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t));
    }
    return __builtin_bit_cast(bf16x8_t, r);
}

constexpr int kA8MmaGroupsInFlight = 2;
constexpr int kA8MmaWaves = 4;          // waves per workgroup, splitting the groups

template <int MT, int NT, int YDT>
__global__ __launch_bounds__(64 * kA8MmaWaves) void k_affine8_mma(const uint8_t* __restrict__ wq, const uint16_t* __restrict__ sc,
                                                     const uint16_t* __restrict__ bi, const uint16_t* __restrict__ x,
                                                     void* __restrict__ y, int M, int N, int K) {
    constexpr int U = kA8MmaGroupsInFlight;
    __shared__ floatx4_t red[kA8MmaWaves][MT][NT][64];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j = lane & 15;
    const int h = lane >> 4;
    const int n0 = (int)blockIdx.x * 16 * NT;
    const int ng = K / 64;
    const uint8_t* wrow[NT];
    const uint16_t* srow[NT];
    const uint16_t* brow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const int nr = min(n0 + nt * 16 + j, N - 1);    // columns past N read the last row, never stored
        wrow[nt] = wq + (int64_t)nr * K;
        srow[nt] = sc + (int64_t)nr * ng;
        brow[nt] = bi + (int64_t)nr * ng;
    }
    const uint16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) xrow[mt] = x + (int64_t)min(mt * 16 + j, M - 1) * K;   // rows past M repeat
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    const floatx4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    floatx4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) acc[mt][nt] = zero4;
    for (int g0 = w * U; g0 < ng; g0 += kA8MmaWaves * U) {
        u32x4_t qv[U][NT], xv[U][MT][2];
        uint32_t sv[U][NT], bv[U][NT];
        bool okv[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int gi = g0 + u;
            okv[u] = gi < ng;
            const int gg = okv[u] ? gi : 0;
            const int k0 = gg * 64 + 16 * h;
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                qv[u][nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wrow[nt] + k0));
                sv[u][nt] = srow[nt][gg];
                bv[u][nt] = brow[nt][gg];
            }
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xrow[mt] + k0);
                xv[u][mt][0] = xp[0];
                xv[u][mt][1] = xp[1];
            }
        }
        __builtin_amdgcn_sched_barrier(0);              // every load of the step issued before any arithmetic
#pragma unroll
        for (int u = 0; u < U; u++) {
            floatx4_t sx[MT];
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, xv[u][mt][0]);
                const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, xv[u][mt][1]);
                sx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ones, zero4, 0, 0, 0);
                sx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ones, sx[mt], 0, 0, 0);
            }
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                const bf16x8_t b0 = codes_bf16(qv[u][nt][0], qv[u][nt][1]);
                const bf16x8_t b1 = codes_bf16(qv[u][nt][2], qv[u][nt][3]);
                const float s = okv[u] ? bf16_to_f32(sv[u][nt]) : 0.0f;
                const float b = okv[u] ? bf16_to_f32(bv[u][nt]) : 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, xv[u][mt][0]);
                    const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, xv[u][mt][1]);
                    floatx4_t qx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, zero4, 0, 0, 0);
                    qx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, qx, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; v++) acc[mt][nt][v] = fmaf(s, qx[v], fmaf(b, sx[mt][v], acc[mt][nt][v]));
                }
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) red[w][mt][nt][lane] = acc[mt][nt];
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const int n = n0 + nt * 16 + j;
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                floatx4_t t = red[0][mt][nt][lane];
#pragma unroll
                for (int ww = 1; ww < kA8MmaWaves; ww++) t += red[ww][mt][nt][lane];
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const int m = mt * 16 + 4 * h + v;
                    if (n < N && m < M) {
                        if constexpr (YDT == DT_BF16) reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16(t[v]);
                        else reinterpret_cast<float*>(y)[(int64_t)m * N + n] = t[v];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_for8(int64_t items, int per_block) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g > (1 << 20)) g = 1 << 20;  // grid-stride loops cover the rest
    return (unsigned)(g < 1 ? 1 : g);
}

hipError_t launch_affine8_quantize(const void* w, int wdt, int64_t N, int64_t K, uint8_t* wq, uint16_t* sc,
                                   uint16_t* bi, hipStream_t s) {
    const int64_t ng = N * (K / 64);
    if (wdt == DT_F32)
        hipLaunchKernelGGL(k_affine8_quantize<DT_F32>, dim3(grid_for8(ng, 256)), dim3(256), 0, s, w, ng, wq, sc, bi);
    else
        hipLaunchKernelGGL(k_affine8_quantize<DT_BF16>, dim3(grid_for8(ng, 256)), dim3(256), 0, s, w, ng, wq, sc, bi);
    return hipGetLastError();
}

hipError_t launch_affine8_dequantize(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, int64_t N, int64_t K,
                                     void* out, int odt, hipStream_t s) {
    const int64_t np = N * (K / 8);
    const dim3 g(grid_for8(np, 256)), b(256);
    if (odt == DT_F16) hipLaunchKernelGGL(k_affine8_dequantize<DT_F16>, g, b, 0, s, wq, sc, bi, np, out);
    else if (odt == DT_BF16) hipLaunchKernelGGL(k_affine8_dequantize<DT_BF16>, g, b, 0, s, wq, sc, bi, np, out);
    else hipLaunchKernelGGL(k_affine8_dequantize<DT_F32>, g, b, 0, s, wq, sc, bi, np, out);
    return hipGetLastError();
}

template <int M>
static void launch_gemv8_m(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, const void* x, int xdt, void* y,
                           int ydt, int N, int K, int mrows, hipStream_t s) {
    const dim3 g((unsigned)((N + 7) / 8)), b(256);
    if (xdt == DT_BF16) {
        if (ydt == DT_BF16)
            hipLaunchKernelGGL((k_affine8_gemv<M, DT_BF16, DT_BF16>), g, b, 0, s, wq, sc, bi, x, y, N, K, mrows);
        else hipLaunchKernelGGL((k_affine8_gemv<M, DT_BF16, DT_F32>), g, b, 0, s, wq, sc, bi, x, y, N, K, mrows);
    } else {
        if (ydt == DT_BF16)
            hipLaunchKernelGGL((k_affine8_gemv<M, DT_F32, DT_BF16>), g, b, 0, s, wq, sc, bi, x, y, N, K, mrows);
        else hipLaunchKernelGGL((k_affine8_gemv<M, DT_F32, DT_F32>), g, b, 0, s, wq, sc, bi, x, y, N, K, mrows);
    }
}

// Row capacities 1, 2, 3, 4, 8 and 16; M between them runs on the next one.
hipError_t launch_affine8_gemv(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, const void* x, int xdt,
                               void* y, int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (M < 1 || M > kAffine8GemvMaxM) return hipErrorInvalidValue;
    const int m = (int)M;
    if (m == 1) launch_gemv8_m<1>(wq, sc, bi, x, xdt, y, ydt, (int)N, (int)K, m, s);
    else if (m == 2) launch_gemv8_m<2>(wq, sc, bi, x, xdt, y, ydt, (int)N, (int)K, m, s);
    else if (m == 3) launch_gemv8_m<3>(wq, sc, bi, x, xdt, y, ydt, (int)N, (int)K, m, s);
    else if (m == 4) launch_gemv8_m<4>(wq, sc, bi, x, xdt, y, ydt, (int)N, (int)K, m, s);
    else if (m <= 8) launch_gemv8_m<8>(wq, sc, bi, x, xdt, y, ydt, (int)N, (int)K, m, s);
    else launch_gemv8_m<16>(wq, sc, bi, x, xdt, y, ydt, (int)N, (int)K, m, s);
    return hipGetLastError();
}

// One 16-row tile (M <= 16): a 16-column tile per workgroup (768 workgroups
// at N = 12288).  Two row tiles: four column tiles per wave, so each X
// fragment (and its sum) serves 64 columns: at M = 32 that cuts the X reads,
// four times the weight bytes otherwise, and was 9% faster (38.4 against
// 42.2 us) despite the 4x fewer workgroups, which cost 11% at M = 16.
hipError_t launch_affine8_mma(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, const void* x, void* y,
                              int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    if (M < 1 || M > kAffine8MmaMaxM) return hipErrorInvalidValue;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const dim3 b(64 * kA8MmaWaves);
    if (M <= 16) {
        const dim3 g((unsigned)((N + 15) / 16));
        if (ydt == DT_BF16) hipLaunchKernelGGL((k_affine8_mma<1, 1, DT_BF16>), g, b, 0, s, wq, sc, bi, xb, y, (int)M, (int)N, (int)K);
        else hipLaunchKernelGGL((k_affine8_mma<1, 1, DT_F32>), g, b, 0, s, wq, sc, bi, xb, y, (int)M, (int)N, (int)K);
    } else {
        const dim3 g((unsigned)((N + 63) / 64));
        if (ydt == DT_BF16) hipLaunchKernelGGL((k_affine8_mma<2, 4, DT_BF16>), g, b, 0, s, wq, sc, bi, xb, y, (int)M, (int)N, (int)K);
        else hipLaunchKernelGGL((k_affine8_mma<2, 4, DT_F32>), g, b, 0, s, wq, sc, bi, xb, y, (int)M, (int)N, (int)K);
    }
    return hipGetLastError();
}

}  // namespace q4
