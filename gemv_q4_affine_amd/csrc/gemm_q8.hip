// gemm_q8.hip -- Q4_0 weights x Q8_1 activations on the int8 matrix cores.
//
// The integer-dot form of the Q4_0 x Q8_1 product (the MMVQ kernels of the
// llama.cpp SYCL repro page, Important source touch points; the DP4A / matrix
// engine variant of the trueno page's KERNEL_WEIGHTS table), at any M:
//
//   y[m][n] = sum_b d4[n][b] * d8[m][b] * isum[m][n][b],
//   isum[m][n][b] = sum_{j<32} (q4[n][b][j] - 8) * q8[m][b][j]     (exact int32)
//
// One 32-weight block is exactly the K depth of v_mfma_i32_32x32x32_i8, so
// every MFMA yields the exact integer dots of one block for a 32 x 32 output
// tile; the block's two scales then multiply those 16 sums per lane before
// they join the fp32 accumulators.  That rescale (a convert, a multiply and
// an fma per output and block) is VALU work the binary16 path does not have:
// it sets this kernel's speed, not the matrix cores.
//
// Workgroup: 128 x 128 outputs, 4 waves in 2 x 2, each 64 x 64 (2 x 2 tiles
// of 32 x 32).  Fragments come straight from global memory (16 bytes per lane:
// X codes of one row and block half, or one column's 16 nibble bytes); the
// scales of 16 blocks at a time go through LDS as fp32.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace q4 {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

constexpr int kQ8Tile = 128;     // rows and columns of a workgroup tile
constexpr int kQ8Chunk = 16;     // blocks whose scales are staged together

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

template <int YDT>
__device__ __forceinline__ void store_out(void* y, int64_t off, float v) {
    if constexpr (YDT == DT_F32) reinterpret_cast<float*>(y)[off] = v;
    else reinterpret_cast<uint16_t*>(y)[off] = (uint16_t)f32_to_bf16(v);
}

// The 16 codes q - 8 of one lane's half block, as int8: half 0 holds elements
// 0..15 (low nibbles of the 16 bytes), half 1 elements 16..31 (high nibbles).
// (q + 0x78) ^ 0x80 is q - 8 in two's complement and never carries between
// bytes (q + 0x78 <= 0x87).
__device__ __forceinline__ i32x4_t q4_codes_i8(u32x4_t raw, int half) {
    i32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t t = (half ? (raw[i] >> 4) : raw[i]) & 0x0F0F0F0Fu;
        r[i] = (int)((t + 0x78787878u) ^ 0x80808080u);
    }
    return r;
}

template <int YDT>
__global__ __launch_bounds__(256) void k_gemm_q8(const uint8_t* __restrict__ wqs, const uint16_t* __restrict__ wd,
                                                 const int8_t* __restrict__ xqs, const uint16_t* __restrict__ xds,
                                                 void* __restrict__ y, int M, int N, int K, int m_tiles) {
    __shared__ float sd8[kQ8Chunk][kQ8Tile];   // d8 of the tile's rows, per block of the chunk
    __shared__ float sd4[kQ8Chunk][kQ8Tile];   // d4 of the tile's columns
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, g = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    const int mt = blockIdx.x % m_tiles, nt = blockIdx.x / m_tiles;
    const int tm0 = mt * kQ8Tile, tn0 = nt * kQ8Tile;
    const int nb = K / 32;

    floatx16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; mi++)
#pragma unroll
        for (int ni = 0; ni < 2; ni++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mi][ni][v] = 0.0f;

    // this lane's fragment rows and columns (clamped reads; zero codes past the edge)
    int arow[2], bcol[2];
    bool aok[2], bok[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
        arow[t] = tm0 + wm * 64 + t * 32 + j;
        aok[t] = arow[t] < M;
        bcol[t] = tn0 + wn * 64 + t * 32 + j;
        bok[t] = bcol[t] < N;
    }

    for (int b0 = 0; b0 < nb; b0 += kQ8Chunk) {
        const int nblk = nb - b0 < kQ8Chunk ? nb - b0 : kQ8Chunk;
        __syncthreads();                       // the previous chunk's scales are no longer read
        if (tid < kQ8Tile) {
            const int m = tm0 + tid;
            for (int c = 0; c < kQ8Chunk; c++)
                sd8[c][tid] = (m < M && c < nblk) ? half_bits_to_f32(xds[((int64_t)m * nb + b0 + c) * 2]) : 0.0f;
        } else {
            const int col = tid - kQ8Tile, n = tn0 + col;
            for (int c = 0; c < kQ8Chunk; c++)
                sd4[c][col] = (n < N && c < nblk) ? half_bits_to_f32(wd[(int64_t)n * nb + b0 + c]) : 0.0f;
        }
        __syncthreads();

        for (int c = 0; c < nblk; c++) {
            const int b = b0 + c;
            i32x4_t a[2], w[2];
#pragma unroll
            for (int t = 0; t < 2; t++) {
                a[t] = aok[t] ? *reinterpret_cast<const i32x4_t*>(xqs + (int64_t)arow[t] * K + b * 32 + g * 16)
                              : i32x4_t{0, 0, 0, 0};
                const u32x4_t raw = bok[t] ? *reinterpret_cast<const u32x4_t*>(wqs + ((int64_t)bcol[t] * nb + b) * 16)
                                           : u32x4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                w[t] = q4_codes_i8(raw, g);
            }
            float d4[2];
#pragma unroll
            for (int ni = 0; ni < 2; ni++) d4[ni] = sd4[c][wn * 64 + ni * 32 + j];
#pragma unroll
            for (int mi = 0; mi < 2; mi++) {
                // d8 of this lane's 16 rows: rows 8q + 4g + 0..3 of the 32-row tile
                float d8[16];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const floatx4_t v4 = *reinterpret_cast<const floatx4_t*>(&sd8[c][wm * 64 + mi * 32 + 8 * q + 4 * g]);
#pragma unroll
                    for (int s = 0; s < 4; s++) d8[4 * q + s] = v4[s];
                }
#pragma unroll
                for (int ni = 0; ni < 2; ni++) {
                    const i32x16_t isum = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[mi], w[ni], i32x16_t{}, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 16; v++)
                        acc[mi][ni][v] = __builtin_fmaf((float)isum[v], d8[v] * d4[ni], acc[mi][ni][v]);
                }
            }
        }
    }

    // outputs: lane column j, rows 8 (v / 4) + 4 g + v % 4 of each 32 x 32 tile
#pragma unroll
    for (int mi = 0; mi < 2; mi++)
#pragma unroll
        for (int ni = 0; ni < 2; ni++) {
            const int n = bcol[ni];
            if (n >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int m = tm0 + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                if (m < M) store_out<YDT>(y, (int64_t)m * N + n, acc[mi][ni][v]);
            }
        }
}

}  // namespace

hipError_t launch_gemm_q8(const uint8_t* wqs, const uint16_t* wd, const int8_t* xqs, const uint16_t* xds, void* y,
                          int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s) {
    const int m_tiles = (int)((M + kQ8Tile - 1) / kQ8Tile);
    const int n_tiles = (int)((N + kQ8Tile - 1) / kQ8Tile);
    const dim3 grid((unsigned)(m_tiles * n_tiles)), block(256);
    if (ydt == DT_BF16)
        hipLaunchKernelGGL((k_gemm_q8<DT_BF16>), grid, block, 0, s, wqs, wd, xqs, xds, y, (int)M, (int)N, (int)K, m_tiles);
    else
        hipLaunchKernelGGL((k_gemm_q8<DT_F32>), grid, block, 0, s, wqs, wd, xqs, xds, y, (int)M, (int)N, (int)K, m_tiles);
    return hipGetLastError();
}

}  // namespace q4
