// gemv.hip -- decode GEMV on gfx950: Q4_0 weights x Q8_1 activations.
//
// y[m][n] = sum_b d4[n][b] * d8[m][b] * isum[m][n][b],
// isum = sum_{j<32} (q4_j - 8) * q8_j   (exact int32)
//
// This is the decode route of the pages: one token goes to a vector-dot
// kernel (llama.cpp PR "et-backend: Q4_0 matrix-engine GEMM rewrite for
// prefill", Overview) -- the q4_0 x q8_1 mul_mat_vec_q kernel, with a fused
// variant for two weight matrices that share one activation ("2026-05-06 Q4
// sync-after focused repro", Important source touch points: gate+up, K+V).
//
// Design (HBM-bound: 4.5 bits per weight streamed once, ~3.5 flop/byte):
//  * one wave owns RW consecutive output rows; its 64 lanes split K by
//    32-weight blocks (lane l takes blocks l, l+64, ...), so every weight load
//    is a coalesced 128-bit load of one block's 16 nibble bytes and a wave
//    instruction reads 1 KiB of contiguous nibbles;
//  * nibbles are unpacked in registers: the low nibbles of a 32-bit word are
//    elements i..i+3, the high nibbles elements i+16..i+19 of the block, so
//    (word & 0x0F0F0F0F) and ((word >> 4) & 0x0F0F0F0F) feed v_dot4_i32_i8
//    directly against the matching activation words; the offset 8 is
//    removed once per block as 8 * sum(q8), giving the exact int32 isum;
//  * the int32 sum is scaled by d4*d8 (exact binary32 product of two binary16
//    values) and accumulated with one fma per block in binary32;
//  * each row's 64 lane partials are summed by a fixed butterfly, so the
//    result is deterministic and independent of which matrix or wave the row
//    sits in: the fused two-matrix launch is bit-identical to two launches.
#include "device_common.hpp"
#include "kernels.hpp"

namespace q4 {

struct GemvArgs {
    const uint8_t* qs[2];
    const uint16_t* d[2];
    float* y[2];
    int n[2];          // rows of each matrix
    const int8_t* xqs;
    const uint16_t* xds;
    int K;
    int nb;            // K / 32
    int total_rows;    // n[0] + n[1]
};

__device__ __forceinline__ int block_isum(const u32x4_t w, const int (&a)[8], int neg8sum) {
    const uint32_t lo = 0x0F0F0F0Fu;
    int s = neg8sum;
    s = __builtin_amdgcn_sdot4((int)(w[0] & lo), a[0], s, false);
    s = __builtin_amdgcn_sdot4((int)(w[1] & lo), a[1], s, false);
    s = __builtin_amdgcn_sdot4((int)(w[2] & lo), a[2], s, false);
    s = __builtin_amdgcn_sdot4((int)(w[3] & lo), a[3], s, false);
    s = __builtin_amdgcn_sdot4((int)((w[0] >> 4) & lo), a[4], s, false);
    s = __builtin_amdgcn_sdot4((int)((w[1] >> 4) & lo), a[5], s, false);
    s = __builtin_amdgcn_sdot4((int)((w[2] >> 4) & lo), a[6], s, false);
    s = __builtin_amdgcn_sdot4((int)((w[3] >> 4) & lo), a[7], s, false);
    return s;
}

template <int M, int RW>
__global__ __launch_bounds__(256) void k_q4_gemv(const GemvArgs args) {
    const int lane = threadIdx.x & (kWave - 1);
    const int gw = (int)blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
    const int row0 = gw * RW;
    if (row0 >= args.total_rows) return;  // whole wave idle (uniform branch)

    const int nb = args.nb;
    const u32x4_t* rqs[RW];
    const uint16_t* rd[RW];
    bool rv[RW];
#pragma unroll
    for (int r = 0; r < RW; r++) {
        const int R = row0 + r;
        rv[r] = R < args.total_rows;
        const int mat = (R >= args.n[0]) ? 1 : 0;
        const int rr = rv[r] ? R - (mat ? args.n[0] : 0) : 0;
        rqs[r] = reinterpret_cast<const u32x4_t*>(args.qs[mat] + (int64_t)rr * nb * 16);
        rd[r] = args.d[mat] + (int64_t)rr * nb;
    }

    float acc[RW][M];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[r][m] = 0.0f;

#pragma unroll 2
    for (int c0 = 0; c0 < nb; c0 += kWave) {
        const int b = c0 + lane;
        const bool act = b < nb;
        u32x4_t wv[RW];
        float dv[RW];
#pragma unroll
        for (int r = 0; r < RW; r++) {
            if (act && rv[r]) {
                wv[r] = __builtin_nontemporal_load(rqs[r] + b);
                dv[r] = f16_to_f32(rd[r][b]);
            } else {
                wv[r] = u32x4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                dv[r] = 0.0f;
            }
        }
#pragma unroll
        for (int m = 0; m < M; m++) {
            int a[8];
            float d8 = 0.0f;
            if (act) {
                const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(args.xqs + (int64_t)m * args.K + (int64_t)b * 32);
                const u32x4_t x0 = xp[0], x1 = xp[1];
                a[0] = (int)x0[0]; a[1] = (int)x0[1]; a[2] = (int)x0[2]; a[3] = (int)x0[3];
                a[4] = (int)x1[0]; a[5] = (int)x1[1]; a[6] = (int)x1[2]; a[7] = (int)x1[3];
                d8 = f16_to_f32(args.xds[((int64_t)m * nb + b) * 2]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) a[i] = 0;
            }
            int sq = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) sq = __builtin_amdgcn_sdot4(a[i], 0x01010101, sq, false);
            const int neg8sum = -8 * sq;
#pragma unroll
            for (int r = 0; r < RW; r++) {
                const int isum = block_isum(wv[r], a, neg8sum);
                acc[r][m] = fmaf((float)isum, dv[r] * d8, acc[r][m]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RW; r++) {
        if (!rv[r]) continue;
        const int R = row0 + r;
        const int mat = (R >= args.n[0]) ? 1 : 0;
        const int rr = R - (mat ? args.n[0] : 0);
        float* yp = args.y[mat];
        const int nrows = args.n[mat];
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float t = wave_sum(acc[r][m]);
            if (lane == 0) yp[(int64_t)m * nrows + rr] = t;
        }
    }
}

template <int M>
static void launch_m(const GemvArgs& a, int rw, hipStream_t s) {
    const int waves_per_block = 4;
    const int waves = (a.total_rows + rw - 1) / rw;
    const dim3 grid((waves + waves_per_block - 1) / waves_per_block), block(waves_per_block * kWave);
    if (rw == 4) hipLaunchKernelGGL((k_q4_gemv<M, 4>), grid, block, 0, s, a);
    else if (rw == 2) hipLaunchKernelGGL((k_q4_gemv<M, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_q4_gemv<M, 1>), grid, block, 0, s, a);
}

// Rows per wave: enough waves to fill 256 CUs several times over, fewer
// rows per wave as M (and with it the register footprint) grows.
static int pick_rows_per_wave(int64_t rows, int64_t M) {
    int rw = rows >= 8192 ? 4 : (rows >= 4096 ? 2 : 1);
    if (M > 8) rw = 1;
    else if (M > 4 && rw > 2) rw = 2;
    return rw;
}

hipError_t launch_q4_gemv(const uint8_t* w0_qs, const uint16_t* w0_d, float* y0, int64_t N0,
                          const uint8_t* w1_qs, const uint16_t* w1_d, float* y1, int64_t N1,
                          const int8_t* x_qs, const uint16_t* x_ds, int64_t M, int64_t K, hipStream_t s) {
    GemvArgs a;
    a.qs[0] = w0_qs; a.d[0] = w0_d; a.y[0] = y0; a.n[0] = (int)N0;
    a.qs[1] = w1_qs ? w1_qs : w0_qs; a.d[1] = w1_d ? w1_d : w0_d; a.y[1] = y1 ? y1 : y0; a.n[1] = (int)N1;
    a.xqs = x_qs; a.xds = x_ds; a.K = (int)K; a.nb = (int)(K / 32);
    a.total_rows = (int)(N0 + N1);
    const int rw = pick_rows_per_wave(N0 + N1, M);
    switch (M) {
        case 1: launch_m<1>(a, rw, s); break;
        case 2: launch_m<2>(a, rw, s); break;
        case 3: launch_m<3>(a, rw, s); break;
        case 4: launch_m<4>(a, rw, s); break;
        case 5: launch_m<5>(a, rw, s); break;
        case 6: launch_m<6>(a, rw, s); break;
        case 7: launch_m<7>(a, rw, s); break;
        case 8: launch_m<8>(a, rw, s); break;
        case 9: launch_m<9>(a, rw, s); break;
        case 10: launch_m<10>(a, rw, s); break;
        case 11: launch_m<11>(a, rw, s); break;
        case 12: launch_m<12>(a, rw, s); break;
        case 13: launch_m<13>(a, rw, s); break;
        case 14: launch_m<14>(a, rw, s); break;
        case 15: launch_m<15>(a, rw, s); break;
        case 16: launch_m<16>(a, rw, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace q4
