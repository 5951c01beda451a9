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
//  * a workgroup of NW waves (NW = min(16, ceil(K/256))) splits K into 8*NW
//    "block lanes": lane l of wave w owns 32-weight block column
//    b = 8w + (l & 7) (and b + 8*NW, ... for longer rows) and row lane
//    l >> 3, so it loads its activation block once (32 int8 + d8) and reuses
//    it for every weight row it visits;
//  * each lane streams RI weight rows (rows r0 + (l >> 3) + 8i): per row one
//    128-bit load of the block's 16 nibble bytes and its binary16 d; the 8
//    lanes of a row read 128 contiguous bytes, whole cache lines.  The
//    (cache-resident) activation is fetched first and the weight rows in
//    order, all before any arithmetic, so the loads are in flight together
//    and row i's arithmetic overlaps the arrival of rows i+1.. (loads return
//    in order);
//  * nibbles are unpacked in registers: the low nibbles of a 32-bit word are
//    elements i..i+3, the high nibbles elements i+16..i+19 of the block, so
//    (word & 0x0F0F0F0F) and ((word >> 4) & 0x0F0F0F0F) feed v_dot4_i32_i8
//    directly against the matching activation words; the offset 8 is
//    removed once per block as 8 * sum(q8), giving the exact int32 isum;
//  * the int32 sum is scaled by d4*d8 (exact binary32 product of two binary16
//    values) and accumulated with one fma per block in binary32;
//  * partial sums meet in a fixed order: an 8-lane butterfly inside the wave,
//    then the NW wave partials added in wave order through LDS.  The order
//    depends on K only, never on the row's position, so the fused
//    two-matrix launch is bit-identical to two single launches.
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

constexpr int kMaxWaves = 16;   // 1024-thread workgroups

// Sum over the 8 lanes of each aligned group of 8, same value on all 8 lanes,
// in a fixed order: swap within pairs, then pairs within quads (DPP
// quad_perm), then the two quads of the group (DPP row_half_mirror).
__device__ __forceinline__ float sum8(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)); // row_half_mirror
    return v;
}

// NMAT: 1 for q4_gemv, 2 for q4_gemv_fused2 (rows past n[0] belong to the
// second matrix).  Per-row arithmetic does not depend on RI or NMAT.
template <int M, int RI, int NMAT>
__global__ __launch_bounds__(1024) void k_q4_gemv(const GemvArgs args) {
    static_assert(RI * M <= 16, "partials per lane");
    __shared__ float red[kMaxWaves][8 * RI * M];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int bl = w * 8 + (lane & 7);          // block lane: first block column
    const int rl = lane >> 3;                   // row lane: 0..7
    const int stride = nw * 8;
    const int nb = args.nb;
    const int r0 = blockIdx.x * 8 * RI;

    // Rows past the end read row 0 of the last matrix (valid memory) and are
    // never written: every load is unconditional.
    const u32x4_t* rqs[RI];
    const uint16_t* rd[RI];
#pragma unroll
    for (int i = 0; i < RI; i++) {
        const int R = r0 + rl + 8 * i;
        const bool second = NMAT == 2 && R >= args.n[0];
        const int rr = (R < args.total_rows) ? R - (second ? args.n[0] : 0) : 0;
        const uint8_t* qbase = second ? args.qs[1] : args.qs[0];
        const uint16_t* dbase = second ? args.d[1] : args.d[0];
        rqs[i] = reinterpret_cast<const u32x4_t*>(qbase + (int64_t)rr * nb * 16);
        rd[i] = dbase + (int64_t)rr * nb;
    }

    float acc[RI][M];
#pragma unroll
    for (int i = 0; i < RI; i++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[i][m] = 0.0f;

    constexpr int MP = M < 4 ? M : 4;   // activation rows fetched ahead of the weights
    for (int b = bl; b < nb; b += stride) {
        // loads: activation (cache-resident) first, then the weight rows in order
        u32x4_t xa[MP][2];
        uint32_t d8r[MP];
#pragma unroll
        for (int m = 0; m < MP; m++) {
            const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(args.xqs + (int64_t)m * args.K + (int64_t)b * 32);
            xa[m][0] = xp[0];
            xa[m][1] = xp[1];
            d8r[m] = args.xds[((int64_t)m * nb + b) * 2];
        }
        u32x4_t wv[RI];
        uint32_t dr[RI];
#pragma unroll
        for (int i = 0; i < RI; i++) {
            dr[i] = rd[i][b];
            wv[i] = __builtin_nontemporal_load(rqs[i] + b);
        }
        __builtin_amdgcn_sched_barrier(0);
        int neg8sum[M];
        int av[M][8];
        float d8[M];
#pragma unroll
        for (int m = 0; m < M; m++) {
            u32x4_t x0, x1;
            uint32_t d8bits;
            if (m < MP) {
                x0 = xa[m < MP ? m : 0][0];
                x1 = xa[m < MP ? m : 0][1];
                d8bits = d8r[m < MP ? m : 0];
            } else {
                const u32x4_t* xp =
                    reinterpret_cast<const u32x4_t*>(args.xqs + (int64_t)m * args.K + (int64_t)b * 32);
                x0 = xp[0];
                x1 = xp[1];
                d8bits = args.xds[((int64_t)m * nb + b) * 2];
            }
            av[m][0] = (int)x0[0]; av[m][1] = (int)x0[1]; av[m][2] = (int)x0[2]; av[m][3] = (int)x0[3];
            av[m][4] = (int)x1[0]; av[m][5] = (int)x1[1]; av[m][6] = (int)x1[2]; av[m][7] = (int)x1[3];
            d8[m] = f16_to_f32(d8bits);
            int sq = 0;
#pragma unroll
            for (int t = 0; t < 8; t++) sq = __builtin_amdgcn_sdot4(av[m][t], 0x01010101, sq, false);
            neg8sum[m] = -8 * sq;
        }
#pragma unroll
        for (int i = 0; i < RI; i++) {
            const float d4 = f16_to_f32(dr[i]);
#pragma unroll
            for (int m = 0; m < M; m++) {
                const int isum = block_isum(wv[i], av[m], neg8sum[m]);
                acc[i][m] = fmaf((float)isum, d4 * d8[m], acc[i][m]);
            }
        }
    }

    // 8 block lanes of a row -> one partial per wave, then wave partials in
    // wave order
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
        const int slot = t / M;                 // i * 8 + rl
        const int R = r0 + (slot & 7) + 8 * (slot >> 3);
        if (R >= args.total_rows) continue;
        float v = red[0][t];
        for (int ww = 1; ww < nw; ww++) v += red[ww][t];
        const bool second = NMAT == 2 && R >= args.n[0];
        float* yp = second ? args.y[1] : args.y[0];
        const int64_t rows = second ? args.n[1] : args.n[0];
        yp[(int64_t)m * rows + (R - (second ? args.n[0] : 0))] = v;
    }
}

template <int M, int NMAT>
static void launch_m(const GemvArgs& a, int ri, int nw, hipStream_t s) {
    const dim3 block(nw * kWave);
    const int rows_per_wg = 8 * ri;
    const dim3 grid((a.total_rows + rows_per_wg - 1) / rows_per_wg);
    if constexpr (M <= 4) {
        if (ri == 4) { hipLaunchKernelGGL((k_q4_gemv<M, 4, NMAT>), grid, block, 0, s, a); return; }
        if (ri == 3) { hipLaunchKernelGGL((k_q4_gemv<M, 3, NMAT>), grid, block, 0, s, a); return; }
    }
    if constexpr (M <= 8) {
        if (ri == 2) { hipLaunchKernelGGL((k_q4_gemv<M, 2, NMAT>), grid, block, 0, s, a); return; }
    }
    hipLaunchKernelGGL((k_q4_gemv<M, 1, NMAT>), grid, block, 0, s, a);
}

template <int M>
static void launch_m(const GemvArgs& a, int ri, int nw, hipStream_t s) {
    if (a.n[1] > 0) launch_m<M, 2>(a, ri, nw, s);
    else launch_m<M, 1>(a, ri, nw, s);
}

// Waves per workgroup: one block lane per 32-weight block of a row, up to 16
// waves.  Rows per lane: enough workgroups to fill the 256 CUs twice, fewer
// rows per lane as M (and with it the register footprint) grows.
static int pick_waves(int64_t nb) {
    int64_t nw = (nb + 7) / 8;
    return (int)(nw < 1 ? 1 : (nw > kMaxWaves ? kMaxWaves : nw));
}

static int pick_rows_per_lane(int64_t rows, int64_t M) {
    int64_t ri = rows / (8 * 512);
    ri = ri < 1 ? 1 : (ri > 4 ? 4 : ri);
    if (M > 8) ri = 1;
    else if (M > 4 && ri > 2) ri = 2;
    return (int)ri;
}

hipError_t launch_q4_gemv(const uint8_t* w0_qs, const uint16_t* w0_d, float* y0, int64_t N0,
                          const uint8_t* w1_qs, const uint16_t* w1_d, float* y1, int64_t N1,
                          const int8_t* x_qs, const uint16_t* x_ds, int64_t M, int64_t K, hipStream_t s) {
    GemvArgs a;
    a.qs[0] = w0_qs; a.d[0] = w0_d; a.y[0] = y0; a.n[0] = (int)N0;
    a.qs[1] = w1_qs ? w1_qs : w0_qs; a.d[1] = w1_d ? w1_d : w0_d; a.y[1] = y1 ? y1 : y0; a.n[1] = (int)N1;
    a.xqs = x_qs; a.xds = x_ds; a.K = (int)K; a.nb = (int)(K / 32);
    a.total_rows = (int)(N0 + N1);
    const int ri = pick_rows_per_lane(N0 + N1, M);
    const int nw = pick_waves(K / 32);
    switch (M) {
#define Q4_GEMV_CASE(m) case m: launch_m<m>(a, ri, nw, s); break;
        Q4_GEMV_CASE(1) Q4_GEMV_CASE(2) Q4_GEMV_CASE(3) Q4_GEMV_CASE(4)
        Q4_GEMV_CASE(5) Q4_GEMV_CASE(6) Q4_GEMV_CASE(7) Q4_GEMV_CASE(8)
        Q4_GEMV_CASE(9) Q4_GEMV_CASE(10) Q4_GEMV_CASE(11) Q4_GEMV_CASE(12)
        Q4_GEMV_CASE(13) Q4_GEMV_CASE(14) Q4_GEMV_CASE(15) Q4_GEMV_CASE(16)
#undef Q4_GEMV_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace q4
