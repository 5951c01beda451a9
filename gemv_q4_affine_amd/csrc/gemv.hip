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
//  * the K/32 block columns of a row are dealt to V = min(16, ceil(K/256))
//    virtual waves of 8 block lanes: virtual lane j = 8v + c owns columns
//    j, j + 8V, j + 16V, ... and sums them in that order.  A workgroup runs
//    V / F physical waves; lane l of wave w plays virtual lanes
//    8(w + f V/F) + (l & 7), f < F, which is to say that it walks columns
//    b = 8w + (l & 7) + k 8V/F and adds column k into accumulator k mod F.
//    Row lane l >> 3 picks the rows.  The sum order thus depends on K only,
//    not on F, the rows per lane or the row's position, so every launch
//    shape, and the fused two-matrix launch, gives the same bits;
//  * each lane streams RI weight rows (rows r0 + (l >> 3) + 8i): per row one
//    128-bit load of the block's 16 nibble bytes and its binary16 d; the 8
//    lanes of a row read 128 contiguous bytes, whole cache lines.  The
//    (cache-resident) activation is fetched first and the weight rows in
//    order, U columns at a time, all before any arithmetic, so the loads are
//    in flight together and row i's arithmetic overlaps the arrival of rows
//    i+1.. (loads return in order);
//  * nibbles are unpacked in registers: the low nibbles of a 32-bit word are
//    elements i..i+3, the high nibbles elements i+16..i+19 of the block, so
//    (word & 0x0F0F0F0F) and ((word >> 4) & 0x0F0F0F0F) feed v_dot4_i32_i8
//    directly against the matching activation words; the offset 8 is
//    removed once per block as 8 * sum(q8), giving the exact int32 isum;
//  * the int32 sum is scaled by d4*d8 (exact binary32 product of two binary16
//    values) and accumulated with one fma per block in binary32;
//  * partial sums meet in a fixed order: an 8-lane butterfly inside the wave
//    per virtual wave, then the V virtual-wave partials added in order
//    through LDS;
//  * the variant on a raw bf16 / f32 activation quantises each block to Q8_1
//    where it is consumed: the 8 row lanes that share a column load 4 values
//    each and produce the block's code words together (q8_1_block over the
//    lanes that agree in l & 7), with the arithmetic of the standalone
//    quantiser, and swap the words through a per-wave LDS slot.
#include <climits>
#include <cstddef>

#include "device_common.hpp"
#include "kernels.hpp"

namespace q4 {

// Up to kGemvMats matrices share one activation.  Each workgroup serves one
// of them: matrix 0 owns workgroups 0 .. wg0[0] - 1, matrix i > 0 owns
// wg0[i-1] .. wg0[i] - 1, each 8*RI of its rows.  Only non-empty matrices
// are passed; the starts of absent ones are INT_MAX.
//
// Every dispatch's argument block is cold in the scalar cache, and a load
// whose address depends on an earlier argument load pays that miss twice.
// So what a one-matrix launch reads comes first, as separate scalar and
// pointer arguments that gfx950 preloads into SGPRs at wave launch (14
// dwords with this source's -amdgpu-kernarg-preload-count: the weights, the
// activation the variant reads, the sizes and the output); the
// several-matrix fields follow in the argument block, read all up front,
// and a workgroup picks its matrix with selects, never with an index into
// the block.  The waves per workgroup are passed, so the hidden block-size
// argument is not read.  The kernel rebuilds a GemvArgs from them.
struct GemvMat {
    const uint8_t* qs;
    const uint16_t* d;
    float* y;
};
struct GemvArgs {
    GemvMat m0;                     // matrix 0
    const int8_t* xqs;
    const uint16_t* xds;
    const void* x;                  // raw activation (bf16 / f32) for the quantising variant
    int nb;                         // K / 32
    int nwp;                        // waves per workgroup
    int n0;                         // rows of matrix 0
    int K;
    // several-matrix launches only
    int wg0[kGemvMats - 1];         // first workgroup of matrices 1 ..
    int nr[kGemvMats - 1];          // rows of matrices 1 ..
    GemvMat mr[kGemvMats - 1];      // matrices 1 ..
};
static_assert(offsetof(GemvArgs, wg0) == 64, "one-matrix fields in the first 64 bytes");
// The several-matrix fields, passed after the one-matrix ones.
struct GemvTail {
    int wg0[kGemvMats - 1];
    int nr[kGemvMats - 1];
    GemvMat mr[kGemvMats - 1];
};

// The matrix of workgroup b (uniform across the workgroup): its pointers,
// rows and first workgroup.
template <int NMAT>
__device__ __forceinline__ void mat_of(const GemvArgs& a, int b, GemvMat& m, int& rows, int& first_wg) {
    m = a.m0;
    rows = a.n0;
    first_wg = 0;
    if constexpr (NMAT > 1) {
#pragma unroll
        for (int t = 1; t < kGemvMats; t++) {
            const bool sel = b >= a.wg0[t - 1];
            m.qs = sel ? a.mr[t - 1].qs : m.qs;
            m.d = sel ? a.mr[t - 1].d : m.d;
            m.y = sel ? a.mr[t - 1].y : m.y;
            rows = sel ? a.nr[t - 1] : rows;
            first_wg = sel ? a.wg0[t - 1] : first_wg;
        }
    }
}

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

// NMAT: 1 for one matrix, kGemvMats for several (q4_gemv_fused2,
// q4_gemv_multi: each workgroup serves one matrix, found from wg0).  XIN: -1 reads Q8_1 activation planes, DT_BF16 / DT_F32 a
// raw activation that the kernel quantises.  U columns in flight per loop
// iteration, all loaded before any arithmetic, F virtual waves per physical
// wave (U a multiple of F).  For
// M == 1 the kernel keeps to 64 VGPRs, so that two 1024-thread workgroups
// (8 waves per SIMD) share a CU and twice the loads are in flight.
template <int M, int RI, int NMAT, int U, int F, int XIN>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(M == 1 ? 8 : 1)))
void k_q4_gemv(const uint8_t* qs0, const uint16_t* d0, const void* xa, const uint16_t* xds, int nb_, int nwp_,
               int n0_, int K_, float* y0, const void* xb, const GemvTail tail) {
    GemvArgs args;
    args.m0.qs = qs0; args.m0.d = d0; args.m0.y = y0;
    args.xqs = static_cast<const int8_t*>(XIN >= 0 ? xb : xa);
    args.x = XIN >= 0 ? xa : xb;
    args.xds = xds;
    args.nb = nb_; args.nwp = nwp_; args.n0 = n0_; args.K = K_;
    if constexpr (NMAT > 1) {
#pragma unroll
        for (int t = 0; t < kGemvMats - 1; t++) {
            args.wg0[t] = tail.wg0[t];
            args.nr[t] = tail.nr[t];
            args.mr[t] = tail.mr[t];
        }
    }
    static_assert(RI * M * F <= 16, "partials per lane");
    static_assert(U % F == 0, "each iteration covers whole virtual-wave rounds");
    static_assert(U == 1 || M <= 4, "several columns in flight only for small M");
    constexpr bool RAW = XIN >= 0;
    static_assert(!RAW || M <= 4, "the quantising variant takes M <= 4");
    __shared__ float red[kMaxWaves][8 * RI * M];
    __shared__ __attribute__((aligned(16))) uint32_t xch[RAW ? kMaxWaves : 1][RAW ? M : 1][64];

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int nwp = args.nwp;                   // physical waves; V = F * nwp virtual ones
    __builtin_assume(nwp >= 1 && nwp <= kMaxWaves);   // keeps column offsets non-negative
    const int bl = w * 8 + (lane & 7);          // first block column of the lane
    const int rl = lane >> 3;                   // row lane: 0..7
    const int stride = nwp * 8;
    const int nb = args.nb;
    GemvMat mat;
    int nrows, first_wg;
    mat_of<NMAT>(args, (int)blockIdx.x, mat, nrows, first_wg);
    const int r0 = ((int)blockIdx.x - first_wg) * 8 * RI;   // first row in its matrix

    // Rows past the end read the last row (valid memory) and are never
    // written: every load is unconditional.
    const u32x4_t* rqs[RI];
    const uint16_t* rd[RI];
#pragma unroll
    for (int i = 0; i < RI; i++) {
        const int rr = min(r0 + rl + 8 * i, nrows - 1);
        rqs[i] = reinterpret_cast<const u32x4_t*>(mat.qs + (int64_t)rr * nb * 16);
        rd[i] = mat.d + (int64_t)rr * nb;
    }

    float acc[F][RI][M];
#pragma unroll
    for (int f = 0; f < F; f++)
#pragma unroll
        for (int i = 0; i < RI; i++)
#pragma unroll
            for (int m = 0; m < M; m++) acc[f][i][m] = 0.0f;

    uint32_t* slot = &xch[RAW ? w : 0][0][(lane & 7) * 8];
    constexpr int MP = M < 4 ? M : 4;   // activation rows fetched ahead of the weights
    // U columns per iteration (b, b + stride, ...), all loads issued before
    // any arithmetic; a column past the end loads column b again and is not
    // accumulated.
    for (int b = bl; b < nb; b += U * stride) {
        u32x4_t xa[U][RAW ? 1 : MP][2];
        uint32_t d8r[U][RAW ? 1 : MP];
        act4_raw_t<RAW ? XIN : DT_BF16> xr[U][RAW ? M : 1];
        u32x4_t wv[U][RI];
        uint32_t dr[U][RI];
        // loads of column u: activation (cache-resident) first, then the weight
        // rows in order
        auto load = [&](int u, int bu) {
            if constexpr (RAW) {
#pragma unroll
                for (int m = 0; m < M; m++)
                    xr[u][m] = load_act4_raw<RAW ? XIN : DT_BF16>(args.x, (int64_t)m * args.K + (int64_t)bu * 32 + rl * 4);
            } else {
#pragma unroll
                for (int m = 0; m < MP; m++) {
                    const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(args.xqs + (int64_t)m * args.K + (int64_t)bu * 32);
                    xa[u][m][0] = xp[0];
                    xa[u][m][1] = xp[1];
                    d8r[u][m] = args.xds[((int64_t)m * nb + bu) * 2];
                }
            }
            __builtin_amdgcn_sched_barrier(0);     // the activation loads stay ahead of the weights
#pragma unroll
            for (int i = 0; i < RI; i++) {
                dr[u][i] = rd[i][bu];
                wv[u][i] = __builtin_nontemporal_load(rqs[i] + bu);
            }
        };
        // arithmetic of column u (block column bu) into accumulator u mod F
        auto compute = [&](int u, int bu) {
            int neg8sum[M];
            int av[M][8];
            float d8[M];
            if constexpr (RAW) {
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float v[4];
                    act4_to_f32<RAW ? XIN : DT_BF16>(xr[u][m], v);
                    uint32_t d16, s16;
                    slot[m * 64 + rl] = q8_1_block<Q8Strided, false>(v, d16, s16);
                    d8[m] = f16_to_f32(d16);
                }
                // the wave reads back what it wrote (LDS operations of one wave
                // are performed in order)
            }
#pragma unroll
            for (int m = 0; m < M; m++) {
                u32x4_t x0, x1;
                if constexpr (RAW) {
                    x0 = *reinterpret_cast<const u32x4_t*>(slot + m * 64);
                    x1 = *reinterpret_cast<const u32x4_t*>(slot + m * 64 + 4);
                } else if (m < MP) {
                    x0 = xa[u][m < MP ? m : 0][0];
                    x1 = xa[u][m < MP ? m : 0][1];
                    d8[m] = f16_to_f32(d8r[u][m < MP ? m : 0]);
                } else {
                    const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(args.xqs + (int64_t)m * args.K + (int64_t)bu * 32);
                    x0 = xp[0];
                    x1 = xp[1];
                    d8[m] = f16_to_f32(args.xds[((int64_t)m * nb + bu) * 2]);
                }
                av[m][0] = (int)x0[0]; av[m][1] = (int)x0[1]; av[m][2] = (int)x0[2]; av[m][3] = (int)x0[3];
                av[m][4] = (int)x1[0]; av[m][5] = (int)x1[1]; av[m][6] = (int)x1[2]; av[m][7] = (int)x1[3];
                int sq = 0;
#pragma unroll
                for (int t = 0; t < 8; t++) sq = __builtin_amdgcn_sdot4(av[m][t], 0x01010101, sq, false);
                neg8sum[m] = -8 * sq;
            }
#pragma unroll
            for (int i = 0; i < RI; i++) {
                const float d4 = f16_to_f32(dr[u][i]);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const int isum = block_isum(wv[u][i], av[m], neg8sum[m]);
                    acc[u % F][i][m] = fmaf((float)isum, d4 * d8[m], acc[u % F][i][m]);
                }
            }
        };
#pragma unroll
        for (int u = 0; u < U; u++) load(u, (b + u * stride < nb) ? b + u * stride : b);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (u > 0 && b + u * stride >= nb) break;
            compute(u, b + u * stride);
        }
    }

    // 8 block lanes of a row -> one partial per virtual wave (w + f * nwp),
    // then the virtual-wave partials in order
#pragma unroll
    for (int f = 0; f < F; f++)
#pragma unroll
        for (int i = 0; i < RI; i++)
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float v = sum8(acc[f][i][m]);
                if ((lane & 7) == 0) red[w + f * nwp][(i * 8 + rl) * M + m] = v;
            }
    __syncthreads();
    const int nv = F * nwp;
    for (int t = threadIdx.x; t < 8 * RI * M; t += nwp * kWave) {
        const int m = t % M;
        const int slot_i = t / M;               // i * 8 + rl
        const int R = r0 + (slot_i & 7) + 8 * (slot_i >> 3);
        if (R >= nrows) continue;
        float v = red[0][t];
        for (int vw = 1; vw < nv; vw++) v += red[vw][t];
        mat.y[(int64_t)m * nrows + R] = v;
    }
}

// Launch shape: V virtual waves (a function of K only), F of them per
// physical wave, ri rows per lane, u columns in flight per iteration.
struct GemvShape {
    int v, f, ri, u;
};

// V = min(16, ceil(K / 256)) virtual waves.  Rows per lane: the fewest that
// let the whole grid be resident at once (32 waves per CU, the M == 1
// occupancy), at most 4; where V physical waves would need more, V / 2 of
// them with two virtual waves each and both columns in flight (M == 1, at
// most 2 rows per lane, which keeps the registers under 64).  Fewer rows per lane as M (and
// with it the register footprint) grows.  Two columns in flight when a lane
// walks more than one and its registers allow.
static GemvShape pick_shape(int64_t rows, int64_t nb, int64_t M) {
    const int64_t cus = current_cu_count();
    GemvShape g;
    g.v = (int)(nb < 8 ? 1 : ((nb + 7) / 8 > kMaxWaves ? kMaxWaves : (nb + 7) / 8));
    g.f = 1;
    auto rows_per_lane = [&](int nwp) {
        const int64_t slots = cus * 32 / nwp;
        return (rows + 8 * slots - 1) / (8 * slots);
    };
    int64_t ri = rows_per_lane(g.v);
    if (ri > 4 && M == 1 && g.v % 2 == 0) {
        g.f = 2;                                 // two columns in flight: at most 2 rows per lane
        ri = rows_per_lane(g.v / 2);
        ri = ri > 2 ? 2 : ri;
    }
    ri = ri < 1 ? 1 : (ri > 4 ? 4 : ri);
    if (M > 8) ri = 1;
    else if (M > 4 && ri > 2) ri = 2;
    g.ri = (int)ri;
    g.u = g.f == 2 ? 2 : ((nb > 8 * g.v && M * ri <= 2) ? 2 : 1);
    return g;
}

// The quantising variant keeps to 3 rows per lane, 2 for two matrices (its
// registers), and, with rows enough for two per lane on every CU, takes at
// least two (up to that cap): its per-column quantisation is then shared by
// more rows.  Two matrices whose shape already wants more take two virtual
// waves per physical wave.
static GemvShape raw_shape(GemvShape g, int64_t rows, int64_t nb, int64_t M, bool two_mats) {
    const int cap = two_mats ? 2 : 3;
    if (g.f == 1 && M == 1) {
        // never past the cap: raising rows per lane only to halve the waves
        // again (two virtual waves per wave) loses more than the shared
        // quantisation saves
        const int64_t two = rows / (16 * (int64_t)current_cu_count());
        int want = (int)(two < 1 ? 1 : (two > 3 ? 3 : two));
        want = want > cap ? cap : want;
        if (g.ri < want) g.ri = want;
    }
    if (g.ri > cap) {
        if (g.f == 1 && M == 1 && g.v % 2 == 0) g.f = 2;
        g.ri = cap;
    }
    if (g.f == 2) g.ri = g.ri > 2 ? 2 : g.ri;
    g.u = g.f == 2 ? 2 : ((nb > 8 * g.v && M * g.ri <= 2) ? 2 : 1);
    return g;
}

static GemvTail tail_of(const GemvArgs& a) {
    GemvTail t;
    for (int k = 0; k < kGemvMats - 1; k++) {
        t.wg0[k] = a.wg0[k];
        t.nr[k] = a.nr[k];
        t.mr[k] = a.mr[k];
    }
    return t;
}

#define Q4_LAUNCH(...)                                            \
    do {                                                          \
        hipLaunchKernelGGL((__VA_ARGS__), grid, block, 0, s, a.m0.qs, a.m0.d, xa_, a.xds, a.nb, a.nwp, a.n0, a.K, a.m0.y, xb_, tail_of(a)); \
        return;                                                   \
    } while (0)

// Workgroups of each matrix for rows_per_wg rows per workgroup, and the total.
static int assign_workgroups(GemvArgs& a, int rows_per_wg) {
    int wg = (a.n0 + rows_per_wg - 1) / rows_per_wg;
    for (int k = 0; k < kGemvMats - 1; k++) {
        a.wg0[k] = a.nr[k] == 0 ? INT_MAX : wg;
        wg += (a.nr[k] + rows_per_wg - 1) / rows_per_wg;
    }
    return wg;
}

template <int M, int NMAT, int XIN>
static void launch_mx(GemvArgs a, const GemvShape& g, hipStream_t s) {
    // the activation the variant reads first among the preloaded arguments
    const void* xa_ = XIN >= 0 ? a.x : static_cast<const void*>(a.xqs);
    const void* xb_ = XIN >= 0 ? static_cast<const void*>(a.xqs) : a.x;
    a.nwp = g.v / g.f;
    const dim3 block(a.nwp * kWave);
    const dim3 grid((unsigned)assign_workgroups(a, 8 * g.ri));
    if constexpr (M == 1) {
        if (g.f == 2) {
            if (g.ri == 2) Q4_LAUNCH(k_q4_gemv<1, 2, NMAT, 2, 2, XIN>);
            Q4_LAUNCH(k_q4_gemv<1, 1, NMAT, 2, 2, XIN>);
        }
        if (g.u == 2 && g.ri == 2) Q4_LAUNCH(k_q4_gemv<1, 2, NMAT, 2, 1, XIN>);
    }
    if constexpr (M <= 2) {
        if (g.u == 2 && g.ri == 1) Q4_LAUNCH(k_q4_gemv<M, 1, NMAT, 2, 1, XIN>);
    }
    if constexpr (M <= 4 && XIN < 0) {
        if (g.ri == 4) Q4_LAUNCH(k_q4_gemv<M, 4, NMAT, 1, 1, XIN>);
    }
    if constexpr (M <= 4 && (XIN < 0 || NMAT == 1)) {
        if (g.ri == 3) Q4_LAUNCH(k_q4_gemv<M, 3, NMAT, 1, 1, XIN>);
    }
    if constexpr (M <= 8) {
        if (g.ri == 2) Q4_LAUNCH(k_q4_gemv<M, 2, NMAT, 1, 1, XIN>);
    }
    Q4_LAUNCH(k_q4_gemv<M, 1, NMAT, 1, 1, XIN>);
}

#undef Q4_LAUNCH

template <int M, int XIN>
static void launch_m(const GemvArgs& a, const GemvShape& g, hipStream_t s) {
    if (a.nr[0] != 0) launch_mx<M, kGemvMats, XIN>(a, g, s);
    else launch_mx<M, 1, XIN>(a, g, s);
}

// Pack the non-empty matrices of the list into the arguments.
static void pack_mats(GemvArgs& a, int nmat, const uint8_t* const* qs, const uint16_t* const* d, const int64_t* n,
                      float* const* y) {
    GemvMat ms[kGemvMats];
    int ns[kGemvMats];
    int k = 0;
    for (int i = 0; i < nmat; i++) {
        if (n[i] <= 0) continue;
        ms[k] = GemvMat{qs[i], d[i], y[i]};
        ns[k] = (int)n[i];
        k++;
    }
    for (; k < kGemvMats; k++) {
        ms[k] = GemvMat{nullptr, nullptr, nullptr};
        ns[k] = 0;
    }
    a.m0 = ms[0];
    a.n0 = ns[0];
    for (k = 1; k < kGemvMats; k++) {
        a.mr[k - 1] = ms[k];
        a.nr[k - 1] = ns[k];
    }
}

hipError_t launch_q4_gemv_multi(int nmat, const uint8_t* const* qs, const uint16_t* const* d, const int64_t* n,
                                float* const* y, const int8_t* x_qs, const uint16_t* x_ds, const void* x, int xdt,
                                int64_t M, int64_t K, hipStream_t s) {
    if (nmat < 1 || nmat > kGemvMats) return hipErrorInvalidValue;
    GemvArgs a;
    pack_mats(a, nmat, qs, d, n, y);
    int64_t total_rows = a.n0;
    for (int k = 0; k < kGemvMats - 1; k++) total_rows += a.nr[k];
    if (total_rows == 0) return hipSuccess;
    a.xqs = x_qs; a.xds = x_ds; a.x = x;
    a.K = (int)K; a.nb = (int)(K / 32);
    const bool several = a.nr[0] != 0;
    if (x == nullptr) {
        const GemvShape g = pick_shape(total_rows, K / 32, M);
        switch (M) {
#define Q4_GEMV_CASE(m) case m: launch_m<m, -1>(a, g, s); break;
            Q4_GEMV_CASE(1) Q4_GEMV_CASE(2) Q4_GEMV_CASE(3) Q4_GEMV_CASE(4)
            Q4_GEMV_CASE(5) Q4_GEMV_CASE(6) Q4_GEMV_CASE(7) Q4_GEMV_CASE(8)
            Q4_GEMV_CASE(9) Q4_GEMV_CASE(10) Q4_GEMV_CASE(11) Q4_GEMV_CASE(12)
            Q4_GEMV_CASE(13) Q4_GEMV_CASE(14) Q4_GEMV_CASE(15) Q4_GEMV_CASE(16)
#undef Q4_GEMV_CASE
            default: return hipErrorInvalidValue;
        }
    } else {
        const GemvShape g = raw_shape(pick_shape(total_rows, K / 32, M), total_rows, K / 32, M, several);
        switch (M) {
#define Q4_GEMV_ACT_CASE(m)                                                  \
    case m:                                                                  \
        if (xdt == DT_F32) launch_m<m, DT_F32>(a, g, s);                     \
        else launch_m<m, DT_BF16>(a, g, s);                                  \
        break;
            Q4_GEMV_ACT_CASE(1) Q4_GEMV_ACT_CASE(2) Q4_GEMV_ACT_CASE(3) Q4_GEMV_ACT_CASE(4)
#undef Q4_GEMV_ACT_CASE
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace q4
