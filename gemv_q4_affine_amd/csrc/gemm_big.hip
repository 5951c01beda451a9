// gemm_big.hip -- the large-M matrix-core GEMM with 256 x 256 output tiles.
//
//   Y[M,N] = X[M,K] . dequant(Wq)[N,K]^T,  fp32 accumulation,
//
// on the same binary16 X image and weight image as k_gemm_pk (gemm.hip),
// for launches with at least one such tile per CU (the prefill shapes of the
// MLX issue #4621 page, Repro: 2048 and 8192 tokens against W 12288 x 4096).
//
// What changes against k_gemm_pk, and why (gfx950):
//  * Each weight is dequantised once per 256 rows instead of 128.  The
//    dequantisation is VALU work issued by the same wave as the MFMAs, and a
//    wave hides only a few VALU instructions under each MFMA; with 256 rows
//    per wave the dequantisation is about 1.6 VALU instructions per
//    v_mfma_f32_32x32x16_f16 instead of 3.3.  The reuse of a dequantised tile
//    across many token rows is the ET-SoC-1 rewrite's "static reuse"
//    (llama.cpp PR "et-backend: Q4_0 matrix-engine GEMM rewrite for
//    prefill", Overview), taken further.
//  * A wave owns 256 rows x 64 columns: 256 fp32 accumulators per lane, which
//    live in the AGPR half of the register file.  That needs the whole file
//    (one wave per SIMD), so there are no producer waves: the four compute
//    waves issue the direct-to-LDS copies themselves (about ten 1 KiB copies
//    each per K step, a few instructions).
//  * Two LDS rings: X tiles (32 KiB per K step, 4 slots) and weight chunks
//    (9 KiB, 3 slots), 155 KiB in all.  During step k the waves multiply X of
//    step k, read the first X fragments of step k+1 and dequantise the
//    weights of step k+1, so both must have landed one step ahead; both are
//    requested three steps ahead, which leaves two steps for the copies.
//  * Persistent workgroups, one per CU, run whole tiles in rounds.  When the
//    last round would leave at least half of the CUs idle, its tiles run as
//    column halves (256 x 128: one 32-column tile per wave), two CUs per
//    tile: 384 tiles (M = 2048, N = 12288) keep 256 CUs equally busy.  No
//    tile is split along K, so no workgroup ever reads another's results: no
//    partial sums, counters or memory fences.
//  * Output stores drain under the next tile's MFMAs.
//  * Workgroup b runs on XCD b mod 8; the tiles of a round are dealt to
//    consecutive workgroups of an XCD, in an order with M fastest, so an
//    XCD's CUs share the X and weight data of a few column tiles in their L2.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace q4 {

constexpr int kBigRows = 256;                      // rows of an output tile
constexpr int kBigCols = 256;                      // columns of an output tile (one weight-image tile)
constexpr int kBigXSlots = 4;
constexpr int kBigWSlots = 3;
constexpr int kBigXBytes = kBigRows * 64 * 2;      // X of one K step: two 128-row image tiles

struct BigArgs {
    const uint8_t* wimg;     // weight image (256-column tiles, 64-wide K steps)
    const uint8_t* ximg;     // binary16 X image (128-row tiles, 64-wide K steps)
    const int8_t* xexp;      // its row exponents
    void* y;
    int M, N, K;
    int m_tiles, n_tiles;    // 256-row and 256-column tiles
    int nsteps;              // K steps of a tile
    int img_mtiles;          // 128-row tiles of the X image
    int rounds;              // whole tiles per workgroup: tile j * grid + v, j < rounds
    int last_full;           // then whole tile rounds * grid + v for v < last_full
    int last_halves;         // or column half v % 2 of tile rounds * grid + v / 2, v < last_halves
};

struct BigLds {
    uint8_t x[kBigXSlots][kBigXBytes];
    uint8_t w[kBigWSlots][kWChunk];
};

// One direct-to-LDS copy of 16 bytes per lane: lane l's 16 bytes at
// src + voff (voff = 16 l) land at LDS byte address m0 + 16 l.  src and m0 are
// wave-uniform (SGPRs), so a copy costs one scalar move and the load itself.
// Written as inline assembly so that the compiler does not track it as an
// LDS store: it would otherwise wait for every copy in flight (vmcnt(0))
// before any LDS read it cannot prove to be elsewhere, which serialises the
// ring.  The ring's own waits (big_barrier) order the copies with the reads;
// the compiler's waits for its own memory operations stay correct, since
// copies it does not count only make them wait longer.  No register receives
// data.
__device__ __forceinline__ void big_dma16(const uint8_t* src, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(src), "s"(m0)
                 : "memory", "m0");
}

// This lane's index in the wave, computed where it is used: volatile, so
// that the compiler keeps it there instead of holding values derived from
// it in registers across the main loop.
__device__ __forceinline__ int big_lane_now() {
    int r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

// Wait until at most VM vector-memory operations of this wave are in flight,
// and all its LDS accesses are done, then the workgroup barrier.
template <int VM>
__device__ __forceinline__ void big_barrier() { step_barrier<VM>(); }

template <int WF, int YDT>
__global__ __launch_bounds__(256, 1) void k_gemm_big(const BigArgs a) {
    static_assert(WF == WF_Q4_0 || WF == WF_AFFINE4, "quantised weights only");
    constexpr int MT = 8;
    __shared__ __attribute__((aligned(16))) BigLds lds;
    using Blk = typename BlkOf<WF>::T;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform: copy addresses stay scalar
    const int j = lane & 31;
    const int g = lane >> 5;

    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int v = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;    // consecutive tiles per XCD
    const int S = a.nsteps;
    const int nb = a.K / 32;
    // this workgroup's units: whole tiles, then at most one column half
    const int nfull = a.rounds + (v < a.last_full ? 1 : 0);
    const bool has_half = v < a.last_halves;
    const int units = nfull + (has_half ? 1 : 0);
    const int L = units * S;                       // K steps of this workgroup
    if (L == 0) return;
    auto unit_tile = [&](int u) -> int {
        return u < a.rounds ? u * G + v : (has_half ? a.rounds * G + v / 2 : a.rounds * G + v);
    };

    // ---- copies -------------------------------------------------------------
    // wave w: X copies 8w .. 8w+7 (waves 0, 1: rows 0-127; 2, 3: rows 128-255)
    // and weight copies w, w+4 (and 8 for wave 0): a half tile copies the
    // whole weight chunk too and reads its half
    const uint32_t lds_x = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)&lds.x[0][0]);
    const uint32_t lds_w = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)&lds.w[0][0]);
    // the next step to request: unit cu, step ck, tile (cmt, cnt)
    int cu = 0, ck = 0, cmt = 0, cnt_ = 0;
    auto set_unit = [&](int u) __attribute__((always_inline)) {
        const int t = unit_tile(u);
        cmt = t % a.m_tiles;
        cnt_ = t / a.m_tiles;
    };
    set_unit(0);
    // Requests are issued in eight parts, one at each boundary between
    // half-segments of a step, a copy or two at a time between MFMAs: a burst
    // of copies holds up the wave's instruction issue long enough to starve
    // the matrix pipe.  X copies 0-7 go one per part; the weight copies
    // `wave`, wave+4 (and 8 for wave 0) ride along in parts 1, 4 and 6.
    struct Req {
        const uint8_t* xs;
        const uint8_t* ws;
        uint32_t xd, wd;
    };
    auto req_prepare = [&](int i) __attribute__((always_inline)) {
        Req q;
        int im = 2 * cmt + (wave >> 1);
        im = im < a.img_mtiles ? im : a.img_mtiles - 1;        // rows past M: never stored
        q.xs = a.ximg + ((int64_t)im * S + ck) * (kImgTile * 2) + (wave & 1) * 8192;
        q.xd = lds_x + (uint32_t)(i % kBigXSlots) * kBigXBytes + (uint32_t)wave * 8192;
        q.ws = a.wimg + ((int64_t)cnt_ * S + ck) * kWChunk;
        q.wd = lds_w + (uint32_t)(i % kBigWSlots) * kWChunk;
        if (++ck == S) {
            ck = 0;
            if (++cu < units) set_unit(cu);
        }
        return q;
    };
    auto req_part = [&](const Req& q, int part) __attribute__((always_inline)) {
        const uint32_t voff = (uint32_t)big_lane_now() * 16;
        big_dma16(q.xs + part * 1024, voff, q.xd + part * 1024);
        if (part == 1) big_dma16(q.ws + wave * 1024, voff, q.wd + wave * 1024);
        if (part == 4) big_dma16(q.ws + (wave + 4) * 1024, voff, q.wd + (wave + 4) * 1024);
        if (part == 6 && wave == 0) big_dma16(q.ws + 8 * 1024, voff, q.wd + 8 * 1024);
    };
    auto request = [&](int i) __attribute__((always_inline)) {
        const Req q = req_prepare(i);
        for (int p = 0; p < 8; p++) req_part(q, p);
    };

    // ---- accumulators and fragments -------------------------------------------
    floatx16_t acc[MT][2];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < MT; mi++)
#pragma unroll
            for (int ni = 0; ni < 2; ni++)
#pragma unroll
                for (int e = 0; e < 16; e++) acc[mi][ni][e] = 0.0f;
    };
    zero_acc();
    u32x4_t bfA[2][4], bfB[2][4];
    u32x4_t a0[MT];
    const NibMasks masks = NibMasks::make();

    // X fragment (mi, s) of this lane: row mi*32 + j, chunk 4g + s, swizzled
    // by the row (rows 128-255 follow rows 0-127 in the slot)
    int aofs[4];
#pragma unroll
    for (int s = 0; s < 4; s++) aofs[s] = j * 64 + (((4 * g + s) ^ img_swz(j)) * 8);
    // fragments 4h .. 4h+3 (half h of the 256 rows)
    auto read_a = [&](int i, int s, int h, u32x4_t (&av)[MT]) __attribute__((always_inline)) {
        const uint16_t* la = reinterpret_cast<const uint16_t*>(lds.x[i % kBigXSlots]);
#pragma unroll
        for (int mi = 4 * h; mi < 4 * h + 4; mi++)
            av[mi] = *reinterpret_cast<const u32x4_t*>(&la[mi * 32 * 64 + aofs[s]]);
    };
    // Scheduling of one half of a segment (a region the copy instructions
    // bound, which the compiler does not schedule across):
    //  * first half: one MFMA, the segment's first LDS reads (X fragments 0-3
    //    of the next slice, and the raw weights in segment 0), then the
    //    remaining MFMAs of the half, each followed by up to `valu` vector
    //    instructions;
    //  * second half: the X fragments 4-7 of the next slice (into the
    //    registers the first half's MFMAs have released), then the half's
    //    MFMAs, each followed by up to `valu` vector instructions.
    // Two half loads keep 48 fragment registers live instead of 64.
    auto order_first = [&](auto nmfma, auto nreads, auto valu) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, decltype(nreads)::value, 0);
#pragma unroll
        for (int e = 1; e < decltype(nmfma)::value; e++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, decltype(valu)::value, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto order_second = [&](auto nmfma, auto valu) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int e = 0; e < decltype(nmfma)::value; e++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, decltype(valu)::value, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- output ------------------------------------------------------------------
    // Lane: column j of each 32x32 tile, rows 8*(e/4) + 4*g + e%4.  A DPP swap
    // of neighbouring lanes gives each lane two adjacent columns of one row
    // (the even lane row r, the odd lane row r+1), stored as a pair.  One
    // 32x32 tile at a time (a scheduling fence after each): the scheduler
    // would otherwise read every accumulator into VGPRs at once.
    const bool pair_ok = (a.N & 1) == 0;
    auto swap_pair = [](float x) __attribute__((always_inline)) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    };
    // A tile wholly inside Y (with N even) takes a path with no bounds test:
    // every pair store is in bounds and aligned, and a lane's stores advance
    // by fixed multiples of N from one base address.
    auto store_tile_w = [&](int m0, int nw0, auto ntc, auto whole_c) __attribute__((always_inline)) {
        constexpr int NT = decltype(ntc)::value;
        constexpr bool kWhole = decltype(whole_c)::value;
        const int ln = big_lane_now();
        const int j = ln & 31, g = ln >> 5;
        const bool odd = (ln & 1) != 0;
#pragma unroll
        for (int mi = 0; mi < MT; mi++) {
            // the X image's exponents of sub-tile mi through the scalar cache
            // (the table covers 128-row tiles: a sub-tile wholly past M reads
            // none and stores nothing), then this lane's 8
            if (!kWhole && m0 + mi * 32 >= a.M) continue;
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
                const int col = nw0 + ni * 32 + (j & ~1);
                const int64_t base = (int64_t)r0 * a.N + col;
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const float a0v = acc[mi][ni][e], a1v = acc[mi][ni][e + 1];
                    const float d0 = swap_pair(a0v), d1 = swap_pair(a1v);
                    // row r of the X image was scaled by 2^e(r)
                    const int ue = -xexp_of(ex, e >> 2, (e >> 1) & 1);
                    const float lo_v = ldexpf(odd ? d1 : a0v, ue);
                    const float hi_v = ldexpf(odd ? a1v : d0, ue);
                    const int dr = 8 * (e >> 2) + (e & 3);
                    if (!kWhole && (r0 + dr >= a.M || col >= a.N)) continue;
                    const int64_t off = base + (int64_t)dr * a.N;
                    const bool pair = kWhole || (pair_ok && col + 1 < a.N);
                    if constexpr (YDT == DT_BF16) {
                        uint16_t* yp = reinterpret_cast<uint16_t*>(a.y) + off;
                        if (pair) {
                            const f32x2_t f = {lo_v, hi_v};
                            *reinterpret_cast<uint32_t*>(yp) =
                                __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
                        } else {
                            yp[0] = (uint16_t)f32_to_bf16(lo_v);
                            if (col + 1 < a.N) yp[1] = (uint16_t)f32_to_bf16(hi_v);
                        }
                    } else {
                        float* yp = reinterpret_cast<float*>(a.y) + off;
                        if (pair) {
                            *reinterpret_cast<f32x2_t*>(yp) = f32x2_t{lo_v, hi_v};
                        } else {
                            yp[0] = lo_v;
                            if (col + 1 < a.N) yp[1] = hi_v;
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto store_tile = [&](int m0, int nw0, auto ntc) __attribute__((always_inline)) {
        constexpr int NT = decltype(ntc)::value;
        const bool whole = m0 + kBigRows <= a.M && nw0 + 32 * NT <= a.N && pair_ok;   // this wave's columns
        if (whole) store_tile_w(m0, nw0, ntc, std::true_type{});
        else store_tile_w(m0, nw0, ntc, std::false_type{});
    };

    // ---- one unit: S steps of one tile, NT = 2 (whole) or 1 (column half) ------
    // wcol: this wave's first column in the weight chunk; the unit's first
    // local step is i0.
    auto run_unit = [&](int i0, int mt, int nt, int wcol, auto ntc) __attribute__((always_inline)) {
        constexpr int NT = decltype(ntc)::value;
        // raw weight blocks of local step i from its ring slot
        auto read_w = [&](int i, Blk (&r)[2]) __attribute__((always_inline)) {
            const uint8_t* wb = lds.w[i % kBigWSlots];
            const int ln = big_lane_now();
            const int j = ln & 31, g = ln >> 5;
#pragma unroll
            for (int ni = 0; ni < NT; ni++) {
                const int cw = wcol + ni * 32 + j;
                r[ni].q = *reinterpret_cast<const u32x4_t*>(wb + (g * 256 + cw) * 16);
                if constexpr (WF == WF_Q4_0) {
                    r[ni].d = reinterpret_cast<const uint16_t*>(wb + 8192)[g * 256 + cw];
                } else {
                    r[ni].s = reinterpret_cast<const uint16_t*>(wb + 8192)[cw];
                    r[ni].b = reinterpret_cast<const uint16_t*>(wb + 8704)[cw];
                }
            }
        };
        // the MFMAs of slice s on fragments 4h .. 4h+3; `first` selects (0, 0)
        // of half 0, else the others
        auto mfma_half = [&](int s, const u32x4_t (&av)[MT], const u32x4_t (&bf)[2][4], int h, bool first)
            __attribute__((always_inline)) {
#pragma unroll
            for (int mi = 4 * h; mi < 4 * h + 4; mi++)
#pragma unroll
                for (int ni = 0; ni < NT; ni++)
                    if ((mi == 0 && ni == 0) == first)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(half8_t, av[mi]), __builtin_bit_cast(half8_t, bf[ni][s]),
                            acc[mi][ni], 0, 0, 0);
        };
        constexpr int kWReads = NT * (WF == WF_Q4_0 ? 2 : 3);
        // One K step in four segments (K slices s = 0..3): the X fragments of
        // slice s+1 are read during slice s (the next step's slice 0 during
        // slice 3), the raw weights of step i+1 in segment 0, and their
        // dequantisation runs word by word under the MFMAs of segments 1-3.
        // At a unit's last step the i+1 data belong to the next unit (or to no
        // step): they are read again when it starts.
        auto body = [&](int i, const u32x4_t (&cur)[2][4], u32x4_t (&nxt)[2][4], bool req, const Req& q)
            __attribute__((always_inline)) {
            Blk r[2];
            BlkConst c0, c1;
            u32x4_t a1[MT], a2[MT], a3[MT];
            using HALF = std::integral_constant<int, MT * NT / 2>;
            // The dequantisation of step i+1's weights, word by word (8 words
            // of 8 weights per lane for two blocks, 4 for one), placed in the
            // half-segments 0B, 1A, 1B, 2A, 2B, 3A, 3B after the raw words
            // arrive (read in half-segment 0A).
            // word w of block ni, then a fence on the fragments it wrote so
            // that the compiler keeps the work here instead of sinking it to
            // the end of the step
            auto word = [&](int ni, const BlkConst& c, int w) __attribute__((always_inline)) {
                blk_word<WF>(r[ni], c, w, masks, nxt[ni]);
                if constexpr (WF == WF_Q4_0) {
                    asm volatile("" : "+v"(nxt[ni][w >> 1]), "+v"(nxt[ni][2 + (w >> 1)]));
                } else {
                    asm volatile("" : "+v"(nxt[ni][w]));
                }
            };
            auto deq = [&](int hs) __attribute__((always_inline)) {
                if constexpr (NT == 2) {
                    if (hs == 1) { c0 = blk_const<WF>(r[0]); word(0, c0, 0); }
                    if (hs == 2) word(0, c0, 1);
                    if (hs == 3) word(0, c0, 2);
                    if (hs == 4) word(0, c0, 3);
                    if (hs == 5) { c1 = blk_const<WF>(r[1]); word(1, c1, 0); }
                    if (hs == 6) { word(1, c1, 1); word(1, c1, 2); }
                    if (hs == 7) word(1, c1, 3);
                } else {
                    if (hs == 1) { c0 = blk_const<WF>(r[0]); word(0, c0, 0); }
                    if (hs == 3) word(0, c0, 1);
                    if (hs == 5) word(0, c0, 2);
                    if (hs == 7) word(0, c0, 3);
                }
            };
            constexpr int kV = NT == 2 ? 2 : 3;      // VALU slots after each MFMA
            // slice s: half A (fragments 0-3, the next slice's 0-3 read), the
            // request's part s, half B (fragments 4-7, the next slice's 4-7
            // read first)
            auto slice = [&](int s, const u32x4_t (&av)[MT], u32x4_t (&an)[MT], int in, int sn)
                __attribute__((always_inline)) {
                mfma_half(s, av, cur, 0, true);
                read_a(in, sn, 0, an);
                if (s == 0) read_w(i + 1, r);
                mfma_half(s, av, cur, 0, false);
                deq(2 * s);
                if (s == 0) order_first(HALF{}, std::integral_constant<int, 4 + kWReads>{}, std::integral_constant<int, kV>{});
                else order_first(HALF{}, std::integral_constant<int, 4>{}, std::integral_constant<int, kV>{});
                if (req) req_part(q, 2 * s);
                read_a(in, sn, 1, an);
                mfma_half(s, av, cur, 1, false);
                deq(2 * s + 1);
                order_second(HALF{}, std::integral_constant<int, kV>{});
                if (req) req_part(q, 2 * s + 1);
            };
            slice(0, a0, a1, i, 1);
            slice(1, a1, a2, i, 2);
            slice(2, a2, a3, i, 3);
            slice(3, a3, a0, i + 1, 0);
#pragma unroll
            for (int ni = 0; ni < NT; ni++)
#pragma unroll
                for (int t = 0; t < 4; t++) asm volatile("" : "+v"(nxt[ni][t]));
        };
        // One step: request step i+3 (into the slots of steps i-1: X, and i:
        // weights, both consumed by the last barrier), multiply step i while
        // dequantising step i+1's weights, then wait until step i+2 has landed
        // (only this step's requests may still be in flight) and meet at the
        // barrier.  Blocks past the end of K (K = 32 mod 64) carry a zero scale
        // in the weight image, and the X image holds zeros there.
        auto step = [&](int i, const u32x4_t (&cur)[2][4], u32x4_t (&nxt)[2][4]) __attribute__((always_inline)) {
            const bool req = i + 3 < L;
            Req q{};
            if (req) q = req_prepare(i + 3);
            body(i, cur, nxt, req, q);
            if (req) {
                if (wave == 0) big_barrier<8 + 3>();
                else big_barrier<8 + 2>();
            } else {
                big_barrier<0>();
            }
        };
        // the unit's first weight fragments and X fragments, from the ring;
        // then a barrier: the first step's request (step i0+3) overwrites the
        // weight slot of step i0
        {
            Blk r[2];
            read_w(i0, r);
#pragma unroll
            for (int ni = 0; ni < NT; ni++) {
                zero_blk<WF>(r[ni], g < nb);
                blk_frags_perm<WF>(r[ni], masks, bfA[ni]);
            }
            read_a(i0, 0, 0, a0);
            read_a(i0, 0, 1, a0);
            big_barrier<63>();
        }
        int i = i0;
        const int pe = i0 + S;
        for (; i + 1 < pe; i += 2) {
            step(i, bfA, bfB);
            step(i + 1, bfB, bfA);
        }
        if (i < pe) step(i, bfA, bfB);
        // the outputs; the stores drain under the next unit's MFMAs
        store_tile(mt * kBigRows, nt * kBigCols + wcol, ntc);
        zero_acc();
    };

    // ---- prologue: steps 0 and 1 requested, then step 2; the first two
    // landed (step 2 may stay in flight) ------------------------------------------
    for (int i = 0; i < 3 && i < L; i++) request(i);
    if (L > 2) {
        if (wave == 0) big_barrier<8 + 3>();
        else big_barrier<8 + 2>();
    } else {
        big_barrier<0>();
    }
    for (int u = 0; u < nfull; u++) {
        const int t = unit_tile(u);
        run_unit(u * S, t % a.m_tiles, t / a.m_tiles, wave * 64, std::integral_constant<int, 2>{});
    }
    if (has_half) {
        const int t = unit_tile(nfull);
        run_unit(nfull * S, t % a.m_tiles, t / a.m_tiles, (v % 2) * 128 + wave * 32, std::integral_constant<int, 1>{});
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

static int64_t big_tiles(int64_t M, int64_t N) { return ((M + kBigRows - 1) / kBigRows) * ((N + kBigCols - 1) / kBigCols); }

// The 256 x 256 kernel takes a launch with at least one such tile per CU.
bool gemm_big_applies(int64_t M, int64_t N, int64_t K) {
    (void)K;
    return big_tiles(M, N) >= current_cu_count();
}

template <int WF, int YDT>
static void launch_big_t(const BigArgs& ba, int grid, hipStream_t s) {
    hipLaunchKernelGGL((k_gemm_big<WF, YDT>), dim3((unsigned)grid), dim3(256), 0, s, ba);
}

hipError_t launch_gemm_big(int wfmt, const void* wimg, const void* ximg, void* y, int ydt, int64_t M, int64_t N,
                           int64_t K, hipStream_t s) {
    BigArgs ba{};
    ba.wimg = static_cast<const uint8_t*>(wimg);
    ba.ximg = static_cast<const uint8_t*>(ximg);
    ba.xexp = x_image_exponents(ximg, M, K);
    ba.y = y;
    ba.M = (int)M;
    ba.N = (int)N;
    ba.K = (int)K;
    ba.m_tiles = (int)((M + kBigRows - 1) / kBigRows);
    ba.n_tiles = (int)((N + kBigCols - 1) / kBigCols);
    ba.nsteps = (int)((K + 63) / 64);
    ba.img_mtiles = (int)((M + kImgRows - 1) / kImgRows);
    const int G = current_cu_count();
    const int64_t T = (int64_t)ba.m_tiles * ba.n_tiles;
    ba.rounds = (int)(T / G);
    const int rem = (int)(T - (int64_t)ba.rounds * G);
    // a last round at most half full runs as column halves on twice the CUs
    ba.last_halves = 2 * rem <= G ? 2 * rem : 0;
    ba.last_full = 2 * rem <= G ? 0 : rem;
    if (wfmt == WF_Q4_0) {
        if (ydt == DT_BF16) launch_big_t<WF_Q4_0, DT_BF16>(ba, G, s);
        else launch_big_t<WF_Q4_0, DT_F32>(ba, G, s);
    } else {
        if (ydt == DT_BF16) launch_big_t<WF_AFFINE4, DT_BF16>(ba, G, s);
        else launch_big_t<WF_AFFINE4, DT_F32>(ba, G, s);
    }
    return hipGetLastError();
}

}  // namespace q4
