/*
 * q4_oracle.c -- plain, slow, obviously-correct CPU reference for 4-bit
 * block-quantised matrix multiply, Y[M,N] = X[M,K] . dequant(Wq)[N,K]^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library: every conversion and every rounding step below
 * is written out again from its definition.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see build.py).
 * -ffp-contract=off matters: the quantisers are defined as separate IEEE
 * binary32 multiplies and adds, never fused.
 *
 * Sources of the definitions
 *  - The Q4_0 format (32-weight blocks, an fp16 scale, 16 bytes of nibbles,
 *    w = (q-8)*d) is the GGUF block format that the pages run:
 *    llama.cpp PR "et-backend: Q4_0 matrix-engine GEMM rewrite for prefill"
 *    (Overview) and "2026-05-06 Q4 sync-after focused repro" (Important source
 *    touch points; Quality-cleared launch recipe).  The pages print neither
 *    the quantiser nor the byte layout; the readings used here are listed at
 *    each function.
 *  - The Q8_1 activation format is named by the same repro page (the
 *    q4_0_q8_1 MMVQ kernels and the Q8 cache flag); again not defined there.
 *  - The affine 4-bit, group-64 format (w ~ q*s + b, bf16 s and b) is the MLX
 *    quantize / dequantize / quantized_matmul API of MLX issue #4621
 *    "quantized_matmul takes 14-41% longer than dequantize + bf16 matmul at
 *    prefill sizes" (Repro).  The page shows the API, not the rule.
 *  - The matmul with transpose=True semantics (W stored [N,K], rows are output
 *    features) is the quantized_matmul call of that same Repro section.
 *
 * parity unpinned: none -- every function here is pinned by tests under
 * tests/ (hand-worked blocks, library conversions, exact rational brute
 * force, BLAS cross-checks, closed forms and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Binary16 / bfloat16 conversions, written from the IEEE-754 definitions.  */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round the integer m * 2^-shift to the nearest integer, ties to even. */
static uint64_t rne_shift(uint64_t m, int shift) {
    if (shift <= 0) return m << (-shift);
    if (shift >= 64) return 0;
    uint64_t q = m >> shift;
    uint64_t rem = m & ((((uint64_t)1) << shift) - 1);
    uint64_t half = ((uint64_t)1) << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) q++;
    return q;
}

/* binary32 -> binary16, round to nearest even, subnormals kept, overflow to
 * infinity, NaN stays NaN (quiet). */
uint16_t or_f32_to_f16(float f) {
    uint32_t x = f32_bits(f);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);   /* NaN */
    if (ax == 0x7F800000u) return (uint16_t)(sign | 0x7C00u);  /* inf */
    if (ax == 0) return sign;
    /* value = m * 2^(e - 23), m < 2^24 */
    int e;
    uint64_t m;
    if ((ax >> 23) == 0) { e = -126; m = ax & 0x7FFFFFu; }          /* f32 subnormal */
    else { e = (int)(ax >> 23) - 127; m = (ax & 0x7FFFFFu) | 0x800000u; }
    /* binary16 quantum at this magnitude: 2^(max(e,-14) - 10) */
    int qexp = (e > -14 ? e : -14) - 10;
    int shift = qexp - (e - 23);
    uint64_t q = rne_shift(m, shift);           /* value in units of 2^qexp */
    uint32_t bits;
    if (e >= -14) {
        /* normal range: q in [2^10, 2^11]; encoding is monotone, so a carry
         * out of the significand bumps the exponent by itself. */
        bits = (uint32_t)(((e + 14) << 10) + q);
    } else {
        bits = (uint32_t)q;                     /* subnormal units of 2^-24 */
    }
    if (bits >= 0x7C00u) bits = 0x7C00u;        /* overflow -> inf */
    return (uint16_t)(sign | bits);
}

float or_f16_to_f32(uint16_t h) {
    uint32_t sign = (h & 0x8000u) ? 1u : 0u;
    uint32_t ex = (h >> 10) & 0x1Fu;
    uint32_t fr = h & 0x3FFu;
    float mag;
    if (ex == 0x1F) {
        mag = fr ? NAN : INFINITY;
    } else if (ex == 0) {
        mag = ldexpf((float)fr, -24);           /* subnormal or zero */
    } else {
        mag = ldexpf((float)(fr | 0x400u), (int)ex - 25);
    }
    return sign ? -mag : mag;
}

/* binary32 -> bfloat16 (the top 16 bits of binary32), round to nearest even. */
uint16_t or_f32_to_bf16(float f) {
    uint32_t x = f32_bits(f);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((x >> 16) & 0x8000u) | 0x7FC0u);
    uint64_t q = rne_shift(x & 0x7FFFFFFFu, 16);  /* monotone encoding again */
    return (uint16_t)(((x >> 16) & 0x8000u) | (uint32_t)q);
}

float or_bf16_to_f32(uint16_t b) { return bits_f32(((uint32_t)b) << 16); }

/* ------------------------------------------------------------------------ */
/* Q4_0                                                                      */
/* ------------------------------------------------------------------------ */

/*
 * Q4_0 quantisation of one row-major weight matrix W[N][K] (K % 32 == 0).
 *
 * Per block of 32 consecutive weights along K (the GGUF Q4_0 convention the
 * pages run; readings where the pages are silent):
 *   1. scan j = 0..31; keep the first element of largest magnitude, with its
 *      sign ("max");
 *   2. d = max / -8 in binary32, so that element maps exactly to code 0;
 *   3. id = 1/d (IEEE binary32 division), or 0 for an all-zero block;
 *   4. q_j = min(15, trunc(w_j*id + 8.5)), each op a separate binary32 op
 *      (the argument is >= 0.5, so truncation is floor: round half up of
 *      w/d + 8; the opposite-signed extreme can reach 16 and is clamped);
 *   5. the scale is stored as binary16(d) (RNE) -- an all-zero block stores
 *      -0.0 (0x8000), since 0 / -8 = -0;
 *   6. nibble order (reading): byte i of the block's 16 bytes holds q_i in
 *      its low nibble and q_{i+16} in its high nibble.
 * Output planes: qs[(n*K/32 + b)*16 + i] and d[n*K/32 + b] (binary16 bits).
 */
void or_q4_0_quantize(const float* w, int64_t N, int64_t K, uint8_t* qs, uint16_t* d) {
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < nb; b++) {
            const float* blk = w + n * K + b * 32;
            float amax = 0.0f, maxv = 0.0f;
            for (int j = 0; j < 32; j++) {
                float a = fabsf(blk[j]);
                if (a > amax) { amax = a; maxv = blk[j]; }
            }
            float dd = maxv / -8.0f;
            float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
            int code[32];
            for (int j = 0; j < 32; j++) {
                float t = blk[j] * id;
                float u = t + 8.5f;
                int c = (int)u;              /* u >= 0.5: truncation == floor */
                code[j] = c < 15 ? c : 15;
            }
            uint8_t* out = qs + (n * nb + b) * 16;
            for (int i = 0; i < 16; i++)
                out[i] = (uint8_t)(code[i] | (code[i + 16] << 4));
            d[n * nb + b] = or_f32_to_f16(dd);
        }
    }
}

/* Code of element j (0..31) of one 16-byte Q4_0 block, per the nibble order above. */
static int q4_code(const uint8_t* blk16, int j) {
    return j < 16 ? (blk16[j] & 0x0F) : (blk16[j - 16] >> 4);
}

/* Dequantised weights, exact: w^ = (q - 8) * d, in binary64. */
void or_q4_0_dequantize(const uint8_t* qs, const uint16_t* d, int64_t N, int64_t K, double* out) {
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nb; b++) {
            double dd = (double)or_f16_to_f32(d[n * nb + b]);
            const uint8_t* blk = qs + (n * nb + b) * 16;
            for (int j = 0; j < 32; j++)
                out[n * K + b * 32 + j] = (double)(q4_code(blk, j) - 8) * dd;
        }
}

/*
 * Dequantise to a 16-bit dense type: the binary32 value of (q-8)*d (exact:
 * a 4-bit integer times an 11-bit significand), then rounded to nearest even
 * into binary16 (half_kind = 0) or bfloat16 (half_kind = 1).
 */
void or_q4_0_dequantize_half(const uint8_t* qs, const uint16_t* d, int64_t N, int64_t K,
                             int half_kind, uint16_t* out) {
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nb; b++) {
            double dd = (double)or_f16_to_f32(d[n * nb + b]);
            const uint8_t* blk = qs + (n * nb + b) * 16;
            for (int j = 0; j < 32; j++) {
                float v = (float)((double)(q4_code(blk, j) - 8) * dd);
                out[n * K + b * 32 + j] = half_kind ? or_f32_to_bf16(v) : or_f32_to_f16(v);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Q8_1 activations                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Q8_1 quantisation of X[M][K] (K % 32 == 0), per block of 32 along K:
 *   amax = max |x_j|;  d = amax / 127;  id = d ? 1/d : 0   (binary32);
 *   q_j = round-half-away-from-zero(x_j * id)  -> [-127, 127];
 *   s = binary16(d * (float)sum_j q_j)   (reading: the scaled integer sum);
 *   ds[(m*K/32 + b)*2 + 0] = binary16(d), ds[... + 1] = s.
 */
void or_q8_1_quantize(const float* x, int64_t M, int64_t K, int8_t* qs, uint16_t* ds) {
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t b = 0; b < nb; b++) {
            const float* blk = x + m * K + b * 32;
            float amax = 0.0f;
            for (int j = 0; j < 32; j++) {
                float a = fabsf(blk[j]);
                if (a > amax) amax = a;
            }
            float dd = amax / 127.0f;
            float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
            int sum = 0;
            for (int j = 0; j < 32; j++) {
                float t = blk[j] * id;
                int q = (int)roundf(t);
                qs[m * K + b * 32 + j] = (int8_t)q;
                sum += q;
            }
            float s = dd * (float)sum;
            ds[(m * nb + b) * 2 + 0] = or_f32_to_f16(dd);
            ds[(m * nb + b) * 2 + 1] = or_f32_to_f16(s);
        }
}

/* Exact dequantised activation: x^ = q * d in binary64. */
void or_q8_1_dequantize(const int8_t* qs, const uint16_t* ds, int64_t M, int64_t K, double* out) {
    const int64_t nb = K / 32;
    for (int64_t m = 0; m < M; m++)
        for (int64_t b = 0; b < nb; b++) {
            double dd = (double)or_f16_to_f32(ds[(m * nb + b) * 2]);
            for (int j = 0; j < 32; j++)
                out[m * K + b * 32 + j] = (double)qs[m * K + b * 32 + j] * dd;
        }
}

/*
 * Per-block integer dot of a Q4_0 weight row with a Q8_1 activation row:
 *   isum[m][n][b] = sum_{j<32} (q4_j - 8) * q8_j      (int32, exact)
 * The decode path of the pages is this integer block dot (ET-SoC-1
 * "vecdot" kernel, PR Overview; q4_0 x q8_1 MMVQ kernels, repro page,
 * Important source touch points).
 */
void or_q4q8_block_dots(const uint8_t* wqs, const int8_t* xqs, int64_t M, int64_t N, int64_t K,
                        int32_t* isum) {
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++)
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t* blk = wqs + (n * nb + b) * 16;
                const int8_t* a = xqs + m * K + b * 32;
                int32_t s = 0;
                for (int j = 0; j < 32; j++) s += (q4_code(blk, j) - 8) * (int32_t)a[j];
                isum[(m * N + n) * nb + b] = s;
            }
}

/*
 * Decode GEMV output of the integer path, in binary64:
 *   y[m][n] = sum_b d4[n][b] * d8[m][b] * isum[m][n][b]
 * which equals dequant(Wq) . dequant(Q8_1(x)) exactly (up to binary64
 * rounding of the sum).
 */
void or_q4q8_gemv(const uint8_t* wqs, const uint16_t* wd, const int8_t* xqs, const uint16_t* xds,
                  int64_t M, int64_t N, int64_t K, double* y) {
    const int64_t nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t* blk = wqs + (n * nb + b) * 16;
                const int8_t* a = xqs + m * K + b * 32;
                int32_t s = 0;
                for (int j = 0; j < 32; j++) s += (q4_code(blk, j) - 8) * (int32_t)a[j];
                double d4 = (double)or_f16_to_f32(wd[n * nb + b]);
                double d8 = (double)or_f16_to_f32(xds[(m * nb + b) * 2]);
                acc += d4 * d8 * (double)s;
            }
            y[m * N + n] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Dense binary64 matmul, transpose=True semantics                           */
/* ------------------------------------------------------------------------ */

/* y[m][n] = sum_k x[m][k] * w[n][k], binary64, k ascending. */
void or_matmul_f64(const double* x, const double* w, int64_t M, int64_t N, int64_t K, double* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            const double* xr = x + m * K;
            const double* wr = w + n * K;
            for (int64_t k = 0; k < K; k++) acc += xr[k] * wr[k];
            y[m * N + n] = acc;
        }
}

/* The same sum for a list of (m, n) output positions only. */
void or_matmul_f64_sampled(const double* x, const double* w, int64_t K, int64_t count,
                           const int64_t* ms, const int64_t* ns, double* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        double acc = 0.0;
        const double* xr = x + ms[i] * K;
        const double* wr = w + ns[i] * K;
        for (int64_t k = 0; k < K; k++) acc += xr[k] * wr[k];
        y[i] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Affine 4-bit, group G (G = 64 on the pages)                               */
/* ------------------------------------------------------------------------ */

/*
 * Affine quantisation of bfloat16 weights W[N][K] (K % G == 0), per group of
 * G consecutive weights along K.  The MLX page shows only the API
 * (quantize(w, group_size=64, bits=4) -> (wq, scales, biases), w ~ q*s + b,
 * bf16 weights); the rule is the plain min/max reading:
 *   mn = min, mx = max of the group (a zero extreme taken as +0);
 *   s  = bfloat16(binary32((mx - mn) / 15));   b = bfloat16(mn)  (exact);
 *   q  = s ? clamp(floor((w - b) / s + 0.5), 0, 15) : 0     (binary32 ops,
 *        with the stored s and b);
 *   packing (reading): element 2i in the low nibble of byte i, 2i+1 in the
 *   high nibble; q plane [N][K/2], s and b planes [N][K/G] (bfloat16 bits).
 */
void or_affine4_quantize(const uint16_t* wbf, int64_t N, int64_t K, int64_t G,
                         uint8_t* wq, uint16_t* scales, uint16_t* biases) {
    const int64_t ng = K / G;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < ng; g++) {
            const uint16_t* grp = wbf + n * K + g * G;
            float mn = or_bf16_to_f32(grp[0]), mx = mn;
            for (int64_t j = 1; j < G; j++) {
                float v = or_bf16_to_f32(grp[j]);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            mn = mn + 0.0f;   /* -0 -> +0 */
            mx = mx + 0.0f;
            float s32 = (mx - mn) / 15.0f;
            uint16_t sb = or_f32_to_bf16(s32);
            uint16_t bb = or_f32_to_bf16(mn);
            float s = or_bf16_to_f32(sb), b = or_bf16_to_f32(bb);
            scales[n * ng + g] = sb;
            biases[n * ng + g] = bb;
            for (int64_t j = 0; j < G; j += 2) {
                int c[2];
                for (int t = 0; t < 2; t++) {
                    float v = or_bf16_to_f32(grp[j + t]);
                    if (s == 0.0f) { c[t] = 0; continue; }
                    float r = (v - b) / s;
                    float f = floorf(r + 0.5f);
                    c[t] = f < 0.0f ? 0 : (f > 15.0f ? 15 : (int)f);
                }
                wq[n * (K / 2) + (g * G + j) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
}

static int affine_code(const uint8_t* wq, int64_t K, int64_t n, int64_t k) {
    uint8_t byte = wq[n * (K / 2) + k / 2];
    return (k & 1) ? (byte >> 4) : (byte & 0x0F);
}

/* Exact dequantised weights: w^ = q*s + b in binary64. */
void or_affine4_dequantize(const uint8_t* wq, const uint16_t* scales, const uint16_t* biases,
                           int64_t N, int64_t K, int64_t G, double* out) {
    const int64_t ng = K / G;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            double s = (double)or_bf16_to_f32(scales[n * ng + k / G]);
            double b = (double)or_bf16_to_f32(biases[n * ng + k / G]);
            out[n * K + k] = (double)affine_code(wq, K, n, k) * s + b;
        }
}

/* Dequantise to binary16 (half_kind 0) or bfloat16 (1): the binary32 value
 * nearest to q*s + b, then rounded to nearest even into the 16-bit type. */
void or_affine4_dequantize_half(const uint8_t* wq, const uint16_t* scales, const uint16_t* biases,
                                int64_t N, int64_t K, int64_t G, int half_kind, uint16_t* out) {
    const int64_t ng = K / G;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            double s = (double)or_bf16_to_f32(scales[n * ng + k / G]);
            double b = (double)or_bf16_to_f32(biases[n * ng + k / G]);
            float v = (float)((double)affine_code(wq, K, n, k) * s + b);
            out[n * K + k] = half_kind ? or_f32_to_bf16(v) : or_f32_to_f16(v);
        }
}

/* ------------------------------------------------------------------------ */
/* Affine 8-bit, group G: the same min/max rule with 255 steps, one code per */
/* byte (byte k of a row is element k).  The MLX page measures quantize /   */
/* dequantize / quantized_matmul at bits = 4 and bits = 8 (Repro); the rule  */
/* is read exactly as for 4 bits above.                                      */
/* ------------------------------------------------------------------------ */
void or_affine8_quantize(const uint16_t* wbf, int64_t N, int64_t K, int64_t G,
                         uint8_t* wq, uint16_t* scales, uint16_t* biases) {
    const int64_t ng = K / G;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < ng; g++) {
            const uint16_t* grp = wbf + n * K + g * G;
            float lo = or_bf16_to_f32(grp[0]), hi = lo;
            for (int64_t j = 1; j < G; j++) {
                float v = or_bf16_to_f32(grp[j]);
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            lo = lo + 0.0f;   /* -0 -> +0 */
            hi = hi + 0.0f;
            float step32 = (hi - lo) / 255.0f;
            uint16_t sb = or_f32_to_bf16(step32);
            uint16_t bb = or_f32_to_bf16(lo);
            float sf = or_bf16_to_f32(sb), bf = or_bf16_to_f32(bb);
            scales[n * ng + g] = sb;
            biases[n * ng + g] = bb;
            for (int64_t j = 0; j < G; j++) {
                int code = 0;
                if (sf != 0.0f) {
                    float t = (or_bf16_to_f32(grp[j]) - bf) / sf;
                    float f8 = floorf(t + 0.5f);
                    code = f8 < 0.0f ? 0 : (f8 > 255.0f ? 255 : (int)f8);
                }
                wq[n * K + g * G + j] = (uint8_t)code;
            }
        }
}

/* Exact dequantised 8-bit weights: w^ = q*s + b in binary64. */
void or_affine8_dequantize(const uint8_t* wq, const uint16_t* scales, const uint16_t* biases,
                           int64_t N, int64_t K, int64_t G, double* out) {
    const int64_t ng = K / G;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            double sv = (double)or_bf16_to_f32(scales[n * ng + k / G]);
            double bv = (double)or_bf16_to_f32(biases[n * ng + k / G]);
            out[n * K + k] = (double)wq[n * K + k] * sv + bv;
        }
}

/* 8-bit codes to binary16 (half_kind 0) or bfloat16 (1): the binary32 value
 * nearest to q*s + b, then rounded to nearest even into the 16-bit type. */
void or_affine8_dequantize_half(const uint8_t* wq, const uint16_t* scales, const uint16_t* biases,
                                int64_t N, int64_t K, int64_t G, int half_kind, uint16_t* out) {
    const int64_t ng = K / G;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            double sv = (double)or_bf16_to_f32(scales[n * ng + k / G]);
            double bv = (double)or_bf16_to_f32(biases[n * ng + k / G]);
            float v = (float)((double)wq[n * K + k] * sv + bv);
            out[n * K + k] = half_kind ? or_f32_to_bf16(v) : or_f32_to_f16(v);
        }
}

/* Helpers for the Python side. */
void or_f32_to_f16_array(const float* in, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = or_f32_to_f16(in[i]);
}
void or_f16_to_f32_array(const uint16_t* in, int64_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = or_f16_to_f32(in[i]);
}
void or_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = or_f32_to_bf16(in[i]);
}
void or_bf16_to_f32_array(const uint16_t* in, int64_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = or_bf16_to_f32(in[i]);
}

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
