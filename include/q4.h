/*
 * q4.h -- C ABI of the MI355X (gfx950) library for matrix multiply against
 * 4-bit block-quantised weights:
 *
 *     Y[M,N] = X[M,K] . dequant(Wq)[N,K]^T
 *
 * W is stored [N,K] (rows are output features), the transpose=True
 * convention of MLX's quantized_matmul (MLX issue #4621 "quantized_matmul
 * takes 14-41% longer than dequantize + bf16 matmul at prefill sizes",
 * Repro).  Two weight formats:
 *
 *   Q4_0 (GGUF block; named by llama.cpp PR "et-backend: Q4_0 matrix-engine
 *   GEMM rewrite for prefill", Overview, and by "2026-05-06 Q4 sync-after
 *   focused repro", Important source touch points):
 *     blocks of 32 weights along K; a binary16 scale d and 16 bytes of
 *     nibbles; w^ = (q - 8) * d.  Passed as two planes (structure of arrays):
 *       w_qs : uint8  [N][K/32][16]   byte i = q_i | q_{i+16} << 4
 *       w_d  : uint16 [N][K/32]       binary16 bit patterns
 *
 *   Affine 4-bit, group 64 (MLX quantize / dequantize, same MLX page, Repro):
 *     w^ = q * s + b, q unsigned 4-bit, s and b bfloat16, one pair per group.
 *       w_q    : uint8  [N][K/2]       byte i = q_{2i} | q_{2i+1} << 4
 *       scales : uint16 [N][K/G]       bfloat16 bit patterns
 *       biases : uint16 [N][K/G]       bfloat16 bit patterns
 *
 *   Q8_1 activations (the q4_0 x q8_1 decode kernels and Q8 cache of the
 *   repro page, Important source touch points / Quality-cleared launch
 *   recipe): blocks of 32 along K, d = max|x|/127, q = round(x/d),
 *   s = d * sum(q), as two planes:
 *       x_qs : int8   [M][K]
 *       x_ds : uint16 [M][K/32][2]    {binary16 d, binary16 s}
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller (hipMalloc'd
 *     or framework-allocated), contiguous row-major, no strides.  The library
 *     never frees, keeps or allocates them.
 *   - Plane pointers must be 16-byte aligned (Q4_ERR_ALIGN otherwise).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue kernels on it: no device synchronisation, no host<->device
 *     copy and no allocation, so they may be captured into a HIP graph.
 *   - Every argument is validated on the host before any HIP call; a failed
 *     check returns its status code and enqueues nothing.
 *   - M == 0 or N == 0 is a no-op that returns Q4_OK once the sizes and dtype
 *     codes are valid; the pointers are not looked at then (empty tensors may
 *     have NULL data pointers).
 *   - K must be a positive multiple of 32 (Q4_0 / Q8_1) or of the group size
 *     (affine).  N and K are limited to 2^30, M to 2^30.
 *   - Outputs of float type are not bit-reproducible against other
 *     summation orders, but every call is deterministic: the same inputs
 *     give the same bits (no atomics, fixed reduction order).
 *   - Thread-safety: calls on different streams may run concurrently; the
 *     dispatch settings (q4_set_dispatch) are process-wide.
 */
#ifndef GEMV_Q4_AFFINE_AMD_Q4_H
#define GEMV_Q4_AFFINE_AMD_Q4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define Q4_OK            0
#define Q4_ERR_NULL     -1   /* a required pointer is NULL                     */
#define Q4_ERR_SHAPE    -2   /* M/N/K out of range or not a block multiple      */
#define Q4_ERR_ALIGN    -3   /* a plane pointer is not 16-byte aligned          */
#define Q4_ERR_DTYPE    -4   /* unsupported dtype code                          */
#define Q4_ERR_HIP      -5   /* a HIP launch or runtime call failed             */
#define Q4_ERR_ARG      -6   /* other invalid argument (dispatch key, path...)  */
#define Q4_ERR_WORKSPACE -7  /* a path that needs workspace got too little */
#define Q4_ERR_SCRATCH  -8   /* the call needs more than Q4_NOALLOC_SCRATCH_BYTES */

/* ---- dtype codes ---------------------------------------------------------- */
#define Q4_F32   0
#define Q4_BF16  1
#define Q4_F16   2

/* ---- formats and dispatch paths ------------------------------------------- */
#define Q4_FMT_Q4_0     0
#define Q4_FMT_AFFINE4  1
#define Q4_FMT_AFFINE8  2  /* the paths and workspace of affine8_gemm, and the
                              weight-image calls */

#define Q4_PATH_GEMV          0  /* integer-dot GEMV on Q8_1 activations (q4_gemv)     */
#define Q4_PATH_SKINNY        1  /* fused, weights streamed once, small M              */
#define Q4_PATH_MFMA          2  /* fused dequant-in-LDS MFMA GEMM, large M             */
#define Q4_PATH_DEQUANT_GEMM  3  /* dequantise to a dense fp16 W, then dense MFMA GEMM  */
#define Q4_PATH_INT8          4  /* X quantised to Q8_1, int8 MFMA GEMM (q4_gemm_q8)     */

/* dispatch keys for q4_set_dispatch / q4_get_dispatch */
#define Q4_KEY_SKINNY_MAX_M    0  /* q4_gemm/affine4_gemm: M <= this -> SKINNY (default
                                     64; with binary32 X the automatic choice takes
                                     MFMA above 16 rows when the workspace holds the
                                     MFMA images, above 32 rows otherwise; with
                                     bfloat16 X and no room for the images, an
                                     automatic MFMA choice up to 128 rows runs the
                                     SKINNY row chunks while this is 64)               */
#define Q4_KEY_DEQUANT_MIN_M   1  /* M >= this (and workspace given) -> DEQUANT_GEMM    */
#define Q4_KEY_FORCE_PATH      2  /* -1 = automatic, else a Q4_PATH_* for q4_gemm etc.;
                                     GEMV and INT8 compute on X quantised to Q8_1 and
                                     serve Q4_0 only (q4_gemm: GEMV needs M <= 4 and an
                                     f32 y, INT8 a workspace of M*K + M*(K/32)*4 bytes;
                                     other cases return Q4_ERR_ARG)                      */
#define Q4_KEY_TILE_ROWS       3  /* MFMA path: 128 = 128x256 output tiles (default),
                                     256 = 256x256 tiles where every CU gets at least one */
#define Q4_KEY_AFFINE8_FUSED_MAX_M 4 /* affine8_gemm: M <= this (0..32) -> the fused
                                     kernels (SKINNY), above -> MFMA; f32 X above
                                     16 rows always takes MFMA                        */

/* Largest M that q4_gemv / q4_gemv_fused2 accept. */
#define Q4_GEMV_MAX_M 16

/* ======================================================================== */
/* Quantisers                                                                */
/* ======================================================================== */

/*
 * q4_quantize -- Q4_0-quantise a weight matrix (one-time weight preparation).
 * Defines (reading of the GGUF Q4_0 block; the pages name the format but do
 * not print the rule): per block of 32 weights along K, max = the first
 * weight of largest magnitude (signed), d = max / -8 (binary32),
 * q_j = min(15, floor(w_j * (1/d) + 8.5)) with separate binary32 multiply and
 * add (q = 8 for an all-zero block), stored d = binary16(d) (RNE; an
 * all-zero block stores -0.0).  Bit-exact, deterministic.
 *   w       : device, [N][K] of w_dtype (Q4_F32 or Q4_BF16)
 *   w_qs    : device out, uint8 [N][K/32][16]
 *   w_d     : device out, uint16 [N][K/32]
 * Errors: NULL, SHAPE (K % 32, sizes), ALIGN, DTYPE, HIP.
 * Inputs must be finite; blocks whose largest magnitude lies in (0, 2^-125)
 * are outside the domain (1/d overflows binary32).
 */
int q4_quantize(const void* w, int w_dtype, int64_t N, int64_t K,
                uint8_t* w_qs, uint16_t* w_d, void* stream);

/*
 * q8_1_quantize_act -- quantise activations to Q8_1 once per token, for reuse
 * by every GEMV that reads them (the Q8 cache of the repro page,
 * Quality-cleared launch recipe).  Per block of 32: amax = max|x|,
 * d = amax/127, q = round-half-away(x * (1/d)), s = binary16(d * sum q),
 * d stored as binary16 (binary32 arithmetic throughout).  Bit-exact.
 *   x       : device, [M][K] of x_dtype (Q4_F32 or Q4_BF16)
 *   x_qs    : device out, int8 [M][K]
 *   x_ds    : device out, uint16 [M][K/32][2] = {d, s}
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP.
 */
int q8_1_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K,
                      int8_t* x_qs, uint16_t* x_ds, void* stream);

/*
 * affine4_quantize -- affine 4-bit quantisation (MLX quantize with bits=4;
 * the page shows the API only, the rule is the min/max reading): per group of
 * G weights (bfloat16, or binary32 first rounded to bfloat16): mn/mx = group
 * min/max (a zero extreme taken as +0), s = bfloat16((mx - mn)/15),
 * b = bfloat16(mn), q = clamp(floor((w - b)/s + 0.5), 0, 15) in binary32
 * (q = 0 when s == 0).  Bit-exact.
 *   w          : device, [N][K] of w_dtype (Q4_BF16 or Q4_F32)
 *   group_size : 64 (other values: Q4_ERR_SHAPE)
 *   w_q        : device out, uint8 [N][K/2]
 *   scales, biases : device out, uint16 [N][K/group_size] (bfloat16 bits)
 */
int affine4_quantize(const void* w, int w_dtype, int64_t N, int64_t K, int64_t group_size,
                     uint8_t* w_q, uint16_t* scales, uint16_t* biases, void* stream);

/* ======================================================================== */
/* Dequantisers (the dequantise-then-GEMM path of the MLX page, Summary and  */
/* Effect on a model)                                                        */
/* ======================================================================== */

/*
 * q4_dequantize -- dense W^ [N][K] = (q - 8) * d rounded to out_dtype:
 * binary16 or bfloat16 (RNE of the exact binary32 value), or binary32 (exact).
 *   out : device out, [N][K] of out_dtype (Q4_F16, Q4_BF16 or Q4_F32)
 */
int q4_dequantize(const uint8_t* w_qs, const uint16_t* w_d, int64_t N, int64_t K,
                  void* out, int out_dtype, void* stream);

/*
 * affine4_dequantize -- dense W^ = q*s + b: the binary32 value nearest the
 * exact one, then RNE into out_dtype (Q4_F16, Q4_BF16 or Q4_F32).
 */
int affine4_dequantize(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases,
                       int64_t group_size, int64_t N, int64_t K,
                       void* out, int out_dtype, void* stream);

/* ======================================================================== */
/* Decode GEMV (M small): integer block dots on Q8_1 activations             */
/* ======================================================================== */

/*
 * q4_gemv -- y[m][n] = sum_b d4[n][b] * d8[m][b] * isum[m][n][b], with the
 * exact int32 block dot isum = sum_{j<32} (q4_j - 8) * q8_j, scaled and
 * accumulated in binary32 (the decode "vecdot" route of the ET-SoC-1 PR,
 * Overview; the q4_0 x q8_1 mul_mat_vec_q kernel of the repro page,
 * Important source touch points).
 *   w_qs, w_d : device, Q4_0 planes of W [N][K]
 *   x_qs, x_ds: device, Q8_1 planes of X [M][K] (from q8_1_quantize_act)
 *   y         : device out, float [M][N]
 *   1 <= M <= Q4_GEMV_MAX_M (else Q4_ERR_SHAPE; M == 0 is a no-op).
 */
int q4_gemv(const uint8_t* w_qs, const uint16_t* w_d,
            const int8_t* x_qs, const uint16_t* x_ds,
            float* y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * q4_gemv_fused2 -- two GEMVs that share one Q8_1 activation (gate+up, or
 * K+V), in one launch that reads the activation once (the fused2 MMVQ kernel
 * of the repro page, Important source touch points).  N0 != N1 is allowed.
 * Results are bit-identical to two q4_gemv calls.
 *   y0 : device out, float [M][N0];  y1 : device out, float [M][N1]
 */
int q4_gemv_fused2(const uint8_t* w0_qs, const uint16_t* w0_d, int64_t N0,
                   const uint8_t* w1_qs, const uint16_t* w1_d, int64_t N1,
                   const int8_t* x_qs, const uint16_t* x_ds,
                   float* y0, float* y1, int64_t M, int64_t K, void* stream);

/*
 * q4_gemv_act -- q4_gemv on a raw activation: the kernel quantises each X
 * block to Q8_1 in registers where it is consumed, with the arithmetic of
 * q8_1_quantize_act, so y is bit-identical to q8_1_quantize_act followed by
 * q4_gemv, in one launch and without the Q8_1 planes in HBM (the decode step
 * of the repro page, Important source touch points: quantise the activation,
 * then the MMVQ GEMV).
 *   x       : device, [M][K] of x_dtype (Q4_BF16 or Q4_F32), 16-byte aligned
 *   y       : device out, float [M][N]
 *   1 <= M <= Q4_GEMV_ACT_MAX_M (else Q4_ERR_SHAPE; M == 0 is a no-op).
 */
#define Q4_GEMV_ACT_MAX_M     4
int q4_gemv_act(const uint8_t* w_qs, const uint16_t* w_d,
                const void* x, int x_dtype,
                float* y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * q4_gemv_fused2_act -- q4_gemv_fused2 on a raw activation, quantised inside
 * the kernel as in q4_gemv_act: bit-identical to q8_1_quantize_act followed by
 * q4_gemv_fused2.  Same limits as q4_gemv_act.
 */
int q4_gemv_fused2_act(const uint8_t* w0_qs, const uint16_t* w0_d, int64_t N0,
                       const uint8_t* w1_qs, const uint16_t* w1_d, int64_t N1,
                       const void* x, int x_dtype,
                       float* y0, float* y1, int64_t M, int64_t K, void* stream);

/*
 * q4_gemv_multi / q4_gemv_multi_act -- up to Q4_GEMV_MAX_MATS matrices (q, k
 * and v; gate and up; or any set) that share one activation, in one launch
 * that reads the activation once: the fused MMVQ kernel of the repro page
 * (Important source touch points) taken from two matrices to several.
 * Results are bit-identical to one q4_gemv (q4_gemv_act) call per matrix.
 *   nmat        : 1 .. Q4_GEMV_MAX_MATS (else Q4_ERR_ARG)
 *   w_qs, w_d, y: host arrays of nmat device pointers; n: host array of the
 *                 nmat row counts (a matrix with n[i] == 0 is skipped, and its
 *                 pointers may be NULL)
 *   y[i]        : device out, float [M][n[i]]
 * The activation and M limits are those of q4_gemv (Q8_1 planes) and
 * q4_gemv_act (raw activation); the rows of all matrices together must fit
 * in 2^31 - 1.
 */
#define Q4_GEMV_MAX_MATS 4
int q4_gemv_multi(int nmat, const uint8_t* const* w_qs, const uint16_t* const* w_d, const int64_t* n,
                  const int8_t* x_qs, const uint16_t* x_ds, float* const* y,
                  int64_t M, int64_t K, void* stream);
int q4_gemv_multi_act(int nmat, const uint8_t* const* w_qs, const uint16_t* const* w_d, const int64_t* n,
                      const void* x, int x_dtype, float* const* y,
                      int64_t M, int64_t K, void* stream);

/* ======================================================================== */
/* GEMM (any M): bf16 / f32 activations                                      */
/* ======================================================================== */

/*
 * q4_gemm -- Y = X . dequant(Wq)^T for Q4_0 weights, fp32 accumulation
 * (the prefill matrix-engine GEMM of the ET-SoC-1 PR, Overview).  The M
 * dispatch (q4_dispatch_path) picks SKINNY, MFMA or DEQUANT_GEMM.  The fused
 * paths multiply on the matrix cores in binary16, with the weights
 * dequantised to binary16 (relative rounding <= 2^-11) and X converted to
 * binary16 by round to nearest even:
 *   - the MFMA path with its X image (a workspace of at least the two tile
 *     images, and q4_gemm_image) first scales each X row by a power of two
 *     2^e that brings the row's largest |x| into [2^14, 2^15), and scales the
 *     row's fp32 results back by 2^-e: the whole bfloat16 / binary32 range is
 *     in its domain, and bfloat16 values within a factor 2^31 of their row's
 *     largest convert exactly;
 *   - the paths without an X image (SKINNY with binary32 X, MFMA with too
 *     little workspace, DEQUANT_GEMM) convert X directly: exact for bfloat16
 *     values with 2^-17 <= |x| <= 65504; |x| > 65504 becomes +-inf.  The SKINNY
 *     path with bfloat16 X (2 <= M <= 64; above 32 rows on row chunks of at
 *     most 32; up to 128 rows when the MFMA path has no room for its images)
 *     multiplies in bfloat16 and has the whole range.
 *   x         : device, [M][K] of x_dtype (Q4_BF16 or Q4_F32)
 *   y         : device out, [M][N] of y_dtype (Q4_BF16 RNE, or Q4_F32)
 *   workspace : device scratch owned by the caller (16-byte aligned), or
 *               NULL.  q4_gemm_workspace_size bytes let the call take its
 *               fastest path.  The MFMA path uses them for tile images of X
 *               (binary16) and of the weights (the same Q4_0 / affine blocks,
 *               regrouped per 256-column tile and 64-wide K step) that its
 *               matrix-core kernel copies straight into LDS, and, when the
 *               output has too few 128x256 tiles to occupy the GPU, for the
 *               fp32 partial results of a K-split (each tile's K range spread
 *               over up to 16 workgroups, the parts then summed in order:
 *               deterministic, rounding order differs from an unsplit call).
 *               Room for the two images but not the partial results runs the
 *               same kernel unsplit; less than the images converts X inside
 *               the GEMM (slower, results within the same bound).  The DEQUANT_GEMM path needs N*K*2 bytes for the
 *               dequantised weights: the automatic dispatch picks it only
 *               with that much, and forcing it without returns
 *               Q4_ERR_WORKSPACE.  Calls that share a workspace must not run
 *               concurrently.
 */
int q4_gemm(const uint8_t* w_qs, const uint16_t* w_d,
            const void* x, int x_dtype, void* y, int y_dtype,
            int64_t M, int64_t N, int64_t K,
            void* workspace, int64_t workspace_bytes, void* stream);

/*
 * affine4_gemm -- Y = X . dequant(Wq)^T for affine 4-bit group-64 weights
 * (MLX quantized_matmul with transpose=True, bits=4, group_size=64; MLX page,
 * Repro).  Same dispatch, precision and workspace rules as q4_gemm.
 *   group_size : 64 only (else Q4_ERR_SHAPE)
 */
int affine4_gemm(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases,
                 int64_t group_size, const void* x, int x_dtype, void* y, int y_dtype,
                 int64_t M, int64_t N, int64_t K,
                 void* workspace, int64_t workspace_bytes, void* stream);

/* ======================================================================== */
/* Affine 8-bit, group 64 (MLX quantize / dequantize / quantized_matmul with  */
/* bits=8: the MLX page's Repro runs bits 4 and 8, and its Summary finds the  */
/* fused kernel ahead at decode sizes and dequantise-then-matmul ahead from   */
/* 512 tokens at both widths)                                                 */
/* ======================================================================== */

/*
 * affine8_quantize -- affine 8-bit quantisation, the affine4_quantize rule
 * with 255 steps: s = bfloat16((mx - mn)/255), b = bfloat16(mn),
 * q = clamp(floor((w - b)/s + 0.5), 0, 255) in binary32 (q = 0 when s == 0).
 * Bit-exact.
 *   w          : device, [N][K] of w_dtype (Q4_BF16 or Q4_F32)
 *   group_size : 64 (other values: Q4_ERR_SHAPE); K % 64 == 0
 *   w_q        : device out, uint8 [N][K], byte k of a row = element k
 *   scales, biases : device out, uint16 [N][K/64] (bfloat16 bits)
 */
int affine8_quantize(const void* w, int w_dtype, int64_t N, int64_t K, int64_t group_size,
                     uint8_t* w_q, uint16_t* scales, uint16_t* biases, void* stream);

/*
 * affine8_dequantize -- dense W^ = q*s + b: the binary32 value nearest the
 * exact one (one fma), then RNE into out_dtype (Q4_F16, Q4_BF16 or Q4_F32).
 */
int affine8_dequantize(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases,
                       int64_t group_size, int64_t N, int64_t K,
                       void* out, int out_dtype, void* stream);

/*
 * affine8_gemm -- Y = X . dequant(Wq)^T for affine 8-bit group-64 weights
 * (quantized_matmul with transpose=True, bits=8, group_size=64).
 * Paths (q4_dispatch_path with Q4_FMT_AFFINE8): SKINNY up to
 * Q4_KEY_AFFINE8_FUSED_MAX_M rows (default 32: the fused kernels below),
 * MFMA above it; Q4_KEY_FORCE_PATH = SKINNY, MFMA or DEQUANT_GEMM forces
 * one of them, other forced values leave the automatic choice.  On SKINNY:
 *   M <= 4 (and M <= 16 on a Q4_F32 activation): one fused launch, no
 *     workspace: each weight is dequantised once in binary32 (q*s + b, one
 *     fma) and multiplied with the M rows in binary32.
 *   5 <= M <= 32 on a Q4_BF16 activation: one fused launch, no workspace:
 *     the bf16 matrix cores multiply X with the raw codes (exact in
 *     bfloat16) per 64-weight group, and s and b scale the group's sums in
 *     binary32.  Both fused kernels sum in an order that depends on K only.
 *   Otherwise (and on MFMA): the matrix-core GEMM of q4_gemm's MFMA path
 *     on a weight image of 17408 bytes per 256 columns and 64 K (the codes
 *     and the group's s and b, dequantised in registers to binary16 as
 *     (q + 1024 - 1024) * s + b with one rounding) and the X image, both
 *     in the workspace: at least ceil(M/128)*128 * (K*2 + 1) +
 *     ceil(N/256) * (K/64) * 17408 bytes, 16-byte aligned (less:
 *     Q4_ERR_WORKSPACE), plus parts*M*N*4 for split-K partial results when
 *     the tile count is small (without that room K is not split).
 *   DEQUANT_GEMM (forced only): the weights are dequantised to binary16 in
 *     the workspace (at least N*K*2 bytes), then the dense binary16 GEMM of
 *     dense_gemm runs on them.
 *   affine8_gemm_workspace_size(M, N, K) is 0 for M <= 16 and the size the
 *   path needs above (enough for either activation type).
 *   x : device, [M][K] of x_dtype (Q4_BF16 or Q4_F32); y : device out, [M][N]
 *   of y_dtype (Q4_BF16 RNE, or Q4_F32).  group_size 64 only, K % 64 == 0.
 *   Calls that share a workspace must not run concurrently.
 */
int64_t affine8_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
int affine8_gemm(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases,
                 int64_t group_size, const void* x, int x_dtype, void* y, int y_dtype,
                 int64_t M, int64_t N, int64_t K,
                 void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Bytes of workspace for the path q4_dispatch_path(M, N, K, fmt, 1) picks:
 * 0 for SKINNY and GEMV (but an automatic SKINNY choice above 16 rows asks
 * for the MFMA bytes below: given them, binary32 X takes the MFMA path there;
 * bfloat16 X uses none of them); M*K + M*(K/32)*4 (the Q8_1 planes of X) for INT8;
 * for MFMA the X and weight tile images,
 * ceil(M/128)*128 * (ceil(K/64)*64 * 2 + 1) + ceil(N/256) * ceil(K/64) * 9216
 * bytes (the X image holds one exponent byte per row after its tiles),
 * plus parts*M*N*4 for the K-split partial results when the tile count is
 * below half the device's CU count (parts: the most, up to 16, that divide
 * ceil(K/64), leave at least 4 K steps each and keep tiles*parts within the
 * CU count); for DEQUANT_GEMM N*K*2 (a dense binary16 W).  fmt
 * Q4_FMT_AFFINE8: affine8_gemm_workspace_size(M, N, K).
 * Returns 0 for invalid arguments.
 */
int64_t q4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int fmt);

/*
 * Weight image for the matrix-core GEMM, prepared once per weight matrix:
 * the MFMA path's per-call weight regrouping (q4_gemm with a workspace) moved
 * out of the call, for callers that multiply the same weights many times
 * (prefill over many prompts).  The dequantisation itself stays fused in the
 * GEMM: the image holds the same 4.5 bits per weight as the planes.
 *
 * q4_weight_image_size -- bytes of the image of an [N][K] matrix,
 * ceil(N/256) * ceil(K/64) * 9216 (Q4_0, affine 4-bit) or
 * ceil(N/256) * (K/64) * 17408 (affine 8-bit); 0 for invalid arguments.
 */
int64_t q4_weight_image_size(int64_t N, int64_t K, int fmt);

/*
 * q4_pack_weight_image -- lay the weight planes out as that image.
 *   fmt   : Q4_FMT_Q4_0 (w_q = qs, w_s = d, w_b unused), Q4_FMT_AFFINE4 or
 *           Q4_FMT_AFFINE8 (w_q = codes, w_s = scales, w_b = biases, as
 *           affine4_quantize / affine8_quantize write them; group size 64)
 *   image : device out, q4_weight_image_size(N, K, fmt) bytes, 16-byte aligned
 * K % 32 == 0 (Q4_0) or K % 64 == 0 (affine), else Q4_ERR_SHAPE.
 */
int q4_pack_weight_image(int fmt, const uint8_t* w_q, const uint16_t* w_s, const uint16_t* w_b,
                         int64_t N, int64_t K, void* image, void* stream);

/*
 * q4_gemm_image -- Y = X . dequant(W)^T on the matrix-core path from a
 * weight image: the same results as q4_gemm / affine4_gemm / affine8_gemm
 * on the MFMA path with a workspace of the same size, for any M >= 1.
 *   workspace : device scratch for the X image, at least
 *               q4_gemm_image_workspace_size(M, K) =
 *               ceil(M/128)*128 * (ceil(K/64)*64 * 2 + 1) bytes (else
 *               Q4_ERR_WORKSPACE).  With room after it for the K-split
 *               partial results (q4_gemm_workspace_size(M, N, K, fmt) bytes
 *               are always enough), a launch with few tiles is split along
 *               K as in q4_gemm.  Calls sharing it must not overlap.
 */
int64_t q4_gemm_image_workspace_size(int64_t M, int64_t K);
int q4_gemm_image(int fmt, const void* image, const void* x, int x_dtype, void* y, int y_dtype,
                  int64_t M, int64_t N, int64_t K,
                  void* workspace, int64_t workspace_bytes, void* stream);

/* Size of the library's fixed device scratch (33 MiB per GPU). */
#define Q4_NOALLOC_SCRATCH_BYTES (33ll << 20)

/*
 * q4_gemm_image_noalloc -- q4_gemm_image for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * q4_gemm_image with a Q4_NOALLOC_SCRATCH_BYTES workspace, except that the
 * workspace is a fixed array inside the library: one per GPU, created when
 * the library's code is loaded on that GPU and held until the process ends.
 * The call allocates nothing and calls no allocating routine.
 *   Limit: q4_gemm_image_workspace_size(M, K) <= Q4_NOALLOC_SCRATCH_BYTES
 *          (e.g. M <= 4096 at K = 4096), else Q4_ERR_SCRATCH and nothing is
 *          enqueued.  Split-K partial results are used when they fit after
 *          the X image, as in q4_gemm_image.
 *   The scratch keeps the last call's contents; every byte a call reads is
 *   written earlier in the same call, so nothing needs clearing.  All calls on
 *   one GPU share that GPU's scratch: calls that can overlap (different
 *   streams, or host threads enqueueing concurrently) race and give wrong
 *   results; serialise them on one stream.
 */
int q4_gemm_image_noalloc(int fmt, const void* image, const void* x, int x_dtype, void* y, int y_dtype,
                          int64_t M, int64_t N, int64_t K, void* stream);

/*
 * q4_gemm_q8 -- y[m][n] = sum_b d4[n][b] * d8[m][b] * isum[m][n][b] for any M,
 * the integer-dot product of q4_gemv on the int8 matrix cores (the DP4A /
 * matrix-engine variant of the Q4_0 x Q8_1 kernel: trueno page,
 * KERNEL_WEIGHTS; the MMVQ pair of the llama.cpp SYCL repro page, Important
 * source touch points).  Each 32-weight block's int32 dots are exact
 * (v_mfma_i32_32x32x32_i8); each is scaled by the fp32 product d4*d8 (exact
 * for binary16 scales) with one fma into fp32 accumulators, in K order.
 *   w_qs, w_d   : Q4_0 planes as in q4_gemv
 *   x_qs, x_ds  : Q8_1 planes as q8_1_quantize_act writes them, [M][K] and
 *                 [M][K/32][2]
 *   y           : device out, [M][N] of y_dtype (Q4_BF16 RNE, or Q4_F32)
 * The per-block rescale is vector-ALU work (a convert, a multiply and an fma
 * per output and block) that the binary16 MFMA path does not have; q4_gemm
 * takes this path only when Q4_KEY_FORCE_PATH is Q4_PATH_INT8.
 */
int q4_gemm_q8(const uint8_t* w_qs, const uint16_t* w_d, const int8_t* x_qs, const uint16_t* x_ds,
               void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * dense_gemm -- Y = X . W^T with a dense binary16 W [N][K] (the GEMM half of
 * dequantise-then-GEMM; MLX page, Repro "jit"/"ref" timings).  Same MFMA
 * tiles and X conversion as the fused paths.
 *   w_f16 : device, uint16 [N][K] binary16 bits
 */
int dense_gemm(const void* x, int x_dtype, const uint16_t* w_f16, void* y, int y_dtype,
               int64_t M, int64_t N, int64_t K, void* stream);

/* ======================================================================== */
/* Dispatch and housekeeping (host only, no HIP calls)                       */
/* ======================================================================== */

/*
 * q4_dispatch_path -- the path q4_gemm (fmt Q4_FMT_Q4_0), affine4_gemm
 * (Q4_FMT_AFFINE4) or affine8_gemm (Q4_FMT_AFFINE8) takes for this shape, given whether a large enough
 * workspace is supplied: Q4_PATH_SKINNY / Q4_PATH_MFMA / Q4_PATH_DEQUANT_GEMM,
 * or a negative status for invalid arguments.  Token-count thresholds follow
 * the pages' pattern (ET-SoC-1 PR Overview: one token goes to the vector-dot
 * kernel; MLX page, Effect on a model: dequantise-then-matmul only from a
 * token count up; vllm.cpp issue #838, Scope: a clamped token-count gate).
 * Defaults come from measurement; the environment variables
 * Q4_SKINNY_MAX_M, Q4_DEQUANT_MIN_M and Q4_FORCE_PATH, read once, override
 * them (clamped), and q4_set_dispatch overrides both.
 */
int q4_dispatch_path(int64_t M, int64_t N, int64_t K, int fmt, int have_workspace);

int q4_set_dispatch(int key, int64_t value);
int q4_get_dispatch(int key, int64_t* value);

/* Static text for a status code. */
const char* q4_status_string(int status);

/* Library version string. */
const char* q4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMV_Q4_AFFINE_AMD_Q4_H */
