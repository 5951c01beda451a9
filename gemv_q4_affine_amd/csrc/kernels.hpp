// kernels.hpp -- launchers of the gfx950 kernels, called by the C ABI layer
// (capi.cpp) after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// dtype codes (same values as Q4_F32 / Q4_BF16 / Q4_F16 in include/q4.h)
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// Compute units of the current device (queried once per device; 256 if the
// query fails).
int current_cu_count();

// Q4_0 x Q8_1 on the int8 matrix cores (gemm_q8.hip): y [M][N] of ydt.
hipError_t launch_gemm_q8(const uint8_t* wqs, const uint16_t* wd, const int8_t* xqs, const uint16_t* xds, void* y,
                          int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s);

// Device address of the current GPU's copy of the library's fixed scratch
// array (Q4_NOALLOC_SCRATCH_BYTES), looked up once per device (noalloc.hip).
hipError_t noalloc_scratch(void** out);

hipError_t launch_q4_quantize(const void* w, int wdt, int64_t N, int64_t K, uint8_t* qs, uint16_t* d,
                              hipStream_t s);
hipError_t launch_q8_1_quantize(const void* x, int xdt, int64_t M, int64_t K, int8_t* qs, uint16_t* ds,
                                hipStream_t s);
hipError_t launch_affine4_quantize(const void* w, int wdt, int64_t N, int64_t K, int64_t G, uint8_t* wq,
                                   uint16_t* sc, uint16_t* bi, hipStream_t s);
hipError_t launch_q4_dequantize(const uint8_t* qs, const uint16_t* d, int64_t N, int64_t K, void* out, int odt,
                                hipStream_t s);
hipError_t launch_affine4_dequantize(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, int64_t G,
                                     int64_t N, int64_t K, void* out, int odt, hipStream_t s);

// Affine 8-bit, group 64 (affine8.hip): quantiser, dequantiser, and the fused
// GEMV for 1 <= M <= kAffine8GemvMaxM.
constexpr int kAffine8GemvMaxM = 16;
hipError_t launch_affine8_quantize(const void* w, int wdt, int64_t N, int64_t K, uint8_t* wq, uint16_t* sc,
                                   uint16_t* bi, hipStream_t s);
hipError_t launch_affine8_dequantize(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, int64_t N, int64_t K,
                                     void* out, int odt, hipStream_t s);
hipError_t launch_affine8_gemv(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, const void* x, int xdt,
                               void* y, int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s);
// bf16-MFMA kernel for 1 <= M <= kAffine8MmaMaxM on a bf16 activation.
constexpr int kAffine8MmaMaxM = 32;
hipError_t launch_affine8_mma(const uint8_t* wq, const uint16_t* sc, const uint16_t* bi, const void* x, void* y,
                              int ydt, int64_t M, int64_t N, int64_t K, hipStream_t s);

// Decode GEMV over 1..kGemvMats weight matrices sharing one activation: the
// Q8_1 planes (x == nullptr), or a raw bf16 / f32 activation x quantised to
// Q8_1 inside the kernel (the same bits; M <= 4).  Host arrays of nmat
// entries; matrices with n == 0 are skipped.
constexpr int kGemvMats = 4;
hipError_t launch_q4_gemv_multi(int nmat, const uint8_t* const* qs, const uint16_t* const* d, const int64_t* n,
                                float* const* y, const int8_t* x_qs, const uint16_t* x_ds, const void* x, int xdt,
                                int64_t M, int64_t K, hipStream_t s);

// GEMM paths.  fmt: 0 = Q4_0 planes (a = qs, b = d), 1 = affine (a = q,
// b = scales, c = biases), 2 = dense binary16 W (a = w).
enum : int { WF_Q4_0 = 0, WF_AFFINE4 = 1, WF_DENSE16 = 2, WF_AFFINE8 = 3 };

hipError_t launch_gemm_mfma(int wfmt, const void* a, const void* b, const void* c,
                            const void* x, int xdt, void* y, int ydt,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
// Large-M quantised GEMM on packed images: converts X into a binary16 tile
// image and the weights into a tile image, both in `img` (16-byte aligned),
// then multiplies.  `img` holds x_image_bytes(M, K) + weight_image_bytes(N, K)
// bytes; with `split` it holds packed_x_bytes(M, N, K), which adds the
// split-K partial results a small tile count asks for.
int64_t packed_x_bytes(int64_t M, int64_t N, int64_t K);
// fp32 partial results of a K-split launch (0: no split for this shape).
int64_t splitk_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_packed(int wfmt, const void* a, const void* b, const void* c,
                              const void* x, int xdt, void* y, int ydt,
                              int64_t M, int64_t N, int64_t K, void* img, bool split, hipStream_t s);
// The two halves of it: the weight image alone (weight_image_bytes(N, K),
// kept by the caller across calls), and the GEMM on a weight image with the
// X image in ximg (x_image_bytes(M, K)) and, if part is not null, the
// split-K partial results in part (splitk_bytes(M, N, K)).
int64_t x_image_bytes(int64_t M, int64_t K);
// The row exponent table inside an X image of x_image_bytes(M, K) bytes.
const int8_t* x_image_exponents(const void* ximg, int64_t M, int64_t K);
int64_t weight_image_bytes(int64_t N, int64_t K);
hipError_t launch_pack_weight_image(int wfmt, const void* a, const void* b, const void* c, int64_t N, int64_t K,
                                    void* wimg, hipStream_t s);
hipError_t launch_gemm_image(int wfmt, const void* wimg, const void* x, int xdt, void* y, int ydt, int64_t M,
                             int64_t N, int64_t K, void* ximg, float* part, hipStream_t s);
// Affine 8-bit weights (codes [N][K], group-64 bf16 scales and biases) on
// the same matrix-core GEMM: the weight image (weight_image8_bytes(N, K)) and
// the X image in `img`, which holds affine8_packed_bytes(M, N, K) bytes with
// the split-K partial results (`split`), or x_image_bytes(M, K) +
// weight_image8_bytes(N, K) without them.  K % 64 == 0.
int64_t weight_image8_bytes(int64_t N, int64_t K);
int64_t affine8_packed_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_affine8_gemm_packed(const uint8_t* wq, const uint16_t* scales, const uint16_t* biases, const void* x,
                                      int xdt, void* y, int ydt, int64_t M, int64_t N, int64_t K, void* img, bool split,
                                      hipStream_t s);
// The 256 x 256-tile matrix-core GEMM (gemm_big.hip) on the X and weight
// images, for launches with at least one such tile per CU
// (gemm_big_applies); use_big_tiles adds the dispatch setting
// (Q4_KEY_TILE_ROWS) that can turn it off.  It needs no scratch.
bool gemm_big_applies(int64_t M, int64_t N, int64_t K);
bool use_big_tiles(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_big(int wfmt, const void* wimg, const void* ximg, void* y, int ydt, int64_t M, int64_t N,
                           int64_t K, hipStream_t s);
hipError_t launch_gemm_skinny(int wfmt, const void* a, const void* b, const void* c,
                              const void* x, int xdt, void* y, int ydt,
                              int64_t M, int64_t N, int64_t K, hipStream_t s);

}  // namespace q4
