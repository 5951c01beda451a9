// capi.cpp -- the exported C ABI (include/q4.h): argument validation, the
// M-threshold dispatch and the kernel launches.
//
// Every check runs on the host before any HIP call, so a rejected call
// enqueues nothing and the checks work on a machine without a GPU.
#include "q4.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "kernels.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;

// ---- dispatch settings -----------------------------------------------------
// Defaults come from the measured crossovers of this library on MI355X.
constexpr int64_t kSkinnyLimit = 64;          // the skinny kernel's largest M
std::atomic<int64_t> g_skinny_max_m{64};
// binary32 activations: the small-M kernels take bfloat16 X, and the binary32
// skinny kernel beats the matrix-core GEMM on its X and weight images only up
// to kF32SkinnyMaxM rows (without room for the images, the GEMM converting X
// in the kernel is slower than the skinny kernel up to kF32SkinnyNoImageMaxM
// rows), so an automatic SKINNY choice above those runs the matrix-core GEMM
constexpr int64_t kF32SkinnyMaxM = 16;
constexpr int64_t kF32SkinnyNoImageMaxM = 32;
// bfloat16 activations with no room for the matrix-core GEMM's images: the
// small-M kernel on 32-row chunks beats the GEMM converting X in the kernel
// up to this many rows (while the skinny range is left at its full width)
constexpr int64_t kBf16ChunkNoImageMaxM = 128;
std::atomic<int64_t> g_dequant_min_m{kMaxDim + 1};   // dequantise-then-GEMM never wins by default
std::atomic<int64_t> g_force_path{-1};
std::atomic<int64_t> g_tile_rows{128};
constexpr int64_t kAffine8FusedLimit = 32;     // the fused affine 8-bit kernels' largest M
std::atomic<int64_t> g_affine8_fused_max_m{kAffine8FusedLimit};
std::once_flag g_env_once;

int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

bool env_int(const char* name, int64_t* out) {
    const char* s = std::getenv(name);
    if (!s || !*s) return false;
    char* end = nullptr;
    long long v = std::strtoll(s, &end, 10);
    if (end == s) return false;
    *out = (int64_t)v;
    return true;
}

// Values Q4_KEY_FORCE_PATH accepts: automatic (-1), or a path q4_gemm /
// affine4_gemm can run.
bool force_path_ok(int64_t v) {
    return v == -1 || v == Q4_PATH_GEMV || v == Q4_PATH_SKINNY || v == Q4_PATH_MFMA || v == Q4_PATH_DEQUANT_GEMM ||
           v == Q4_PATH_INT8;
}

// Workspace of the INT8 path: the Q8_1 planes of X (codes, then {d, s} pairs).
int64_t q8_planes_bytes(int64_t M, int64_t K) { return M * K + M * (K / 32) * 4; }

// Environment overrides, read once per process and clamped (the clamped
// token-count gate pattern of vllm.cpp issue #838, Scope).
void read_env() {
    std::call_once(g_env_once, [] {
        int64_t v;
        if (env_int("Q4_SKINNY_MAX_M", &v)) g_skinny_max_m = clamp64(v, 0, kSkinnyLimit);
        if (env_int("Q4_DEQUANT_MIN_M", &v)) g_dequant_min_m = clamp64(v, 1, kMaxDim + 1);
        // the setter's rule: a value it would reject leaves the default
        if (env_int("Q4_FORCE_PATH", &v) && force_path_ok(v)) g_force_path = v;
        if (env_int("Q4_TILE_ROWS", &v) && (v == 128 || v == 256)) g_tile_rows = v;
        if (env_int("Q4_AFFINE8_FUSED_MAX_M", &v)) g_affine8_fused_max_m = clamp64(v, 0, kAffine8FusedLimit);
    });
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptrs_aligned(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p) return Q4_ERR_NULL;
    for (const void* p : ps)
        if (!aligned16(p)) return Q4_ERR_ALIGN;
    return Q4_OK;
}

int check_dims(int64_t M, int64_t N, int64_t K, int64_t kmult) {
    if (M < 0 || N < 0 || K <= 0) return Q4_ERR_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return Q4_ERR_SHAPE;
    if (K % kmult != 0) return Q4_ERR_SHAPE;
    return Q4_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

namespace q4 {

bool use_big_tiles(int64_t M, int64_t N, int64_t K) {
    read_env();
    return g_tile_rows == 256 && gemm_big_applies(M, N, K);
}

int current_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];   // 0: not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace q4

extern "C" {

const char* q4_status_string(int status) {
    switch (status) {
        case Q4_OK: return "ok";
        case Q4_ERR_NULL: return "a required pointer is NULL";
        case Q4_ERR_SHAPE: return "M, N or K out of range or not a multiple of the block/group size";
        case Q4_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case Q4_ERR_DTYPE: return "unsupported dtype";
        case Q4_ERR_HIP: return "HIP launch or runtime error";
        case Q4_ERR_ARG: return "invalid argument";
        case Q4_ERR_WORKSPACE: return "the workspace is missing or smaller than the path needs";
        case Q4_ERR_SCRATCH: return "the call needs more than the library's fixed scratch (Q4_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

const char* q4_version(void) { return "gemv_q4_affine_amd 0.1.0 (gfx950)"; }

// ---- dispatch ------------------------------------------------------------------

int q4_set_dispatch(int key, int64_t value) {
    read_env();
    switch (key) {
        case Q4_KEY_SKINNY_MAX_M: g_skinny_max_m = clamp64(value, 0, kSkinnyLimit); return Q4_OK;
        case Q4_KEY_DEQUANT_MIN_M: g_dequant_min_m = clamp64(value, 1, kMaxDim + 1); return Q4_OK;
        case Q4_KEY_FORCE_PATH:
            if (!force_path_ok(value)) return Q4_ERR_ARG;
            g_force_path = value;
            return Q4_OK;
        case Q4_KEY_TILE_ROWS:
            if (value != 128 && value != 256) return Q4_ERR_ARG;
            g_tile_rows = value;
            return Q4_OK;
        case Q4_KEY_AFFINE8_FUSED_MAX_M: g_affine8_fused_max_m = clamp64(value, 0, kAffine8FusedLimit); return Q4_OK;
        default: return Q4_ERR_ARG;
    }
}

int q4_get_dispatch(int key, int64_t* value) {
    read_env();
    if (!value) return Q4_ERR_NULL;
    switch (key) {
        case Q4_KEY_SKINNY_MAX_M: *value = g_skinny_max_m; return Q4_OK;
        case Q4_KEY_DEQUANT_MIN_M: *value = g_dequant_min_m; return Q4_OK;
        case Q4_KEY_FORCE_PATH: *value = g_force_path; return Q4_OK;
        case Q4_KEY_TILE_ROWS: *value = g_tile_rows; return Q4_OK;
        case Q4_KEY_AFFINE8_FUSED_MAX_M: *value = g_affine8_fused_max_m; return Q4_OK;
        default: return Q4_ERR_ARG;
    }
}

int q4_dispatch_path(int64_t M, int64_t N, int64_t K, int fmt, int have_workspace) {
    read_env();
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_AFFINE4 && fmt != Q4_FMT_AFFINE8) return Q4_ERR_ARG;
    const int rc = check_dims(M, N, K, fmt == Q4_FMT_Q4_0 ? 32 : 64);
    if (rc) return rc;
    const int64_t forced = g_force_path;
    if (fmt == Q4_FMT_AFFINE8) {
        // the fused kernels (small M) or the matrix-core GEMM on images;
        // dequantise-then-GEMM only when forced; a forced path that
        // affine8_gemm has no kernel for leaves the automatic choice
        if (forced == Q4_PATH_SKINNY || forced == Q4_PATH_MFMA || forced == Q4_PATH_DEQUANT_GEMM) return (int)forced;
        return M <= g_affine8_fused_max_m ? Q4_PATH_SKINNY : Q4_PATH_MFMA;
    }
    if (forced >= 0) return (int)forced;
    if (M <= g_skinny_max_m) return Q4_PATH_SKINNY;
    if (have_workspace && M >= g_dequant_min_m) return Q4_PATH_DEQUANT_GEMM;
    return Q4_PATH_MFMA;
}

int64_t q4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int fmt) {
    if (fmt == Q4_FMT_AFFINE8) return affine8_gemm_workspace_size(M, N, K);
    const int path = q4_dispatch_path(M, N, K, fmt, 1);
    if (path == Q4_PATH_MFMA) return q4::packed_x_bytes(M, N, K);
    // an automatic SKINNY choice above kF32SkinnyMaxM rows runs the
    // matrix-core GEMM for binary32 X: room for it (bfloat16 X uses none)
    if (path == Q4_PATH_SKINNY && g_force_path < 0 && M > kF32SkinnyMaxM) return q4::packed_x_bytes(M, N, K);
    if (path == Q4_PATH_DEQUANT_GEMM) return N * K * 2;
    if (path == Q4_PATH_INT8 && fmt == Q4_FMT_Q4_0) return q8_planes_bytes(M, K);
    return 0;
}

// ---- quantisers ------------------------------------------------------------------

int q4_quantize(const void* w, int w_dtype, int64_t N, int64_t K, uint8_t* w_qs, uint16_t* w_d, void* stream) {
    if (w_dtype != Q4_F32 && w_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    int rc = check_dims(0, N, K, 32);
    if (rc) return rc;
    if (N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w, w_qs, w_d}))) return rc;
    return hip_status(q4::launch_q4_quantize(w, w_dtype, N, K, w_qs, w_d, as_stream(stream)));
}

int q8_1_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* x_qs, uint16_t* x_ds, void* stream) {
    if (x_dtype != Q4_F32 && x_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    int rc = check_dims(M, 0, K, 32);
    if (rc) return rc;
    if (M == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({x, x_qs, x_ds}))) return rc;
    return hip_status(q4::launch_q8_1_quantize(x, x_dtype, M, K, x_qs, x_ds, as_stream(stream)));
}

int affine4_quantize(const void* w, int w_dtype, int64_t N, int64_t K, int64_t group_size, uint8_t* w_q,
                     uint16_t* scales, uint16_t* biases, void* stream) {
    if (w_dtype != Q4_F32 && w_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (group_size != 64) return Q4_ERR_SHAPE;
    int rc = check_dims(0, N, K, 64);
    if (rc) return rc;
    if (N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w, w_q, scales, biases}))) return rc;
    return hip_status(q4::launch_affine4_quantize(w, w_dtype, N, K, group_size, w_q, scales, biases, as_stream(stream)));
}

int q4_dequantize(const uint8_t* w_qs, const uint16_t* w_d, int64_t N, int64_t K, void* out, int out_dtype,
                  void* stream) {
    if (out_dtype != Q4_F32 && out_dtype != Q4_BF16 && out_dtype != Q4_F16) return Q4_ERR_DTYPE;
    int rc = check_dims(0, N, K, 32);
    if (rc) return rc;
    if (N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_qs, w_d, out}))) return rc;
    return hip_status(q4::launch_q4_dequantize(w_qs, w_d, N, K, out, out_dtype, as_stream(stream)));
}

int affine4_dequantize(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases, int64_t group_size,
                       int64_t N, int64_t K, void* out, int out_dtype, void* stream) {
    if (out_dtype != Q4_F32 && out_dtype != Q4_BF16 && out_dtype != Q4_F16) return Q4_ERR_DTYPE;
    if (group_size != 64) return Q4_ERR_SHAPE;
    int rc = check_dims(0, N, K, 64);
    if (rc) return rc;
    if (N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_q, scales, biases, out}))) return rc;
    return hip_status(
        q4::launch_affine4_dequantize(w_q, scales, biases, group_size, N, K, out, out_dtype, as_stream(stream)));
}

// ---- decode GEMV -------------------------------------------------------------------

// Shared checks and launch of every GEMV entry point: nmat matrices (host
// arrays) sharing the activation -- Q8_1 planes (x == nullptr) or the raw
// activation x of x_dtype, quantised inside the kernel.
static int gemv_common(int nmat, const uint8_t* const* qs, const uint16_t* const* d, const int64_t* n,
                       float* const* y, const int8_t* x_qs, const uint16_t* x_ds, const void* x, int x_dtype,
                       int64_t M, int64_t K, void* stream) {
    if (nmat < 1 || nmat > Q4_GEMV_MAX_MATS) return Q4_ERR_ARG;
    if (!qs || !d || !n || !y) return Q4_ERR_NULL;
    int64_t total = 0;
    for (int i = 0; i < nmat; i++) {
        const int rc = check_dims(M, n[i], K, 32);
        if (rc) return rc;
        total += n[i];
    }
    const bool raw = x != nullptr || (x_qs == nullptr && x_ds == nullptr);
    if (raw) {
        if (x_dtype != Q4_F32 && x_dtype != Q4_BF16) return Q4_ERR_DTYPE;
        if (M > Q4_GEMV_ACT_MAX_M) return Q4_ERR_SHAPE;
    } else if (M > Q4_GEMV_MAX_M) {
        return Q4_ERR_SHAPE;
    }
    if (total > int64_t(0x7FFFFFFF)) return Q4_ERR_SHAPE;
    if (M == 0 || total == 0) return Q4_OK;
    int rc = raw ? check_ptrs_aligned({x}) : check_ptrs_aligned({x_qs, x_ds});
    if (rc) return rc;
    for (int i = 0; i < nmat; i++)
        if (n[i] > 0 && (rc = check_ptrs_aligned({qs[i], d[i], y[i]}))) return rc;
    return hip_status(q4::launch_q4_gemv_multi(nmat, qs, d, n, y, raw ? nullptr : x_qs, raw ? nullptr : x_ds,
                                               raw ? x : nullptr, x_dtype, M, K, as_stream(stream)));
}

int q4_gemv(const uint8_t* w_qs, const uint16_t* w_d, const int8_t* x_qs, const uint16_t* x_ds, float* y,
            int64_t M, int64_t N, int64_t K, void* stream) {
    if (!x_qs || !x_ds) {
        const int rc = check_dims(M, N, K, 32);
        if (rc) return rc;
        if (M > Q4_GEMV_MAX_M) return Q4_ERR_SHAPE;
        if (M == 0 || N == 0) return Q4_OK;
        return Q4_ERR_NULL;
    }
    const uint8_t* qs[1] = {w_qs};
    const uint16_t* d[1] = {w_d};
    const int64_t n[1] = {N};
    float* ys[1] = {y};
    return gemv_common(1, qs, d, n, ys, x_qs, x_ds, nullptr, Q4_BF16, M, K, stream);
}

int q4_gemv_fused2(const uint8_t* w0_qs, const uint16_t* w0_d, int64_t N0, const uint8_t* w1_qs,
                   const uint16_t* w1_d, int64_t N1, const int8_t* x_qs, const uint16_t* x_ds, float* y0, float* y1,
                   int64_t M, int64_t K, void* stream) {
    if (!x_qs || !x_ds) {
        int rc = check_dims(M, N0, K, 32);
        if (rc || (rc = check_dims(M, N1, K, 32))) return rc;
        if (M > Q4_GEMV_MAX_M) return Q4_ERR_SHAPE;
        if (M == 0 || N0 + N1 == 0) return Q4_OK;
        return Q4_ERR_NULL;
    }
    const uint8_t* qs[2] = {w0_qs, w1_qs};
    const uint16_t* d[2] = {w0_d, w1_d};
    const int64_t n[2] = {N0, N1};
    float* ys[2] = {y0, y1};
    return gemv_common(2, qs, d, n, ys, x_qs, x_ds, nullptr, Q4_BF16, M, K, stream);
}

int q4_gemv_act(const uint8_t* w_qs, const uint16_t* w_d, const void* x, int x_dtype, float* y, int64_t M,
                int64_t N, int64_t K, void* stream) {
    const uint8_t* qs[1] = {w_qs};
    const uint16_t* d[1] = {w_d};
    const int64_t n[1] = {N};
    float* ys[1] = {y};
    return gemv_common(1, qs, d, n, ys, nullptr, nullptr, x, x_dtype, M, K, stream);
}

int q4_gemv_fused2_act(const uint8_t* w0_qs, const uint16_t* w0_d, int64_t N0, const uint8_t* w1_qs,
                       const uint16_t* w1_d, int64_t N1, const void* x, int x_dtype, float* y0, float* y1,
                       int64_t M, int64_t K, void* stream) {
    const uint8_t* qs[2] = {w0_qs, w1_qs};
    const uint16_t* d[2] = {w0_d, w1_d};
    const int64_t n[2] = {N0, N1};
    float* ys[2] = {y0, y1};
    return gemv_common(2, qs, d, n, ys, nullptr, nullptr, x, x_dtype, M, K, stream);
}

int q4_gemv_multi(int nmat, const uint8_t* const* w_qs, const uint16_t* const* w_d, const int64_t* n,
                  const int8_t* x_qs, const uint16_t* x_ds, float* const* y, int64_t M, int64_t K, void* stream) {
    if (!x_qs || !x_ds) return Q4_ERR_NULL;
    return gemv_common(nmat, w_qs, w_d, n, y, x_qs, x_ds, nullptr, Q4_BF16, M, K, stream);
}

int q4_gemv_multi_act(int nmat, const uint8_t* const* w_qs, const uint16_t* const* w_d, const int64_t* n,
                      const void* x, int x_dtype, float* const* y, int64_t M, int64_t K, void* stream) {
    if (!x) return Q4_ERR_NULL;
    return gemv_common(nmat, w_qs, w_d, n, y, nullptr, nullptr, x, x_dtype, M, K, stream);
}

// ---- GEMM ----------------------------------------------------------------------------

static int gemm_common(int wf, const void* a, const void* b, const void* c, const void* x, int x_dtype, void* y,
                       int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                       void* stream) {
    const int fmt = (wf == q4::WF_Q4_0) ? Q4_FMT_Q4_0 : Q4_FMT_AFFINE4;
    // "have workspace" for the dispatch: enough for the dequantised weights
    const bool have_ws = workspace != nullptr && workspace_bytes >= N * K * 2;
    int path = q4_dispatch_path(M, N, K, fmt, have_ws ? 1 : 0);
    if (path < 0) return path;
    if (M == 0 || N == 0) return Q4_OK;
    const bool have_images =
        workspace != nullptr && workspace_bytes >= q4::x_image_bytes(M, K) + q4::weight_image_bytes(N, K);
    if (path == Q4_PATH_SKINNY && g_force_path < 0 && x_dtype == Q4_F32 && M > kF32SkinnyMaxM &&
        (have_images || M > kF32SkinnyNoImageMaxM))
        path = Q4_PATH_MFMA;
    if (path == Q4_PATH_MFMA && g_force_path < 0 && x_dtype == Q4_BF16 && !have_images && M > kSkinnyLimit &&
        M <= kBf16ChunkNoImageMaxM && g_skinny_max_m >= kSkinnyLimit)
        return hip_status(q4::launch_gemm_skinny(wf, a, b, c, x, x_dtype, y, y_dtype, M, N, K, as_stream(stream)));
    hipStream_t s = as_stream(stream);
    switch (path) {
        case Q4_PATH_GEMV: {
            // the integer-dot GEMV on X quantised to Q8_1 inside the kernel
            if (wf != q4::WF_Q4_0 || M > Q4_GEMV_ACT_MAX_M || y_dtype != Q4_F32) return Q4_ERR_ARG;
            const uint8_t* qs[1] = {static_cast<const uint8_t*>(a)};
            const uint16_t* d[1] = {static_cast<const uint16_t*>(b)};
            const int64_t n[1] = {N};
            float* ys[1] = {static_cast<float*>(y)};
            return gemv_common(1, qs, d, n, ys, nullptr, nullptr, x, x_dtype, M, K, stream);
        }
        case Q4_PATH_INT8: {
            // X quantised to Q8_1 in the workspace, then the int8 matrix-core GEMM
            if (wf != q4::WF_Q4_0) return Q4_ERR_ARG;
            if (workspace == nullptr || workspace_bytes < q8_planes_bytes(M, K)) return Q4_ERR_WORKSPACE;
            if (!aligned16(workspace)) return Q4_ERR_ALIGN;
            int8_t* xq = static_cast<int8_t*>(workspace);
            uint16_t* xds = reinterpret_cast<uint16_t*>(xq + M * K);
            if (q4::launch_q8_1_quantize(x, x_dtype, M, K, xq, xds, s) != hipSuccess) return Q4_ERR_HIP;
            return hip_status(q4::launch_gemm_q8(static_cast<const uint8_t*>(a), static_cast<const uint16_t*>(b), xq,
                                                 xds, y, y_dtype, M, N, K, s));
        }
        case Q4_PATH_SKINNY:
            if (M > kSkinnyLimit) return Q4_ERR_ARG;
            return hip_status(q4::launch_gemm_skinny(wf, a, b, c, x, x_dtype, y, y_dtype, M, N, K, s));
        case Q4_PATH_MFMA:
            // the images alone run the packed GEMM; room for the partial
            // results as well lets small tile counts split K
            if (workspace != nullptr && workspace_bytes >= q4::x_image_bytes(M, K) + q4::weight_image_bytes(N, K)) {
                if (!aligned16(workspace)) return Q4_ERR_ALIGN;
                const bool split = workspace_bytes >= q4::packed_x_bytes(M, N, K);
                return hip_status(
                    q4::launch_gemm_packed(wf, a, b, c, x, x_dtype, y, y_dtype, M, N, K, workspace, split, s));
            }
            return hip_status(q4::launch_gemm_mfma(wf, a, b, c, x, x_dtype, y, y_dtype, M, N, K, s));
        case Q4_PATH_DEQUANT_GEMM: {
            if (!have_ws) return Q4_ERR_WORKSPACE;
            if (!aligned16(workspace)) return Q4_ERR_ALIGN;
            hipError_t e = (wf == q4::WF_Q4_0)
                               ? q4::launch_q4_dequantize(static_cast<const uint8_t*>(a),
                                                          static_cast<const uint16_t*>(b), N, K, workspace,
                                                          q4::DT_F16, s)
                               : q4::launch_affine4_dequantize(static_cast<const uint8_t*>(a),
                                                               static_cast<const uint16_t*>(b),
                                                               static_cast<const uint16_t*>(c), 64, N, K, workspace,
                                                               q4::DT_F16, s);
            if (e != hipSuccess) return Q4_ERR_HIP;
            if (M <= kSkinnyLimit && M <= g_skinny_max_m)
                return hip_status(q4::launch_gemm_skinny(q4::WF_DENSE16, workspace, nullptr, nullptr, x, x_dtype, y,
                                                         y_dtype, M, N, K, s));
            return hip_status(q4::launch_gemm_mfma(q4::WF_DENSE16, workspace, nullptr, nullptr, x, x_dtype, y,
                                                   y_dtype, M, N, K, s));
        }
        default: return Q4_ERR_ARG;
    }
}

int q4_gemm(const uint8_t* w_qs, const uint16_t* w_d, const void* x, int x_dtype, void* y, int y_dtype, int64_t M,
            int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
    if ((x_dtype != Q4_BF16 && x_dtype != Q4_F32) || (y_dtype != Q4_BF16 && y_dtype != Q4_F32)) return Q4_ERR_DTYPE;
    int rc = check_dims(M, N, K, 32);
    if (rc) return rc;
    if (M == 0 || N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_qs, w_d, x, y}))) return rc;
    return gemm_common(q4::WF_Q4_0, w_qs, w_d, nullptr, x, x_dtype, y, y_dtype, M, N, K, workspace, workspace_bytes,
                       stream);
}

int affine4_gemm(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases, int64_t group_size,
                 const void* x, int x_dtype, void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                 int64_t workspace_bytes, void* stream) {
    if ((x_dtype != Q4_BF16 && x_dtype != Q4_F32) || (y_dtype != Q4_BF16 && y_dtype != Q4_F32)) return Q4_ERR_DTYPE;
    if (group_size != 64) return Q4_ERR_SHAPE;
    int rc = check_dims(M, N, K, 64);
    if (rc) return rc;
    if (M == 0 || N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_q, scales, biases, x, y}))) return rc;
    return gemm_common(q4::WF_AFFINE4, w_q, scales, biases, x, x_dtype, y, y_dtype, M, N, K, workspace,
                       workspace_bytes, stream);
}

int q4_gemm_q8(const uint8_t* w_qs, const uint16_t* w_d, const int8_t* x_qs, const uint16_t* x_ds, void* y,
               int y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    if (y_dtype != Q4_BF16 && y_dtype != Q4_F32) return Q4_ERR_DTYPE;
    int rc = check_dims(M, N, K, 32);
    if (rc) return rc;
    if (M == 0 || N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_qs, w_d, x_qs, x_ds, y}))) return rc;
    return hip_status(q4::launch_gemm_q8(w_qs, w_d, x_qs, x_ds, y, y_dtype, M, N, K, as_stream(stream)));
}

static int image_dims(int fmt, int64_t M, int64_t N, int64_t K) {
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_AFFINE4 && fmt != Q4_FMT_AFFINE8) return Q4_ERR_ARG;
    return check_dims(M, N, K, fmt == Q4_FMT_Q4_0 ? 32 : 64);
}

static int image_wf(int fmt) {
    return fmt == Q4_FMT_Q4_0 ? q4::WF_Q4_0 : fmt == Q4_FMT_AFFINE4 ? q4::WF_AFFINE4 : q4::WF_AFFINE8;
}

int64_t q4_weight_image_size(int64_t N, int64_t K, int fmt) {
    if (image_dims(fmt, 0, N, K) != Q4_OK) return 0;
    return fmt == Q4_FMT_AFFINE8 ? q4::weight_image8_bytes(N, K) : q4::weight_image_bytes(N, K);
}

int q4_pack_weight_image(int fmt, const uint8_t* w_q, const uint16_t* w_s, const uint16_t* w_b, int64_t N,
                         int64_t K, void* image, void* stream) {
    int rc = image_dims(fmt, 0, N, K);
    if (rc) return rc;
    if (N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_q, w_s, image}))) return rc;
    if (fmt != Q4_FMT_Q4_0 && (rc = check_ptrs_aligned({w_b}))) return rc;
    return hip_status(q4::launch_pack_weight_image(image_wf(fmt), w_q, w_s, fmt == Q4_FMT_Q4_0 ? nullptr : w_b, N, K,
                                                   image, as_stream(stream)));
}

int64_t q4_gemm_image_workspace_size(int64_t M, int64_t K) {
    if (check_dims(M, 0, K, 32) != Q4_OK) return 0;
    return q4::x_image_bytes(M, K);
}

int q4_gemm_image(int fmt, const void* image, const void* x, int x_dtype, void* y, int y_dtype, int64_t M,
                  int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
    if ((x_dtype != Q4_BF16 && x_dtype != Q4_F32) || (y_dtype != Q4_BF16 && y_dtype != Q4_F32)) return Q4_ERR_DTYPE;
    int rc = image_dims(fmt, M, N, K);
    if (rc) return rc;
    if (M == 0 || N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({image, x, y}))) return rc;
    const int64_t ximg = q4::x_image_bytes(M, K);
    if (workspace == nullptr || workspace_bytes < ximg) return Q4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return Q4_ERR_ALIGN;
    // room for the split-K partial results after the X image: split small tile counts
    const int64_t part = q4::splitk_bytes(M, N, K);
    float* pp = (part > 0 && workspace_bytes >= ximg + part)
                    ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ximg) : nullptr;
    return hip_status(q4::launch_gemm_image(image_wf(fmt), image, x, x_dtype, y, y_dtype, M, N, K, workspace, pp,
                                            as_stream(stream)));
}

// For callers that cannot allocate: the workspace is the library's fixed
// per-GPU scratch array.
int q4_gemm_image_noalloc(int fmt, const void* image, const void* x, int x_dtype, void* y, int y_dtype, int64_t M,
                          int64_t N, int64_t K, void* stream) {
    if ((x_dtype != Q4_BF16 && x_dtype != Q4_F32) || (y_dtype != Q4_BF16 && y_dtype != Q4_F32)) return Q4_ERR_DTYPE;
    int rc = image_dims(fmt, M, N, K);
    if (rc) return rc;
    if (M == 0 || N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({image, x, y}))) return rc;
    if (q4::x_image_bytes(M, K) > Q4_NOALLOC_SCRATCH_BYTES) return Q4_ERR_SCRATCH;
    void* scratch = nullptr;
    if (q4::noalloc_scratch(&scratch) != hipSuccess) return Q4_ERR_HIP;
    return q4_gemm_image(fmt, image, x, x_dtype, y, y_dtype, M, N, K, scratch, Q4_NOALLOC_SCRATCH_BYTES, stream);
}

// ---- affine 8-bit ------------------------------------------------------------------

int affine8_quantize(const void* w, int w_dtype, int64_t N, int64_t K, int64_t group_size, uint8_t* w_q,
                     uint16_t* scales, uint16_t* biases, void* stream) {
    if (w_dtype != Q4_F32 && w_dtype != Q4_BF16) return Q4_ERR_DTYPE;
    if (group_size != 64) return Q4_ERR_SHAPE;
    int rc = check_dims(0, N, K, 64);
    if (rc) return rc;
    if (N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w, w_q, scales, biases}))) return rc;
    return hip_status(q4::launch_affine8_quantize(w, w_dtype, N, K, w_q, scales, biases, as_stream(stream)));
}

int affine8_dequantize(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases, int64_t group_size,
                       int64_t N, int64_t K, void* out, int out_dtype, void* stream) {
    if (out_dtype != Q4_F32 && out_dtype != Q4_BF16 && out_dtype != Q4_F16) return Q4_ERR_DTYPE;
    if (group_size != 64) return Q4_ERR_SHAPE;
    int rc = check_dims(0, N, K, 64);
    if (rc) return rc;
    if (N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_q, scales, biases, out}))) return rc;
    return hip_status(q4::launch_affine8_dequantize(w_q, scales, biases, N, K, out, out_dtype, as_stream(stream)));
}

int64_t affine8_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (check_dims(M, N, K, 64) != Q4_OK) return 0;
    // the fused kernels use none; dequantise-then-GEMM the binary16 weights;
    // the matrix-core GEMM its two images and split-K partials.  Enough for
    // either activation type (f32 X above 16 rows leaves the fused kernels).
    const int path = q4_dispatch_path(M, N, K, Q4_FMT_AFFINE8, 1);
    if (path == Q4_PATH_SKINNY && M <= q4::kAffine8GemvMaxM) return 0;
    if (path == Q4_PATH_DEQUANT_GEMM) return N * K * 2;
    return q4::affine8_packed_bytes(M, N, K);
}

int affine8_gemm(const uint8_t* w_q, const uint16_t* scales, const uint16_t* biases, int64_t group_size,
                 const void* x, int x_dtype, void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                 int64_t workspace_bytes, void* stream) {
    if ((x_dtype != Q4_BF16 && x_dtype != Q4_F32) || (y_dtype != Q4_BF16 && y_dtype != Q4_F32)) return Q4_ERR_DTYPE;
    if (group_size != 64) return Q4_ERR_SHAPE;
    int rc = check_dims(M, N, K, 64);
    if (rc) return rc;
    if (M == 0 || N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({w_q, scales, biases, x, y}))) return rc;
    hipStream_t s = as_stream(stream);
    const int path = q4_dispatch_path(M, N, K, Q4_FMT_AFFINE8, workspace != nullptr ? 1 : 0);
    if (path < 0) return path;
    if (path == Q4_PATH_SKINNY) {
        // M <= 4: the fused vector kernel; bf16 X up to 32 rows: the bf16-MFMA
        // kernel on the raw codes; f32 X up to 16 rows: the vector kernel;
        // f32 X above that goes on to the matrix-core GEMM
        if (M <= 4 || (x_dtype == Q4_F32 && M <= q4::kAffine8GemvMaxM))
            return hip_status(q4::launch_affine8_gemv(w_q, scales, biases, x, x_dtype, y, y_dtype, M, N, K, s));
        if (x_dtype == Q4_BF16 && M <= q4::kAffine8MmaMaxM)
            return hip_status(q4::launch_affine8_mma(w_q, scales, biases, x, y, y_dtype, M, N, K, s));
    }
    if (path != Q4_PATH_DEQUANT_GEMM) {
        // the weight and X images in the workspace (with room for them, the
        // split-K partials too), then the matrix-core GEMM
        if (workspace == nullptr || workspace_bytes < q4::x_image_bytes(M, K) + q4::weight_image8_bytes(N, K))
            return Q4_ERR_WORKSPACE;
        if (!aligned16(workspace)) return Q4_ERR_ALIGN;
        const bool split = workspace_bytes >= q4::affine8_packed_bytes(M, N, K);
        return hip_status(q4::launch_affine8_gemm_packed(w_q, scales, biases, x, x_dtype, y, y_dtype, M, N, K,
                                                         workspace, split, s));
    }
    // dequantise to binary16 in the workspace, then the dense GEMM
    if (workspace == nullptr || workspace_bytes < N * K * 2) return Q4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return Q4_ERR_ALIGN;
    if (q4::launch_affine8_dequantize(w_q, scales, biases, N, K, workspace, q4::DT_F16, s) != hipSuccess)
        return Q4_ERR_HIP;
    if (M <= g_skinny_max_m)
        return hip_status(
            q4::launch_gemm_skinny(q4::WF_DENSE16, workspace, nullptr, nullptr, x, x_dtype, y, y_dtype, M, N, K, s));
    return hip_status(q4::launch_gemm_mfma(q4::WF_DENSE16, workspace, nullptr, nullptr, x, x_dtype, y, y_dtype, M, N, K, s));
}

int dense_gemm(const void* x, int x_dtype, const uint16_t* w_f16, void* y, int y_dtype, int64_t M, int64_t N,
               int64_t K, void* stream) {
    if ((x_dtype != Q4_BF16 && x_dtype != Q4_F32) || (y_dtype != Q4_BF16 && y_dtype != Q4_F32)) return Q4_ERR_DTYPE;
    int rc = check_dims(M, N, K, 32);
    if (rc) return rc;
    if (M == 0 || N == 0) return Q4_OK;
    if ((rc = check_ptrs_aligned({x, w_f16, y}))) return rc;
    read_env();
    hipStream_t s = as_stream(stream);
    if (M <= g_skinny_max_m)
        return hip_status(
            q4::launch_gemm_skinny(q4::WF_DENSE16, w_f16, nullptr, nullptr, x, x_dtype, y, y_dtype, M, N, K, s));
    return hip_status(q4::launch_gemm_mfma(q4::WF_DENSE16, w_f16, nullptr, nullptr, x, x_dtype, y, y_dtype, M, N, K, s));
}

}  // extern "C"
