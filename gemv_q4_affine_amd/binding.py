"""Thin ctypes binding of libq4.so (include/q4.h), same names as the C ABI.

Argument marshalling only: it turns torch tensors into device pointers, the
current HIP stream and dtype codes, allocates outputs with torch.empty when
the caller passes none, and raises Q4Error on a non-zero status.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# Q4_LIB_PATH: another build of the same library (the host-side sanitizer
# build that tests load); by default the in-tree libq4.so.
LIB_PATH = os.environ.get("Q4_LIB_PATH") or os.path.join(_PKG, "libq4.so")

# status, dtype, format and path codes (include/q4.h)
(Q4_OK, Q4_ERR_NULL, Q4_ERR_SHAPE, Q4_ERR_ALIGN, Q4_ERR_DTYPE, Q4_ERR_HIP, Q4_ERR_ARG, Q4_ERR_WORKSPACE,
 Q4_ERR_SCRATCH) = (0, -1, -2, -3, -4, -5, -6, -7, -8)
Q4_NOALLOC_SCRATCH_BYTES = 33 << 20
Q4_F32, Q4_BF16, Q4_F16 = 0, 1, 2
Q4_FMT_Q4_0, Q4_FMT_AFFINE4, Q4_FMT_AFFINE8 = 0, 1, 2
Q4_PATH_GEMV, Q4_PATH_SKINNY, Q4_PATH_MFMA, Q4_PATH_DEQUANT_GEMM, Q4_PATH_INT8 = 0, 1, 2, 3, 4
Q4_KEY_SKINNY_MAX_M, Q4_KEY_DEQUANT_MIN_M, Q4_KEY_FORCE_PATH, Q4_KEY_TILE_ROWS, Q4_KEY_AFFINE8_FUSED_MAX_M = 0, 1, 2, 3, 4
Q4_GEMV_MAX_M = 16
Q4_GEMV_ACT_MAX_M = 4
Q4_GEMV_MAX_MATS = 4

# exported symbols and their ctypes signatures
_P, _I64, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "q4_quantize": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P]),
    "q8_1_quantize_act": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P]),
    "affine4_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P]),
    "q4_dequantize": (_INT, [_P, _P, _I64, _I64, _P, _INT, _P]),
    "affine4_dequantize": (_INT, [_P, _P, _P, _I64, _I64, _I64, _P, _INT, _P]),
    "q4_gemv": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "q4_gemv_fused2": (_INT, [_P, _P, _I64, _P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _P]),
    "q4_gemv_act": (_INT, [_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P]),
    "q4_gemv_fused2_act": (_INT, [_P, _P, _I64, _P, _P, _I64, _P, _INT, _P, _P, _I64, _I64, _P]),
    "q4_gemv_multi": (_INT, [_INT, _P, _P, _P, _P, _P, _P, _I64, _I64, _P]),
    "q4_gemv_multi_act": (_INT, [_INT, _P, _P, _P, _P, _INT, _P, _I64, _I64, _P]),
    "q4_gemm": (_INT, [_P, _P, _P, _INT, _P, _INT, _I64, _I64, _I64, _P, _I64, _P]),
    "affine4_gemm": (_INT, [_P, _P, _P, _I64, _P, _INT, _P, _INT, _I64, _I64, _I64, _P, _I64, _P]),
    "q4_gemm_workspace_size": (_I64, [_I64, _I64, _I64, _INT]),
    "dense_gemm": (_INT, [_P, _INT, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "q4_weight_image_size": (_I64, [_I64, _I64, _INT]),
    "q4_pack_weight_image": (_INT, [_INT, _P, _P, _P, _I64, _I64, _P, _P]),
    "q4_gemm_image_workspace_size": (_I64, [_I64, _I64]),
    "q4_gemm_image": (_INT, [_INT, _P, _P, _INT, _P, _INT, _I64, _I64, _I64, _P, _I64, _P]),
    "q4_gemm_image_noalloc": (_INT, [_INT, _P, _P, _INT, _P, _INT, _I64, _I64, _I64, _P]),
    "q4_gemm_q8": (_INT, [_P, _P, _P, _P, _P, _INT, _I64, _I64, _I64, _P]),
    "q4_dispatch_path": (_INT, [_I64, _I64, _I64, _INT, _INT]),
    "q4_set_dispatch": (_INT, [_INT, _I64]),
    "q4_get_dispatch": (_INT, [_INT, ctypes.POINTER(ctypes.c_int64)]),
    "affine8_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P]),
    "affine8_dequantize": (_INT, [_P, _P, _P, _I64, _I64, _I64, _P, _INT, _P]),
    "affine8_gemm_workspace_size": (_I64, [_I64, _I64, _I64]),
    "affine8_gemm": (_INT, [_P, _P, _P, _I64, _P, _INT, _P, _INT, _I64, _I64, _I64, _P, _I64, _P]),
    "q4_status_string": (ctypes.c_char_p, [_INT]),
    "q4_version": (ctypes.c_char_p, []),
}


class Q4Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libq4.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gemv_q4_affine_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().q4_status_string(status).decode()


def version() -> str:
    return lib().q4_version().decode()


def _check(fn: str, status: int):
    if status != Q4_OK:
        raise Q4Error(fn, status, status_string(status))


_DT = {torch.float32: Q4_F32, torch.bfloat16: Q4_BF16, torch.float16: Q4_F16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _p(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return t  # raw pointer (int) passed through
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _alloc_stream(stream):
    """The torch stream that owns memory this call allocates: the stream the
    kernels are enqueued on, so that the caching allocator hands a freed block
    (an "auto" workspace, dropped on return) to no other stream's work while
    the kernels may still use it."""
    if stream is None:
        return None
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _empty(shape, dtype, like, stream=None):
    s = _alloc_stream(stream)
    if s is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    with torch.cuda.stream(s):
        return torch.empty(shape, dtype=dtype, device=like.device)


# ---- quantisers ---------------------------------------------------------------

def q4_quantize(w, w_qs=None, w_d=None, stream=None):
    """W [N, K] (f32 or bf16) -> (qs uint8 [N, K/32, 16], d int16 bits [N, K/32])."""
    N, K = w.shape
    w_qs = _empty((N, K // 32, 16), torch.uint8, w, stream) if w_qs is None else w_qs
    w_d = _empty((N, K // 32), torch.int16, w, stream) if w_d is None else w_d
    _check("q4_quantize", lib().q4_quantize(_p(w), _dt(w), N, K, _p(w_qs), _p(w_d), _stream(stream)))
    return w_qs, w_d


def q8_1_quantize_act(x, x_qs=None, x_ds=None, stream=None):
    """X [M, K] (f32 or bf16) -> (qs int8 [M, K], ds int16 bits [M, K/32, 2])."""
    M, K = x.shape
    x_qs = _empty((M, K), torch.int8, x, stream) if x_qs is None else x_qs
    x_ds = _empty((M, K // 32, 2), torch.int16, x, stream) if x_ds is None else x_ds
    _check("q8_1_quantize_act",
           lib().q8_1_quantize_act(_p(x), _dt(x), M, K, _p(x_qs), _p(x_ds), _stream(stream)))
    return x_qs, x_ds


def affine4_quantize(w, group_size=64, w_q=None, scales=None, biases=None, stream=None):
    """W [N, K] (bf16 or f32) -> (q uint8 [N, K/2], scales, biases int16 bits [N, K/G])."""
    N, K = w.shape
    w_q = _empty((N, K // 2), torch.uint8, w, stream) if w_q is None else w_q
    scales = _empty((N, K // group_size), torch.int16, w, stream) if scales is None else scales
    biases = _empty((N, K // group_size), torch.int16, w, stream) if biases is None else biases
    _check("affine4_quantize", lib().affine4_quantize(_p(w), _dt(w), N, K, group_size, _p(w_q), _p(scales),
                                                      _p(biases), _stream(stream)))
    return w_q, scales, biases


def q4_dequantize(w_qs, w_d, out_dtype=torch.float16, out=None, stream=None):
    N, nb = w_d.shape[0], w_d.shape[1]
    K = nb * 32
    out = _empty((N, K), out_dtype, w_qs, stream) if out is None else out
    _check("q4_dequantize", lib().q4_dequantize(_p(w_qs), _p(w_d), N, K, _p(out), _dt(out), _stream(stream)))
    return out


def affine4_dequantize(w_q, scales, biases, group_size=64, out_dtype=torch.float16, out=None, stream=None):
    N, K = w_q.shape[0], w_q.shape[1] * 2
    out = _empty((N, K), out_dtype, w_q, stream) if out is None else out
    _check("affine4_dequantize", lib().affine4_dequantize(_p(w_q), _p(scales), _p(biases), group_size, N, K,
                                                          _p(out), _dt(out), _stream(stream)))
    return out


# ---- decode GEMV ----------------------------------------------------------------

def q4_gemv(w_qs, w_d, x_qs, x_ds, y=None, stream=None):
    """y float32 [M, N] from Q4_0 planes and Q8_1 activation planes."""
    N = w_d.shape[0]
    M, K = x_qs.shape
    y = _empty((M, N), torch.float32, x_qs, stream) if y is None else y
    _check("q4_gemv", lib().q4_gemv(_p(w_qs), _p(w_d), _p(x_qs), _p(x_ds), _p(y), M, N, K, _stream(stream)))
    return y


def q4_gemv_fused2(w0_qs, w0_d, w1_qs, w1_d, x_qs, x_ds, y0=None, y1=None, stream=None):
    N0, N1 = w0_d.shape[0], w1_d.shape[0]
    M, K = x_qs.shape
    y0 = _empty((M, N0), torch.float32, x_qs, stream) if y0 is None else y0
    y1 = _empty((M, N1), torch.float32, x_qs, stream) if y1 is None else y1
    _check("q4_gemv_fused2", lib().q4_gemv_fused2(_p(w0_qs), _p(w0_d), N0, _p(w1_qs), _p(w1_d), N1, _p(x_qs),
                                                  _p(x_ds), _p(y0), _p(y1), M, K, _stream(stream)))
    return y0, y1


def q4_gemv_act(w_qs, w_d, x, y=None, stream=None):
    """q4_gemv on a raw bf16 / f32 activation x [M, K], quantised to Q8_1 inside
    the kernel; bit-identical to q8_1_quantize_act followed by q4_gemv."""
    N = w_d.shape[0]
    M, K = x.shape
    y = _empty((M, N), torch.float32, x, stream) if y is None else y
    _check("q4_gemv_act", lib().q4_gemv_act(_p(w_qs), _p(w_d), _p(x), _dt(x), _p(y), M, N, K, _stream(stream)))
    return y


def q4_gemv_fused2_act(w0_qs, w0_d, w1_qs, w1_d, x, y0=None, y1=None, stream=None):
    N0, N1 = w0_d.shape[0], w1_d.shape[0]
    M, K = x.shape
    y0 = _empty((M, N0), torch.float32, x, stream) if y0 is None else y0
    y1 = _empty((M, N1), torch.float32, x, stream) if y1 is None else y1
    _check("q4_gemv_fused2_act", lib().q4_gemv_fused2_act(_p(w0_qs), _p(w0_d), N0, _p(w1_qs), _p(w1_d), N1,
                                                          _p(x), _dt(x), _p(y0), _p(y1), M, K,
                                                          _stream(stream)))
    return y0, y1


def _mat_arrays(mats, ys):
    n = len(mats)
    qs = (ctypes.c_void_p * n)(*[_p(q) for q, _ in mats])
    ds = (ctypes.c_void_p * n)(*[_p(d) for _, d in mats])
    rows = (ctypes.c_int64 * n)(*[d.shape[0] for _, d in mats])
    yp = (ctypes.c_void_p * n)(*[_p(y) for y in ys])
    return qs, ds, rows, yp


def q4_gemv_multi(mats, x_qs, x_ds, ys=None, stream=None):
    """One launch over several Q4_0 matrices [(qs, d), ...] sharing the Q8_1
    activation; returns a list of float32 [M, N_i]."""
    M, K = x_qs.shape
    ys = [_empty((M, d.shape[0]), torch.float32, x_qs, stream) for _, d in mats] if ys is None else ys
    qs, ds, rows, yp = _mat_arrays(mats, ys)
    _check("q4_gemv_multi", lib().q4_gemv_multi(len(mats), qs, ds, rows, _p(x_qs), _p(x_ds), yp, M, K,
                                                _stream(stream)))
    return ys


def q4_gemv_multi_act(mats, x, ys=None, stream=None):
    """q4_gemv_multi on a raw bf16 / f32 activation, quantised to Q8_1 in the kernel."""
    M, K = x.shape
    ys = [_empty((M, d.shape[0]), torch.float32, x, stream) for _, d in mats] if ys is None else ys
    qs, ds, rows, yp = _mat_arrays(mats, ys)
    _check("q4_gemv_multi_act", lib().q4_gemv_multi_act(len(mats), qs, ds, rows, _p(x), _dt(x), yp, M, K,
                                                        _stream(stream)))
    return ys


# ---- GEMM -----------------------------------------------------------------------------

def _workspace(workspace, M, N, K, fmt, like, stream=None):
    """"auto": a fresh scratch tensor of q4_gemm_workspace_size bytes (None if
    that is 0), owned by the call's stream; None: no workspace; else the
    caller's tensor."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
        n = q4_gemm_workspace_size(M, N, K, fmt)
        return _empty((n,), torch.uint8, like, stream) if n > 0 else None
    return workspace


def q4_gemm(w_qs, w_d, x, y_dtype=torch.bfloat16, y=None, workspace="auto", stream=None):
    N = w_d.shape[0]
    M, K = x.shape
    y = _empty((M, N), y_dtype, x, stream) if y is None else y
    workspace = _workspace(workspace, M, N, K, Q4_FMT_Q4_0, x, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("q4_gemm", lib().q4_gemm(_p(w_qs), _p(w_d), _p(x), _dt(x), _p(y), _dt(y), M, N, K, _p(workspace),
                                    ws_bytes, _stream(stream)))
    return y


def affine4_gemm(w_q, scales, biases, x, group_size=64, y_dtype=torch.bfloat16, y=None, workspace="auto",
                 stream=None):
    N = w_q.shape[0]
    M, K = x.shape
    y = _empty((M, N), y_dtype, x, stream) if y is None else y
    workspace = _workspace(workspace, M, N, K, Q4_FMT_AFFINE4, x, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("affine4_gemm", lib().affine4_gemm(_p(w_q), _p(scales), _p(biases), group_size, _p(x), _dt(x), _p(y),
                                              _dt(y), M, N, K, _p(workspace), ws_bytes, _stream(stream)))
    return y


# ---- affine 8-bit ---------------------------------------------------------------

def affine8_quantize(w, group_size=64, w_q=None, scales=None, biases=None, stream=None):
    """W [N, K] (bf16 or f32) -> (q uint8 [N, K], scales, biases int16 bits [N, K/G])."""
    N, K = w.shape
    w_q = _empty((N, K), torch.uint8, w, stream) if w_q is None else w_q
    scales = _empty((N, K // group_size), torch.int16, w, stream) if scales is None else scales
    biases = _empty((N, K // group_size), torch.int16, w, stream) if biases is None else biases
    _check("affine8_quantize", lib().affine8_quantize(_p(w), _dt(w), N, K, group_size, _p(w_q), _p(scales),
                                                      _p(biases), _stream(stream)))
    return w_q, scales, biases


def affine8_dequantize(w_q, scales, biases, group_size=64, out_dtype=torch.float16, out=None, stream=None):
    N, K = w_q.shape
    out = _empty((N, K), out_dtype, w_q, stream) if out is None else out
    _check("affine8_dequantize", lib().affine8_dequantize(_p(w_q), _p(scales), _p(biases), group_size, N, K,
                                                          _p(out), _dt(out), _stream(stream)))
    return out


def affine8_gemm(w_q, scales, biases, x, group_size=64, y_dtype=torch.bfloat16, y=None, workspace="auto",
                 stream=None):
    """Y [M, N] = X . dequant(W)^T for affine 8-bit weights (workspace "auto": allocated when M needs one)."""
    N, K = w_q.shape
    M = x.shape[0]
    y = _empty((M, N), y_dtype, x, stream) if y is None else y
    if isinstance(workspace, str):
        n = int(lib().affine8_gemm_workspace_size(M, N, K))
        workspace = _empty((n,), torch.uint8, x, stream) if n > 0 else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("affine8_gemm", lib().affine8_gemm(_p(w_q), _p(scales), _p(biases), group_size, _p(x), _dt(x), _p(y),
                                              _dt(y), M, N, K, _p(workspace), ws_bytes, _stream(stream)))
    return y


def q4_gemm_workspace_size(M, N, K, fmt=Q4_FMT_Q4_0) -> int:
    return int(lib().q4_gemm_workspace_size(M, N, K, fmt))


def affine8_gemm_workspace_size(M, N, K) -> int:
    return int(lib().affine8_gemm_workspace_size(M, N, K))


def q4_weight_image_size(N, K, fmt=Q4_FMT_Q4_0) -> int:
    return int(lib().q4_weight_image_size(N, K, fmt))


def q4_gemm_image_workspace_size(M, K) -> int:
    return int(lib().q4_gemm_image_workspace_size(M, K))


def q4_pack_weight_image(w_q, w_s, w_b=None, fmt=None, image=None, stream=None):
    """The matrix-core GEMM's weight image of Q4_0 planes (w_q = qs [N, K/32, 16],
    w_s = d) or affine planes (w_s = scales, w_b = biases; w_q [N, K/2] for
    4-bit codes, [N, K] for 8-bit codes)."""
    N = w_s.shape[0]
    if fmt is None:
        if w_b is None:
            fmt = Q4_FMT_Q4_0
        else:
            fmt = Q4_FMT_AFFINE8 if w_q.shape[-1] == w_s.shape[1] * 64 else Q4_FMT_AFFINE4
    K = w_s.shape[1] * (32 if fmt == Q4_FMT_Q4_0 else 64)
    if image is None:
        n = lib().q4_weight_image_size(N, K, fmt)
        image = _empty((max(n, 16),), torch.uint8, w_q, stream)
    _check("q4_pack_weight_image", lib().q4_pack_weight_image(fmt, _p(w_q), _p(w_s), _p(w_b),
                                                              N, K, _p(image), _stream(stream)))
    return image


def q4_gemm_image(image, x, N, fmt=Q4_FMT_Q4_0, y_dtype=torch.bfloat16, y=None, workspace=None, stream=None):
    """Y [M, N] = X . dequant(W)^T from a weight image (q4_pack_weight_image)."""
    M, K = x.shape
    y = _empty((M, N), y_dtype, x, stream) if y is None else y
    if workspace is None:
        workspace = _empty((max(lib().q4_gemm_image_workspace_size(M, K), 16),), torch.uint8, x, stream)
    _check("q4_gemm_image", lib().q4_gemm_image(fmt, _p(image), _p(x), _dt(x), _p(y), _dt(y), M, N, K,
                                                _p(workspace), workspace.numel() * workspace.element_size(),
                                                _stream(stream)))
    return y


def q4_gemm_image_noalloc(image, x, N, fmt=Q4_FMT_Q4_0, y_dtype=torch.bfloat16, y=None, stream=None):
    """q4_gemm_image with the library's fixed per-GPU scratch as workspace:
    no device allocation when `y` is given.  Calls on one GPU must not overlap."""
    M, _ = x.shape
    y = _empty((M, N), y_dtype, x, stream) if y is None else y
    _check("q4_gemm_image_noalloc", lib().q4_gemm_image_noalloc(fmt, _p(image), _p(x), _dt(x), _p(y), _dt(y), M, N,
                                                                x.shape[1], _stream(stream)))
    return y


def q4_gemm_q8(w_qs, w_d, x_qs, x_ds, y_dtype=torch.float32, y=None, stream=None):
    """Q4_0 planes x Q8_1 planes (q8_1_quantize_act) on the int8 matrix cores, any M."""
    N = w_d.shape[0]
    M, K = x_qs.shape
    y = _empty((M, N), y_dtype, x_qs, stream) if y is None else y
    _check("q4_gemm_q8", lib().q4_gemm_q8(_p(w_qs), _p(w_d), _p(x_qs), _p(x_ds), _p(y), _dt(y), M, N, K,
                                          _stream(stream)))
    return y


def dense_gemm(x, w_f16, y_dtype=torch.bfloat16, y=None, stream=None):
    N, K = w_f16.shape
    M = x.shape[0]
    y = _empty((M, N), y_dtype, x, stream) if y is None else y
    _check("dense_gemm", lib().dense_gemm(_p(x), _dt(x), _p(w_f16), _p(y), _dt(y), M, N, K, _stream(stream)))
    return y


# ---- dispatch -------------------------------------------------------------------------

def q4_dispatch_path(M, N, K, fmt=Q4_FMT_Q4_0, have_workspace=False) -> int:
    return int(lib().q4_dispatch_path(M, N, K, fmt, 1 if have_workspace else 0))


def q4_set_dispatch(key: int, value: int):
    _check("q4_set_dispatch", lib().q4_set_dispatch(key, value))


def q4_get_dispatch(key: int) -> int:
    v = ctypes.c_int64(0)
    _check("q4_get_dispatch", lib().q4_get_dispatch(key, ctypes.byref(v)))
    return int(v.value)
