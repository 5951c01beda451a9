"""CPU oracle for 4-bit block-quantised matrix multiply (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``q4_oracle.c`` (plain C, OpenMP over rows,
binary64 matmul) through ctypes and shares nothing with the HIP library: not
a header, not a helper, not a table.  The product library never loads it.

Every function takes and returns numpy arrays.  16-bit floating-point values
travel as ``uint16`` bit patterns so that no library conversion sneaks in.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (compiling the checker is not using it)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64


def build_sanitized(out: str) -> str:
    """The oracle built with clang's AddressSanitizer and
    UndefinedBehaviorSanitizer (serial: no OpenMP), for the sanitizer test."""
    if not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        tmp = out + ".tmp"
        subprocess.check_call(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
                               "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-std=c11",
                               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libsan",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("Q4_ORACLE_LIB")  # a planted-mistake build, for the mutation tests
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        sigs = {
            "or_q4_0_quantize": [_P, _I, _I, _P, _P],
            "or_q4_0_dequantize": [_P, _P, _I, _I, _P],
            "or_q4_0_dequantize_half": [_P, _P, _I, _I, ctypes.c_int, _P],
            "or_q8_1_quantize": [_P, _I, _I, _P, _P],
            "or_q8_1_dequantize": [_P, _P, _I, _I, _P],
            "or_q4q8_block_dots": [_P, _P, _I, _I, _I, _P],
            "or_q4q8_gemv": [_P, _P, _P, _P, _I, _I, _I, _P],
            "or_matmul_f64": [_P, _P, _I, _I, _I, _P],
            "or_matmul_f64_sampled": [_P, _P, _I, _I, _P, _P, _P],
            "or_affine4_quantize": [_P, _I, _I, _I, _P, _P, _P],
            "or_affine4_dequantize": [_P, _P, _P, _I, _I, _I, _P],
            "or_affine4_dequantize_half": [_P, _P, _P, _I, _I, _I, ctypes.c_int, _P],
            "or_affine8_quantize": [_P, _I, _I, _I, _P, _P, _P],
            "or_affine8_dequantize": [_P, _P, _P, _I, _I, _I, _P],
            "or_affine8_dequantize_half": [_P, _P, _P, _I, _I, _I, ctypes.c_int, _P],
            "or_f32_to_f16_array": [_P, _I, _P],
            "or_f16_to_f32_array": [_P, _I, _P],
            "or_f32_to_bf16_array": [_P, _I, _P],
            "or_bf16_to_f32_array": [_P, _I, _P],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = None
        lib.or_num_threads.argtypes = []
        lib.or_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().or_num_threads())


# ---- 16-bit float conversions (bit patterns) ------------------------------

def f32_to_f16_bits(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().or_f32_to_f16_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_bits_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().or_f16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


def f32_to_bf16_bits(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().or_f32_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(b):
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    _load().or_bf16_to_f32_array(_ptr(b), b.size, _ptr(out))
    return out


# ---- Q4_0 ------------------------------------------------------------------

def q4_0_quantize(w):
    """W float32 [N, K] -> (qs uint8 [N, K/32, 16], d uint16 [N, K/32])."""
    w = _c(w, np.float32)
    N, K = w.shape
    assert K % 32 == 0
    qs = np.empty((N, K // 32, 16), np.uint8)
    d = np.empty((N, K // 32), np.uint16)
    _load().or_q4_0_quantize(_ptr(w), N, K, _ptr(qs), _ptr(d))
    return qs, d


def q4_0_dequantize(qs, d):
    """Exact (q-8)*d as float64 [N, K]."""
    qs = _c(qs, np.uint8)
    d = _c(d, np.uint16)
    N, nb = d.shape
    K = nb * 32
    out = np.empty((N, K), np.float64)
    _load().or_q4_0_dequantize(_ptr(qs), _ptr(d), N, K, _ptr(out))
    return out


def q4_0_dequantize_half(qs, d, kind: str):
    """(q-8)*d rounded to 'f16' or 'bf16' (RNE), as uint16 bits [N, K]."""
    qs = _c(qs, np.uint8)
    d = _c(d, np.uint16)
    N, nb = d.shape
    K = nb * 32
    out = np.empty((N, K), np.uint16)
    _load().or_q4_0_dequantize_half(_ptr(qs), _ptr(d), N, K, {"f16": 0, "bf16": 1}[kind], _ptr(out))
    return out


# ---- Q8_1 ------------------------------------------------------------------

def q8_1_quantize(x):
    """X float32 [M, K] -> (qs int8 [M, K], ds uint16 [M, K/32, 2] = {d, s})."""
    x = _c(x, np.float32)
    M, K = x.shape
    assert K % 32 == 0
    qs = np.empty((M, K), np.int8)
    ds = np.empty((M, K // 32, 2), np.uint16)
    _load().or_q8_1_quantize(_ptr(x), M, K, _ptr(qs), _ptr(ds))
    return qs, ds


def q8_1_dequantize(qs, ds):
    qs = _c(qs, np.int8)
    ds = _c(ds, np.uint16)
    M, K = qs.shape
    out = np.empty((M, K), np.float64)
    _load().or_q8_1_dequantize(_ptr(qs), _ptr(ds), M, K, _ptr(out))
    return out


def q4q8_block_dots(wqs, xqs):
    """int32 isum [M, N, K/32] = sum_j (q4_j - 8) * q8_j."""
    wqs = _c(wqs, np.uint8)
    xqs = _c(xqs, np.int8)
    N, nb = wqs.shape[0], wqs.shape[1]
    M, K = xqs.shape
    assert K == nb * 32
    out = np.empty((M, N, nb), np.int32)
    _load().or_q4q8_block_dots(_ptr(wqs), _ptr(xqs), M, N, K, _ptr(out))
    return out


def q4q8_gemv(wqs, wd, xqs, xds):
    """float64 y [M, N] = sum_b d4 * d8 * isum."""
    wqs = _c(wqs, np.uint8)
    wd = _c(wd, np.uint16)
    xqs = _c(xqs, np.int8)
    xds = _c(xds, np.uint16)
    N = wd.shape[0]
    M, K = xqs.shape
    out = np.empty((M, N), np.float64)
    _load().or_q4q8_gemv(_ptr(wqs), _ptr(wd), _ptr(xqs), _ptr(xds), M, N, K, _ptr(out))
    return out


# ---- dense binary64 matmul --------------------------------------------------

def matmul_f64(x, w):
    """y [M, N] = x [M, K] . w [N, K]^T in binary64."""
    x = _c(x, np.float64)
    w = _c(w, np.float64)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    out = np.empty((M, N), np.float64)
    _load().or_matmul_f64(_ptr(x), _ptr(w), M, N, K, _ptr(out))
    return out


def matmul_f64_sampled(x, w, ms, ns):
    """y[i] = sum_k x[ms[i], k] * w[ns[i], k] in binary64."""
    x = _c(x, np.float64)
    w = _c(w, np.float64)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert ms.shape == ns.shape
    out = np.empty(ms.shape, np.float64)
    _load().or_matmul_f64_sampled(_ptr(x), _ptr(w), x.shape[1], ms.size, _ptr(ms), _ptr(ns), _ptr(out))
    return out


# ---- affine 4-bit -------------------------------------------------------------

def affine4_quantize(w_bf16_bits, group: int = 64):
    """W bf16 bits [N, K] -> (q uint8 [N, K/2], s uint16 [N, K/G], b uint16 [N, K/G])."""
    w = _c(w_bf16_bits, np.uint16)
    N, K = w.shape
    assert K % group == 0 and group % 2 == 0
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // group), np.uint16)
    b = np.empty((N, K // group), np.uint16)
    _load().or_affine4_quantize(_ptr(w), N, K, group, _ptr(q), _ptr(s), _ptr(b))
    return q, s, b


def affine4_dequantize(q, s, b, group: int = 64):
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    b = _c(b, np.uint16)
    N = q.shape[0]
    K = q.shape[1] * 2
    out = np.empty((N, K), np.float64)
    _load().or_affine4_dequantize(_ptr(q), _ptr(s), _ptr(b), N, K, group, _ptr(out))
    return out


def affine4_dequantize_half(q, s, b, kind: str, group: int = 64):
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    b = _c(b, np.uint16)
    N = q.shape[0]
    K = q.shape[1] * 2
    out = np.empty((N, K), np.uint16)
    _load().or_affine4_dequantize_half(_ptr(q), _ptr(s), _ptr(b), N, K, group,
                                       {"f16": 0, "bf16": 1}[kind], _ptr(out))
    return out


# ---- affine 8-bit -------------------------------------------------------------

def affine8_quantize(w_bf16_bits, group: int = 64):
    """W bf16 bits [N, K] -> (q uint8 [N, K], s uint16 [N, K/G], b uint16 [N, K/G])."""
    w = _c(w_bf16_bits, np.uint16)
    N, K = w.shape
    assert K % group == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty((N, K // group), np.uint16)
    b = np.empty((N, K // group), np.uint16)
    _load().or_affine8_quantize(_ptr(w), N, K, group, _ptr(q), _ptr(s), _ptr(b))
    return q, s, b


def affine8_dequantize(q, s, b, group: int = 64):
    """Exact q*s + b as float64 [N, K]."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    b = _c(b, np.uint16)
    N, K = q.shape
    out = np.empty((N, K), np.float64)
    _load().or_affine8_dequantize(_ptr(q), _ptr(s), _ptr(b), N, K, group, _ptr(out))
    return out


def affine8_dequantize_half(q, s, b, kind: str, group: int = 64):
    """q*s + b rounded to 'f16' or 'bf16' (RNE of the nearest binary32), as uint16 bits."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    b = _c(b, np.uint16)
    N, K = q.shape
    out = np.empty((N, K), np.uint16)
    _load().or_affine8_dequantize_half(_ptr(q), _ptr(s), _ptr(b), N, K, group,
                                       {"f16": 0, "bf16": 1}[kind], _ptr(out))
    return out


# ---- whole-path references ---------------------------------------------------

def rel_frobenius(y, ref) -> float:
    """||y - ref||_F / ||ref||_F in binary64."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((y - ref).ravel())
    return float(num / den) if den > 0 else float(num)
