"""Host-only checks of the C ABI: they run without a GPU.

* libq4.so loads and exports every function include/q4.h declares;
* every validation error is returned before any HIP call (fake, never
  dereferenced pointers are enough to reach them);
* the M-threshold dispatch predicate at its boundaries, through the API and
  through the environment overrides (read once per process, clamped).
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from gemv_q4_affine_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")

# fake device pointers: 16-byte aligned, never dereferenced by these tests
P = 0x10000
P2 = 0x20000
MIS = 0x10008  # 8-byte aligned only


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) == 30, names
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in q4.h but not exported"
    # and the binding covers them all with a signature
    assert set(names) == set(B.SIGNATURES), set(names) ^ set(B.SIGNATURES)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\S+)$", out, flags=re.M))
    assert set(names) <= exported


def test_version_and_status_strings():
    assert "gfx950" in B.version()
    for code in range(-8, 1):
        assert B.status_string(code) and B.status_string(code) != "unknown status"
    assert B.status_string(-99) == "unknown status"


L = None


def lib():
    global L
    if L is None:
        L = B.lib()
    return L


def test_quantize_validation():
    q = lib().q4_quantize
    assert q(None, B.Q4_F32, 4, 64, P, P, None) == B.Q4_ERR_NULL
    assert q(P, B.Q4_F32, 4, 64, None, P, None) == B.Q4_ERR_NULL
    assert q(P, B.Q4_F32, 4, 48, P, P, None) == B.Q4_ERR_SHAPE
    assert q(P, B.Q4_F32, 4, 0, P, P, None) == B.Q4_ERR_SHAPE
    assert q(P, B.Q4_F32, -1, 64, P, P, None) == B.Q4_ERR_SHAPE
    assert q(P, B.Q4_F32, 1 << 31, 64, P, P, None) == B.Q4_ERR_SHAPE
    assert q(P, B.Q4_F16, 4, 64, P, P, None) == B.Q4_ERR_DTYPE
    assert q(P, 7, 4, 64, P, P, None) == B.Q4_ERR_DTYPE
    assert q(MIS, B.Q4_F32, 4, 64, P, P, None) == B.Q4_ERR_ALIGN
    assert q(P, B.Q4_F32, 0, 64, P, P, None) == B.Q4_OK          # N == 0: no-op, no HIP call
    a = lib().q8_1_quantize_act
    assert a(P, B.Q4_BF16, 1, 40, P, P, None) == B.Q4_ERR_SHAPE
    assert a(P, B.Q4_BF16, 1, 64, P, MIS, None) == B.Q4_ERR_ALIGN
    assert a(P, B.Q4_F16, 1, 64, P, P, None) == B.Q4_ERR_DTYPE
    assert a(P, B.Q4_BF16, 0, 64, P, P, None) == B.Q4_OK
    f = lib().affine4_quantize
    assert f(P, B.Q4_BF16, 4, 64, 32, P, P, P, None) == B.Q4_ERR_SHAPE
    assert f(P, B.Q4_BF16, 4, 96, 64, P, P, P, None) == B.Q4_ERR_SHAPE
    assert f(P, B.Q4_BF16, 4, 128, 64, P, P, None, None) == B.Q4_ERR_NULL
    d = lib().q4_dequantize
    assert d(P, P, 4, 64, P, 9, None) == B.Q4_ERR_DTYPE
    assert d(P, P, 4, 65, P, B.Q4_F16, None) == B.Q4_ERR_SHAPE
    e = lib().affine4_dequantize
    assert e(P, P, P, 128, 4, 128, P, B.Q4_F16, None) == B.Q4_ERR_SHAPE


def test_gemv_validation():
    g = lib().q4_gemv
    assert g(P, P, P, P, P, 17, 8, 64, None) == B.Q4_ERR_SHAPE            # M above the GEMV limit
    assert g(P, P, P, P, P, 1, 8, 50, None) == B.Q4_ERR_SHAPE
    assert g(P, P, P, P, None, 1, 8, 64, None) == B.Q4_ERR_NULL
    assert g(P, P, MIS, P, P, 1, 8, 64, None) == B.Q4_ERR_ALIGN
    assert g(P, P, P, P, P, 0, 8, 64, None) == B.Q4_OK                  # M == 0
    assert g(P, P, P, P, P, 3, 0, 64, None) == B.Q4_OK                  # N == 0
    f = lib().q4_gemv_fused2
    assert f(P, P, 8, P, P, 8, P, P, P, P, 17, 64, None) == B.Q4_ERR_SHAPE
    assert f(P, P, 8, P, P, -8, P, P, P, P, 1, 64, None) == B.Q4_ERR_SHAPE
    assert f(P, P, 8, None, P, 8, P, P, P, P, 1, 64, None) == B.Q4_ERR_NULL
    assert f(P, P, 8, P, P, 8, P, P, P, P, 0, 64, None) == B.Q4_OK
    a = lib().q4_gemv_act
    assert a(P, P, P, B.Q4_BF16, P, 5, 8, 64, None) == B.Q4_ERR_SHAPE     # M above the fused-quantise limit
    assert a(P, P, P, B.Q4_F16, P, 1, 8, 64, None) == B.Q4_ERR_DTYPE
    assert a(P, P, P, B.Q4_BF16, P, 1, 8, 50, None) == B.Q4_ERR_SHAPE
    assert a(P, P, MIS, B.Q4_BF16, P, 1, 8, 64, None) == B.Q4_ERR_ALIGN
    assert a(P, P, None, B.Q4_F32, P, 1, 8, 64, None) == B.Q4_ERR_NULL
    assert a(P, P, P, B.Q4_BF16, P, 0, 8, 64, None) == B.Q4_OK
    assert a(P, P, P, B.Q4_BF16, P, 4, 0, 64, None) == B.Q4_OK
    f = lib().q4_gemv_fused2_act
    assert f(P, P, 8, P, P, 8, P, B.Q4_BF16, P, P, 5, 64, None) == B.Q4_ERR_SHAPE
    assert f(P, P, 8, P, P, 8, P, 9, P, P, 1, 64, None) == B.Q4_ERR_DTYPE
    assert f(P, P, 8, None, P, 8, P, B.Q4_BF16, P, P, 1, 64, None) == B.Q4_ERR_NULL
    assert f(P, P, 8, P, P, 8, P, B.Q4_BF16, P, P, 0, 64, None) == B.Q4_OK


def test_gemm_validation():
    g = lib().q4_gemm
    assert g(P, P, P, B.Q4_F16, P, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_DTYPE
    assert g(P, P, P, B.Q4_BF16, P, B.Q4_F16, 4, 8, 64, None, 0, None) == B.Q4_ERR_DTYPE
    assert g(P, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 60, None, 0, None) == B.Q4_ERR_SHAPE
    assert g(P, P, None, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_NULL
    assert g(P, P, P, B.Q4_BF16, MIS, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_ALIGN
    assert g(P, P, P, B.Q4_BF16, P, B.Q4_BF16, 0, 8, 64, None, 0, None) == B.Q4_OK
    a = lib().affine4_gemm
    assert a(P, P, P, 32, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_SHAPE
    assert a(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 96, None, 0, None) == B.Q4_ERR_SHAPE
    assert a(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 4, 0, 128, None, 0, None) == B.Q4_OK
    # the matrix-core path's workspace holds the X image (M and K rounded up
    # to the 128-row tile and the 64-wide K step, binary16) and the weight
    # image (9216 bytes per 256-column tile and K step)
    # image (9216 bytes per 256-column tile and K step)
    assert lib().q4_gemm_workspace_size(2048, 12288, 4096, 0) == 2048 * (4096 * 2 + 1) + 48 * 64 * 9216
    assert lib().q4_gemm_workspace_size(129, 300, 96, 0) == 256 * (128 * 2 + 1) + 2 * 2 * 9216
    assert lib().q4_gemm_workspace_size(4, 300, 4096, 0) == 0            # skinny: none
    assert lib().q4_gemm_workspace_size(4, 300, 4000, 0) == 0            # invalid K
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
    try:
        assert lib().q4_gemm_workspace_size(2048, 12288, 4096, 0) == 12288 * 4096 * 2
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    d = lib().dense_gemm
    assert d(P, B.Q4_BF16, P, P, B.Q4_BF16, 4, 8, 48, None) == B.Q4_ERR_SHAPE
    assert d(P, B.Q4_BF16, None, P, B.Q4_BF16, 4, 8, 64, None) == B.Q4_ERR_NULL


def test_affine8_validation():
    """Affine 8-bit entry points reject bad arguments on the host, before any HIP call."""
    q = lib().affine8_quantize
    assert q(P, B.Q4_F16, 8, 64, 64, P, P, P, None) == B.Q4_ERR_DTYPE
    assert q(P, B.Q4_BF16, 8, 64, 32, P, P, P, None) == B.Q4_ERR_SHAPE
    assert q(P, B.Q4_BF16, 8, 96, 64, P, P, P, None) == B.Q4_ERR_SHAPE
    assert q(P, B.Q4_BF16, 8, 64, 64, P, None, P, None) == B.Q4_ERR_NULL
    assert q(P, B.Q4_BF16, 0, 64, 64, P, P, P, None) == B.Q4_OK
    dq = lib().affine8_dequantize
    assert dq(P, P, P, 64, 8, 64, P, 7, None) == B.Q4_ERR_DTYPE
    assert dq(P, P, MIS, 64, 8, 64, P, B.Q4_F16, None) == B.Q4_ERR_ALIGN
    g = lib().affine8_gemm
    assert g(P, P, P, 64, P, B.Q4_F16, P, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_DTYPE
    assert g(P, P, P, 128, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_SHAPE
    assert g(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 96, None, 0, None) == B.Q4_ERR_SHAPE
    assert g(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 0, 8, 64, None, 0, None) == B.Q4_OK
    # above the fused kernels (f32 X: M > 16, bf16 X: M > 32) the matrix-core GEMM
    # builds its X image (128-row tiles, K*2 + 1 bytes a row) and weight image
    # (17408 bytes per 256 columns and 64 K) in the workspace: less room is
    # Q4_ERR_WORKSPACE, checked before any launch
    need = 128 * (64 * 2 + 1) + 17408
    assert g(P, P, P, 64, P, B.Q4_F32, P, B.Q4_BF16, 17, 8, 64, None, 0, None) == B.Q4_ERR_WORKSPACE
    assert g(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 33, 8, 64, None, 0, None) == B.Q4_ERR_WORKSPACE
    assert g(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 33, 8, 64, P, need - 1, None) == B.Q4_ERR_WORKSPACE
    assert g(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 33, 8, 64, MIS, need, None) == B.Q4_ERR_ALIGN
    ws = lib().affine8_gemm_workspace_size
    assert ws(16, 12288, 4096) == 0 and ws(17, 8, 96) == 0
    assert ws(17, 12288, 4096) >= 128 * (4096 * 2 + 1) + 48 * 64 * 17408
    # a forced dequantise-then-GEMM wants the binary16 weights
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
    try:
        assert ws(17, 12288, 4096) == 12288 * 4096 * 2
        assert g(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 33, 8, 64, P, 8 * 64 * 2 - 1, None) == B.Q4_ERR_WORKSPACE
        assert g(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 33, 8, 64, MIS, 8 * 64 * 2, None) == B.Q4_ERR_ALIGN
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)


def test_gemv_multi_validation():
    import ctypes
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    rows = lambda *v: (ctypes.c_int64 * len(v))(*v)
    m = lib().q4_gemv_multi
    a = lib().q4_gemv_multi_act
    three = (arr(P, P, P), arr(P, P, P), rows(8, 8, 8), arr(P, P, P))
    assert m(0, *three[:3], P, P, three[3], 1, 64, None) == B.Q4_ERR_ARG
    assert m(5, *three[:3], P, P, three[3], 1, 64, None) == B.Q4_ERR_ARG
    assert m(3, None, three[1], three[2], P, P, three[3], 1, 64, None) == B.Q4_ERR_NULL
    assert m(3, *three[:3], None, P, three[3], 1, 64, None) == B.Q4_ERR_NULL
    assert m(3, *three[:3], P, P, three[3], 17, 64, None) == B.Q4_ERR_SHAPE
    assert m(3, three[0], three[1], rows(8, -1, 8), P, P, three[3], 1, 64, None) == B.Q4_ERR_SHAPE
    assert m(3, arr(P, None, P), three[1], three[2], P, P, three[3], 1, 64, None) == B.Q4_ERR_NULL
    # an empty matrix may have NULL pointers
    assert m(3, arr(P, None, P), arr(P, None, P), rows(0, 0, 0), P, P, arr(P, None, P), 1, 64, None) == B.Q4_OK
    assert a(3, *three[:3], P, B.Q4_F16, three[3], 1, 64, None) == B.Q4_ERR_DTYPE
    assert a(3, *three[:3], P, B.Q4_BF16, three[3], 5, 64, None) == B.Q4_ERR_SHAPE
    assert a(3, *three[:3], None, B.Q4_BF16, three[3], 1, 64, None) == B.Q4_ERR_NULL
    assert a(3, *three[:3], MIS, B.Q4_BF16, three[3], 1, 64, None) == B.Q4_ERR_ALIGN
    assert a(3, *three[:3], P, B.Q4_BF16, three[3], 0, 64, None) == B.Q4_OK


def test_weight_image_validation_and_sizes():
    assert lib().q4_weight_image_size(12288, 4096, B.Q4_FMT_Q4_0) == 48 * 64 * 9216
    assert lib().q4_weight_image_size(300, 96, B.Q4_FMT_Q4_0) == 2 * 2 * 9216
    assert lib().q4_weight_image_size(300, 96, B.Q4_FMT_AFFINE4) == 0        # K % 64 != 0
    assert lib().q4_weight_image_size(300, 128, 5) == 0
    # affine 8-bit: 17408-byte chunks (codes of 256 columns x 64 K, then s and b)
    assert lib().q4_weight_image_size(12288, 4096, B.Q4_FMT_AFFINE8) == 48 * 64 * 17408
    assert lib().q4_weight_image_size(300, 128, B.Q4_FMT_AFFINE8) == 2 * 2 * 17408
    assert lib().q4_weight_image_size(300, 96, B.Q4_FMT_AFFINE8) == 0
    for M in (1, 33, 2048):
        assert lib().q4_gemm_workspace_size(M, 12288, 4096, B.Q4_FMT_AFFINE8) == \
            lib().affine8_gemm_workspace_size(M, 12288, 4096)
    assert lib().q4_gemm_image_workspace_size(2048, 4096) == 2048 * (4096 * 2 + 1)
    assert lib().q4_gemm_image_workspace_size(129, 96) == 256 * (128 * 2 + 1)
    p = lib().q4_pack_weight_image
    assert p(5, P, P, None, 8, 64, P, None) == B.Q4_ERR_ARG
    assert p(B.Q4_FMT_Q4_0, P, P, None, 8, 48, P, None) == B.Q4_ERR_SHAPE
    assert p(B.Q4_FMT_AFFINE4, P, P, P, 8, 96, P, None) == B.Q4_ERR_SHAPE
    assert p(B.Q4_FMT_AFFINE4, P, P, None, 8, 128, P, None) == B.Q4_ERR_NULL   # affine needs biases
    assert p(B.Q4_FMT_AFFINE8, P, P, None, 8, 128, P, None) == B.Q4_ERR_NULL
    assert p(B.Q4_FMT_AFFINE8, P, P, P, 8, 96, P, None) == B.Q4_ERR_SHAPE
    assert p(B.Q4_FMT_Q4_0, P, P, None, 8, 64, MIS, None) == B.Q4_ERR_ALIGN
    assert p(B.Q4_FMT_Q4_0, P, P, None, 0, 64, P, None) == B.Q4_OK
    g = lib().q4_gemm_image
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_F16, P, B.Q4_BF16, 4, 8, 64, P2, 1 << 20, None) == B.Q4_ERR_DTYPE
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_WORKSPACE
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, P2, 128 * (64 * 2 + 1) - 1, None) == B.Q4_ERR_WORKSPACE
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, MIS, 1 << 20, None) == B.Q4_ERR_ALIGN
    assert g(B.Q4_FMT_Q4_0, None, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, P2, 1 << 20, None) == B.Q4_ERR_NULL
    assert g(B.Q4_FMT_AFFINE4, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 96, P2, 1 << 20, None) == B.Q4_ERR_SHAPE
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_BF16, P, B.Q4_BF16, 0, 8, 64, None, 0, None) == B.Q4_OK


def test_gemm_q8_validation():
    g = lib().q4_gemm_q8
    assert g(P, P, P, P, P, B.Q4_F16, 4, 8, 64, None) == B.Q4_ERR_DTYPE
    assert g(P, P, P, P, P, B.Q4_F32, 4, 8, 48, None) == B.Q4_ERR_SHAPE
    assert g(P, P, P, P, P, B.Q4_F32, -1, 8, 64, None) == B.Q4_ERR_SHAPE
    assert g(P, P, None, P, P, B.Q4_F32, 4, 8, 64, None) == B.Q4_ERR_NULL
    assert g(P, P, P, MIS, P, B.Q4_F32, 4, 8, 64, None) == B.Q4_ERR_ALIGN
    assert g(P, P, P, P, P, B.Q4_BF16, 0, 8, 64, None) == B.Q4_OK
    assert g(None, None, None, None, None, B.Q4_BF16, 4, 0, 64, None) == B.Q4_OK


def test_noalloc_gemm_rejects_before_any_device_call():
    """q4_gemm_image_noalloc: the same argument checks as q4_gemm_image, and
    an X image beyond the fixed scratch is refused with its own status before
    anything is enqueued (no GPU here, so reaching a HIP call would fail
    differently)."""
    assert B.Q4_NOALLOC_SCRATCH_BYTES == 33 << 20
    g = lib().q4_gemm_image_noalloc
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_F16, P, B.Q4_BF16, 4, 8, 64, None) == B.Q4_ERR_DTYPE
    assert g(5, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None) == B.Q4_ERR_ARG
    assert g(B.Q4_FMT_AFFINE4, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 96, None) == B.Q4_ERR_SHAPE
    assert g(B.Q4_FMT_Q4_0, None, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None) == B.Q4_ERR_NULL
    assert g(B.Q4_FMT_Q4_0, P, MIS, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None) == B.Q4_ERR_ALIGN
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_BF16, P, B.Q4_BF16, 0, 8, 64, None) == B.Q4_OK
    # X image: ceil(M/128)*128 * (ceil(K/64)*64 * 2 + 1) bytes against 33 MiB
    assert lib().q4_gemm_image_workspace_size(4096, 4096) <= B.Q4_NOALLOC_SCRATCH_BYTES
    assert lib().q4_gemm_image_workspace_size(4097, 4096) > B.Q4_NOALLOC_SCRATCH_BYTES
    assert g(B.Q4_FMT_Q4_0, P, P, B.Q4_BF16, P, B.Q4_BF16, 4097, 256, 4096, None) == B.Q4_ERR_SCRATCH
    assert g(B.Q4_FMT_AFFINE4, P, P, B.Q4_F32, P, B.Q4_F32, 8192, 256, 4096, None) == B.Q4_ERR_SCRATCH
    assert "scratch" in B.status_string(B.Q4_ERR_SCRATCH)


def test_forced_dequant_path_without_workspace_is_an_error():
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
    try:
        g = lib().q4_gemm
        assert g(P, P, P, B.Q4_BF16, P, B.Q4_BF16, 512, 256, 64, None, 0, None) == B.Q4_ERR_WORKSPACE
        assert g(P, P, P, B.Q4_BF16, P, B.Q4_BF16, 512, 256, 64, P2, 100, None) == B.Q4_ERR_WORKSPACE
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)


def test_dispatch_predicate_boundaries():
    skinny = B.q4_get_dispatch(B.Q4_KEY_SKINNY_MAX_M)
    assert 1 <= skinny <= 64
    for fmt, K in ((B.Q4_FMT_Q4_0, 4096), (B.Q4_FMT_AFFINE4, 4096)):
        assert B.q4_dispatch_path(1, 12288, K, fmt) == B.Q4_PATH_SKINNY
        assert B.q4_dispatch_path(skinny, 12288, K, fmt) == B.Q4_PATH_SKINNY
        assert B.q4_dispatch_path(skinny + 1, 12288, K, fmt) == B.Q4_PATH_MFMA
        assert B.q4_dispatch_path(8192, 12288, K, fmt) == B.Q4_PATH_MFMA
    assert B.q4_dispatch_path(4, 8, 48, B.Q4_FMT_Q4_0) == B.Q4_ERR_SHAPE
    assert B.q4_dispatch_path(4, 8, 96, B.Q4_FMT_AFFINE4) == B.Q4_ERR_SHAPE
    assert B.q4_dispatch_path(4, 8, 64, 5) == B.Q4_ERR_ARG
    # a dequantise threshold only applies with a workspace
    old = B.q4_get_dispatch(B.Q4_KEY_DEQUANT_MIN_M)
    try:
        B.q4_set_dispatch(B.Q4_KEY_DEQUANT_MIN_M, 512)
        assert B.q4_dispatch_path(511, 12288, 4096, have_workspace=True) == B.Q4_PATH_MFMA
        assert B.q4_dispatch_path(512, 12288, 4096, have_workspace=True) == B.Q4_PATH_DEQUANT_GEMM
        assert B.q4_dispatch_path(513, 12288, 4096, have_workspace=False) == B.Q4_PATH_MFMA
    finally:
        B.q4_set_dispatch(B.Q4_KEY_DEQUANT_MIN_M, old)
    # set/get clamp and reject
    B.q4_set_dispatch(B.Q4_KEY_SKINNY_MAX_M, 1000)
    assert B.q4_get_dispatch(B.Q4_KEY_SKINNY_MAX_M) == 64
    B.q4_set_dispatch(B.Q4_KEY_SKINNY_MAX_M, skinny)
    with pytest.raises(B.Q4Error):
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, 9)
    with pytest.raises(B.Q4Error):
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, 5)
    with pytest.raises(B.Q4Error):
        B.q4_set_dispatch(77, 1)
    # affine 8-bit: fused kernels up to Q4_KEY_AFFINE8_FUSED_MAX_M (default 32),
    # the matrix-core GEMM above; SKINNY, MFMA and DEQUANT_GEMM can be forced
    A8 = B.Q4_FMT_AFFINE8
    assert B.q4_get_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M) == 32
    assert B.q4_dispatch_path(32, 4096, 4096, A8) == B.Q4_PATH_SKINNY
    assert B.q4_dispatch_path(33, 4096, 4096, A8) == B.Q4_PATH_MFMA
    assert B.q4_dispatch_path(1, 4096, 4064, A8) == B.Q4_ERR_SHAPE     # K % 64
    ws8 = lib().affine8_gemm_workspace_size
    B.q4_set_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M, 4)
    try:
        assert B.q4_dispatch_path(5, 4096, 4096, A8) == B.Q4_PATH_MFMA
        assert ws8(5, 4096, 4096) >= 128 * (4096 * 2 + 1) + 16 * 64 * 17408 and ws8(4, 4096, 4096) == 0
        assert lib().affine8_gemm(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_BF16, 5, 8, 64, None, 0, None) == \
            B.Q4_ERR_WORKSPACE
        B.q4_set_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M, 1000)
        assert B.q4_get_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M) == 32
    finally:
        B.q4_set_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M, 32)
    for forced, want_small, want_big in ((B.Q4_PATH_DEQUANT_GEMM, B.Q4_PATH_DEQUANT_GEMM, B.Q4_PATH_DEQUANT_GEMM),
                                         (B.Q4_PATH_SKINNY, B.Q4_PATH_SKINNY, B.Q4_PATH_SKINNY),
                                         (B.Q4_PATH_MFMA, B.Q4_PATH_MFMA, B.Q4_PATH_MFMA),
                                         (B.Q4_PATH_INT8, B.Q4_PATH_SKINNY, B.Q4_PATH_MFMA)):
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, forced)
        try:
            assert B.q4_dispatch_path(1, 64, 64, A8) == want_small
            assert B.q4_dispatch_path(2048, 64, 64, A8) == want_big
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    # the Q8_1 paths: forced only, Q4_0 only; INT8 wants the Q8_1 planes as workspace
    g = lib().q4_gemm
    a = lib().affine4_gemm
    for path in (B.Q4_PATH_GEMV, B.Q4_PATH_INT8):
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, path)
        try:
            assert B.q4_dispatch_path(8, 64, 64) == path
            assert a(P, P, P, 64, P, B.Q4_BF16, P, B.Q4_F32, 4, 8, 128, P2, 1 << 20, None) == B.Q4_ERR_ARG
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_GEMV)
    try:
        assert B.q4_gemm_workspace_size(4, 64, 64) == 0
        assert g(P, P, P, B.Q4_BF16, P, B.Q4_F32, 5, 8, 64, None, 0, None) == B.Q4_ERR_ARG      # M > 4
        assert g(P, P, P, B.Q4_BF16, P, B.Q4_BF16, 4, 8, 64, None, 0, None) == B.Q4_ERR_ARG     # bf16 y
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_INT8)
    try:
        assert B.q4_gemm_workspace_size(100, 64, 4096) == 100 * 4096 + 100 * 128 * 4
        need = 4 * 64 + 4 * 2 * 4
        assert g(P, P, P, B.Q4_BF16, P, B.Q4_F32, 4, 8, 64, None, 0, None) == B.Q4_ERR_WORKSPACE
        assert g(P, P, P, B.Q4_BF16, P, B.Q4_F32, 4, 8, 64, P2, need - 1, None) == B.Q4_ERR_WORKSPACE
        assert g(P, P, P, B.Q4_BF16, P, B.Q4_F32, 4, 8, 64, MIS, need, None) == B.Q4_ERR_ALIGN
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    # tile rows: 128 (default) or 256, nothing else
    assert B.q4_get_dispatch(B.Q4_KEY_TILE_ROWS) == 128
    for bad in (0, 64, 192, 512):
        with pytest.raises(B.Q4Error):
            B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, bad)
    B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, 256)
    assert B.q4_get_dispatch(B.Q4_KEY_TILE_ROWS) == 256
    B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, 128)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)
    try:
        assert B.q4_dispatch_path(1, 64, 64) == B.Q4_PATH_MFMA
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)


_ENV_PROBE = r"""
import sys
sys.path.insert(0, {root!r})
from gemv_q4_affine_amd import binding as B
print(B.q4_get_dispatch(B.Q4_KEY_SKINNY_MAX_M), B.q4_get_dispatch(B.Q4_KEY_DEQUANT_MIN_M),
      B.q4_get_dispatch(B.Q4_KEY_FORCE_PATH),
      B.q4_dispatch_path(19, 4096, 4096), B.q4_dispatch_path(64, 4096, 4096, have_workspace=True),
      int(B.q4_gemm_workspace_size(64, 4096, 4096) > 0),
      B.q4_get_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M), B.q4_dispatch_path(20, 4096, 4096, B.Q4_FMT_AFFINE8))
"""


@pytest.mark.parametrize("env,expect", [
    ({"Q4_SKINNY_MAX_M": "1"}, (1, None, -1, B.Q4_PATH_MFMA, B.Q4_PATH_MFMA)),
    ({"Q4_SKINNY_MAX_M": "500"}, (64, None, -1, B.Q4_PATH_SKINNY, B.Q4_PATH_SKINNY)),
    ({"Q4_SKINNY_MAX_M": "-3"}, (0, None, -1, B.Q4_PATH_MFMA, B.Q4_PATH_MFMA)),
    ({"Q4_SKINNY_MAX_M": "8", "Q4_DEQUANT_MIN_M": "64"}, (8, 64, -1, B.Q4_PATH_MFMA, B.Q4_PATH_DEQUANT_GEMM)),
    ({"Q4_FORCE_PATH": "3"}, (None, None, 3, B.Q4_PATH_DEQUANT_GEMM, B.Q4_PATH_DEQUANT_GEMM)),
    ({"Q4_FORCE_PATH": "0"}, (None, None, 0, B.Q4_PATH_GEMV, B.Q4_PATH_GEMV, 0)),
    ({"Q4_FORCE_PATH": "4"}, (None, None, 4, B.Q4_PATH_INT8, B.Q4_PATH_INT8, 1)),
    # values the setter rejects leave the automatic dispatch (17: no such path;
    # SKINNY up to 64 rows, with room for the MFMA path that binary32 X takes
    # above 16)
    ({"Q4_FORCE_PATH": "17"}, (None, None, -1, B.Q4_PATH_SKINNY, B.Q4_PATH_SKINNY, 1)),
    ({"Q4_FORCE_PATH": "-5"}, (None, None, -1, B.Q4_PATH_SKINNY, B.Q4_PATH_SKINNY, 1)),
    ({"Q4_FORCE_PATH": "junk"}, (None, None, -1, None, None)),
    ({"Q4_AFFINE8_FUSED_MAX_M": "16"}, (None, None, -1, None, None, None, 16, B.Q4_PATH_MFMA)),
    ({"Q4_AFFINE8_FUSED_MAX_M": "99"}, (None, None, -1, None, None, None, 32, B.Q4_PATH_SKINNY)),
])
def test_dispatch_environment_overrides(env, expect):
    full = dict(os.environ)
    for k in ("Q4_SKINNY_MAX_M", "Q4_DEQUANT_MIN_M", "Q4_FORCE_PATH", "Q4_AFFINE8_FUSED_MAX_M"):
        full.pop(k, None)
    full.update(env)
    out = subprocess.run([sys.executable, "-c", _ENV_PROBE.format(root=ROOT)], env=full, capture_output=True,
                         text=True, check=True).stdout.split()
    got = tuple(int(v) for v in out)
    for g, e in zip(got, expect):
        if e is not None:
            assert g == e, (env, got, expect)
