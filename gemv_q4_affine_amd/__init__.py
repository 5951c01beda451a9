"""MI355X (gfx950) library for matrix multiply against 4-bit block-quantised
weights: Q4_0 and affine-4 (group 64) GEMV / GEMM behind the C ABI of
include/q4.h.  ``binding`` is the thin ctypes layer over libq4.so."""
from .binding import (  # noqa: F401
    Q4Error,
    affine4_dequantize,
    affine4_gemm,
    affine4_quantize,
    dense_gemm,
    q4_dequantize,
    q4_dispatch_path,
    q4_gemm,
    q4_gemm_workspace_size,
    q4_gemv,
    q4_gemv_fused2,
    q4_get_dispatch,
    q4_quantize,
    q4_set_dispatch,
    q8_1_quantize_act,
    status_string,
    version,
)
