"""q4_gemm_image_noalloc, the entry point for callers that cannot allocate,
through the C ABI against q4_gemm_image on a torch-allocated workspace of the
same size (the same kernels, so the same bits).  Two calls in a row, the
second with a smaller input, so that the second runs on scratch that still
holds the first call's larger X image."""
import ctypes

import numpy as np
import pytest
import torch

from gemv_q4_affine_amd import binding as B
from gemv_q4_affine_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _image(rng, fmt, N, K):
    w = torch.from_numpy(synth.weights(rng, N, K)).cuda()
    if fmt == B.Q4_FMT_Q4_0:
        qs, d = B.q4_quantize(w)
        return B.q4_pack_weight_image(qs, d, fmt=fmt)
    if fmt == B.Q4_FMT_AFFINE8:
        q, s, b = B.affine8_quantize(w.to(torch.bfloat16))
    else:
        q, s, b = B.affine4_quantize(w.to(torch.bfloat16), 64)
    return B.q4_pack_weight_image(q, s, b, fmt=fmt)


def _codes(x, y):
    xdt = B.Q4_BF16 if x.dtype == torch.bfloat16 else B.Q4_F32
    ydt = B.Q4_BF16 if y.dtype == torch.bfloat16 else B.Q4_F32
    return xdt, ydt


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _call_noalloc(fmt, img, x, y, N):
    M, K = x.shape
    xdt, ydt = _codes(x, y)
    return B.lib().q4_gemm_image_noalloc(fmt, img.data_ptr(), x.data_ptr(), xdt, y.data_ptr(), ydt, M, N, K,
                                         _stream())


def _call_workspace(fmt, img, x, y, N, ws):
    M, K = x.shape
    xdt, ydt = _codes(x, y)
    return B.lib().q4_gemm_image(fmt, img.data_ptr(), x.data_ptr(), xdt, y.data_ptr(), ydt, M, N, K,
                                 ws.data_ptr(), ws.numel(), _stream())


@pytest.mark.parametrize("fmt,N,K,calls", [
    # a prefill-sized call (16 MiB X image), then a ragged small one that also
    # uses the split-K partial results after the X image
    (B.Q4_FMT_Q4_0, 12288, 4096, [(2048, torch.bfloat16, torch.bfloat16), (77, torch.bfloat16, torch.float32)]),
    (B.Q4_FMT_AFFINE4, 4160, 2048, [(1000, torch.float32, torch.float32), (33, torch.bfloat16, torch.bfloat16)]),
    (B.Q4_FMT_AFFINE8, 2304, 1024, [(600, torch.bfloat16, torch.bfloat16), (40, torch.float32, torch.float32)]),
])
def test_noalloc_matches_workspace_entry_point(fmt, N, K, calls):
    rng = np.random.default_rng(N + K)
    img = _image(rng, fmt, N, K)
    ws = torch.empty(B.Q4_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    for M, xdt, ydt in calls:
        _say(f"noalloc fmt={fmt} M={M} N={N} K={K} x={xdt} y={ydt}")
        x = torch.from_numpy(synth.activations(rng, M, K)).cuda().to(xdt)
        y_ws = torch.full((M, N), float("nan"), dtype=ydt, device="cuda")
        y_na = torch.full((M, N), float("nan"), dtype=ydt, device="cuda")
        torch.cuda.synchronize()
        assert _call_noalloc(fmt, img, x, y_na, N) == B.Q4_OK
        torch.cuda.synchronize()
        assert _call_workspace(fmt, img, x, y_ws, N, ws) == B.Q4_OK
        torch.cuda.synchronize()
        assert bool(torch.isfinite(y_ws.float()).all())
        assert torch.equal(y_ws, y_na), (M, (y_ws.float() - y_na.float()).abs().max().item())


def test_noalloc_limit_is_an_error_on_the_gpu():
    """M beyond the scratch: Q4_ERR_SCRATCH, nothing enqueued, output untouched."""
    N, K = 256, 4096
    img = _image(np.random.default_rng(1), B.Q4_FMT_Q4_0, N, K)
    x = torch.zeros((4097, K), dtype=torch.bfloat16, device="cuda")
    y = torch.full((4097, N), 3.0, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    assert _call_noalloc(B.Q4_FMT_Q4_0, img, x, y, N) == B.Q4_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
