"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: bit-exact for codes, packing, dequantised values and integer block dots;
relative Frobenius error <= 2e-3 against the binary64 oracle for float
outputs (bf16 or fp32 output).  GEMV outputs are fp32 and are also held to a
tighter 1e-5, derived from fp32 accumulation of K/32 exact block terms.

Inputs come from gemv_q4_affine_amd.synth (seeded); every expected value is
computed by oracle/ on the same host arrays.  Full-size configurations are
checked on sampled outputs the oracle computes one by one.
"""
import hashlib
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from gemv_q4_affine_amd import binding as B
from gemv_q4_affine_amd import synth

pytestmark = pytest.mark.gpu

BAR = 2e-3          # relative Frobenius bar for float outputs
GEMV_TIGHT = 1e-5   # fp32 GEMV against binary64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    a = t.numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def bf16_dev(x_f32: np.ndarray) -> torch.Tensor:
    return dev(synth.bf16_bits(x_f32)).view(torch.bfloat16)


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel(y, ref):
    return oracle.rel_frobenius(y, ref)


# ---------------------------------------------------------------------------
# quantisers and dequantisers: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(256, 512), (37, 96), (1, 32), (12288, 4096)])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_q4_quantize_bitexact(N, K, wdt):
    say(f"q4_quantize N={N} K={K} {wdt}")
    rng = np.random.default_rng(N + K)
    W = synth.weights(rng, N, K)
    W[0, :8] = 0.0                      # a partly zero block
    if N > 1:
        W[1, :32] = 0.0                 # an all-zero block (d = -0)
    if wdt == "bf16":
        Wb = synth.bf16_bits(W)
        Wref = synth.bf16_bits_to_f32(Wb)
        wt = dev(Wb).view(torch.bfloat16)
    else:
        Wref = W
        wt = dev(W)
    qs, d = B.q4_quantize(wt)
    torch.cuda.synchronize()
    rqs, rd = oracle.q4_0_quantize(Wref)
    assert np.array_equal(host(qs), rqs)
    assert np.array_equal(host(d, np.uint16), rd)


def _golden_q4_matrix():
    path = os.path.join(os.path.dirname(__file__), "golden", "q4_0_blocks.txt")
    cases = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, ws, dhex, qhex = [p.strip() for p in line.split("|")]
        w = np.zeros(32, np.float32)
        if ws:
            for item in ws.split(","):
                i, v = item.split("=")
                w[int(i)] = np.float32(float(v))
        cases.append((w, int(dhex, 16), bytes.fromhex(qhex.replace(" ", ""))))
    return cases


def test_q4_quantize_golden_blocks_on_gpu():
    cases = _golden_q4_matrix()
    W = np.concatenate([c[0] for c in cases]).reshape(1, -1)
    qs, d = B.q4_quantize(dev(W))
    torch.cuda.synchronize()
    qs, d = host(qs), host(d, np.uint16)
    for b, (_, dbits, qbytes) in enumerate(cases):
        assert int(d[0, b]) == dbits
        assert bytes(qs[0, b]) == qbytes


@pytest.mark.parametrize("M,K", [(1, 4096), (7, 544), (16, 2048), (3, 32)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_q8_1_quantize_bitexact(M, K, xdt):
    say(f"q8_1 M={M} K={K} {xdt}")
    rng = np.random.default_rng(M * 7 + K)
    X = synth.activations(rng, M, K)
    X[0, :32] = 0.0
    X[-1, 32 % K:64 % K or K] *= 1e-3
    if xdt == "bf16":
        Xb = synth.bf16_bits(X)
        Xref = synth.bf16_bits_to_f32(Xb)
        xt = dev(Xb).view(torch.bfloat16)
    else:
        Xref, xt = X, dev(X)
    qs, ds = B.q8_1_quantize_act(xt)
    torch.cuda.synchronize()
    rqs, rds = oracle.q8_1_quantize(Xref)
    assert np.array_equal(host(qs), rqs)
    assert np.array_equal(host(ds, np.uint16), rds)


def test_q8_1_golden_halves():
    # values with exact .5 products: d = 1 (amax 127) -> round half away from zero
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5]
    qs, ds = B.q8_1_quantize_act(dev(x))
    torch.cuda.synchronize()
    assert host(qs)[0, :6].tolist() == [127, 3, -3, 1, -1, 2]
    assert host(ds, np.uint16)[0, 0].tolist() == [0x3C00, 0x5808]


@pytest.mark.parametrize("N,K", [(64, 128), (33, 192), (12288, 4096)])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_affine4_quantize_bitexact(N, K, wdt):
    say(f"affine4_quantize N={N} K={K} {wdt}")
    rng = np.random.default_rng(N * 3 + K)
    W = synth.weights(rng, N, K)
    W[0, :64] = 0.25                    # constant group: s = 0
    Wb = synth.bf16_bits(W)
    wt = dev(Wb).view(torch.bfloat16) if wdt == "bf16" else dev(W)
    q, s, b = B.affine4_quantize(wt)
    torch.cuda.synchronize()
    # the f32 entry point first rounds to bf16 with the same RNE the oracle uses
    rq, rs, rb = oracle.affine4_quantize(oracle.f32_to_bf16_bits(W), 64)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s, np.uint16), rs)
    assert np.array_equal(host(b, np.uint16), rb)


@pytest.mark.parametrize("N,K", [(37, 96), (12288, 4096)])
def test_dequantize_bitexact(N, K):
    say(f"dequantize N={N} K={K}")
    rng = np.random.default_rng(5)
    W = synth.weights(rng, N, K)
    qs, d = oracle.q4_0_quantize(W)
    tq, td = dev(qs), dev(d)
    for kind, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        got = host(B.q4_dequantize(tq, td, out_dtype=dt), np.uint16)
        assert np.array_equal(got, oracle.q4_0_dequantize_half(qs, d, kind)), kind
    got32 = host(B.q4_dequantize(tq, td, out_dtype=torch.float32)).astype(np.float64)
    assert np.array_equal(got32, oracle.q4_0_dequantize(qs, d))
    if K % 64 == 0:
        q, s, b = oracle.affine4_quantize(synth.bf16_bits(W), 64)
        aq, as_, ab = dev(q), dev(s), dev(b)
        for kind, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
            got = host(B.affine4_dequantize(aq, as_, ab, out_dtype=dt), np.uint16)
            assert np.array_equal(got, oracle.affine4_dequantize_half(q, s, b, kind)), kind
        got32 = host(B.affine4_dequantize(aq, as_, ab, out_dtype=torch.float32))
        assert np.array_equal(got32, oracle.affine4_dequantize(q, s, b).astype(np.float32))


# ---------------------------------------------------------------------------
# decode GEMV
# ---------------------------------------------------------------------------

def test_gemv_unit_scales_are_exact_integer_sums():
    """d4 = d8 = 1: the fp32 output is the integer sum of block dots, bit-exact."""
    rng = np.random.default_rng(31)
    for (M, N, K) in [(1, 300, 4096), (3, 65, 32), (2, 129, 4128), (16, 17, 544)]:
        say(f"gemv unit scales M={M} N={N} K={K}")
        wqs = rng.integers(0, 256, (N, K // 32, 16), dtype=np.uint8)
        wd = np.full((N, K // 32), 0x3C00, np.uint16)
        xqs = rng.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
        xds = np.zeros((M, K // 32, 2), np.uint16)
        xds[..., 0] = 0x3C00
        y = B.q4_gemv(dev(wqs), dev(wd), dev(xqs), dev(xds))
        torch.cuda.synchronize()
        isum = oracle.q4q8_block_dots(wqs, xqs).astype(np.int64).sum(axis=2)   # [M, N]
        assert np.array_equal(host(y).astype(np.int64), isum)
        assert np.array_equal(host(y), isum.astype(np.float32))


def test_gemv_block_dot_extremes():
    N, K = 2, 32
    wqs = np.zeros((N, 1, 16), np.uint8)
    wqs[1] = 0xFF
    wd = np.full((N, 1), 0x3C00, np.uint16)
    for v, want in ((-127, [32512, -28448]), (127, [-32512, 28448])):
        xqs = np.full((1, K), v, np.int8)
        xds = np.array([[[0x3C00, 0]]], np.uint16)
        y = host(B.q4_gemv(dev(wqs), dev(wd), dev(xqs), dev(xds)))
        assert y[0].tolist() == want


def _gemv_case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    wqs, wd = oracle.q4_0_quantize(W)
    xqs, xds = oracle.q8_1_quantize(X)
    return wqs, wd, xqs, xds


def test_gemv_decode_config():
    wl = synth.DECODE
    say(f"gemv decode config N={wl.N} K={wl.K}")
    W, X = synth.workload_inputs(wl)
    wqs, wd = oracle.q4_0_quantize(W)
    # the activation is quantised on the GPU (bit-checked) and fed to the GEMV
    xq, xd = B.q8_1_quantize_act(dev(X))
    xqs, xds = oracle.q8_1_quantize(X)
    assert np.array_equal(host(xq), xqs) and np.array_equal(host(xd, np.uint16), xds)
    y = B.q4_gemv(dev(wqs), dev(wd), xq, xd)
    ref = oracle.q4q8_gemv(wqs, wd, xqs, xds)
    e = rel(host(y).astype(np.float64), ref)
    say(f"  rel err {e:.3e}")
    assert e <= BAR and e <= GEMV_TIGHT


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_gemv_all_m_ragged(M):
    for (N, K) in [(257, 544), (1000, 4128)]:
        wqs, wd, xqs, xds = _gemv_case(M, N, K, seed=M * 1000 + N)
        y = host(B.q4_gemv(dev(wqs), dev(wd), dev(xqs), dev(xds))).astype(np.float64)
        ref = oracle.q4q8_gemv(wqs, wd, xqs, xds)
        assert rel(y, ref) <= GEMV_TIGHT, (M, N, K)


@pytest.mark.parametrize("M,N0,N1,K", [(1, 12288, 12288, 4096), (3, 512, 300, 2048), (1, 1, 17, 64), (16, 64, 8192, 2048)])
def test_fused2_bit_identical_to_two_gemvs(M, N0, N1, K):
    say(f"fused2 M={M} N0={N0} N1={N1} K={K}")
    w0qs, w0d, xqs, xds = _gemv_case(M, N0, K, seed=N0)
    rng = np.random.default_rng(N1 + 1)
    w1qs, w1d = oracle.q4_0_quantize(synth.weights(rng, N1, K))
    t = [dev(a) for a in (w0qs, w0d, w1qs, w1d, xqs, xds)]
    y0, y1 = B.q4_gemv_fused2(t[0], t[1], t[2], t[3], t[4], t[5])
    z0 = B.q4_gemv(t[0], t[1], t[4], t[5])
    z1 = B.q4_gemv(t[2], t[3], t[4], t[5])
    assert torch.equal(y0, z0) and torch.equal(y1, z1)
    assert rel(host(y1).astype(np.float64), oracle.q4q8_gemv(w1qs, w1d, xqs, xds)) <= GEMV_TIGHT


@pytest.mark.parametrize("M,N,K", [(1, 12288, 4096), (1, 300, 96), (2, 1000, 4128), (3, 257, 544),
                                   (4, 640, 14336), (1, 64, 65536), (4, 3, 32), (1, 8192, 8192)])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_gemv_act_bit_identical_to_quantise_then_gemv(M, N, K, xdt):
    """The GEMV that quantises its own activation gives the bits of
    q8_1_quantize_act followed by q4_gemv, and the oracle's value."""
    say(f"gemv_act M={M} N={N} K={K} {xdt}")
    rng = np.random.default_rng(M * 7 + N + K)
    wqs, wd = oracle.q4_0_quantize(synth.weights(rng, N, K))
    X = synth.activations(rng, M, K)
    x = bf16_dev(X) if xdt == "bf16" else dev(X.astype(np.float32))
    Xh = synth.bf16_bits_to_f32(synth.bf16_bits(X)) if xdt == "bf16" else X.astype(np.float32)
    tw = (dev(wqs), dev(wd))
    y = B.q4_gemv_act(*tw, x)
    xq, xd = B.q8_1_quantize_act(x)
    assert torch.equal(y, B.q4_gemv(*tw, xq, xd))
    xqs, xds = oracle.q8_1_quantize(Xh)
    assert rel(host(y).astype(np.float64), oracle.q4q8_gemv(wqs, wd, xqs, xds)) <= GEMV_TIGHT


@pytest.mark.parametrize("M,N0,N1,K", [(1, 14336, 14336, 4096), (2, 512, 300, 2048), (4, 1, 17, 64)])
def test_gemv_fused2_act_bit_identical(M, N0, N1, K):
    say(f"fused2_act M={M} N0={N0} N1={N1} K={K}")
    rng = np.random.default_rng(N0 + N1)
    w0 = oracle.q4_0_quantize(synth.weights(rng, N0, K))
    w1 = oracle.q4_0_quantize(synth.weights(rng, N1, K))
    x = bf16_dev(synth.activations(rng, M, K))
    t = [dev(a) for a in (*w0, *w1)]
    y0, y1 = B.q4_gemv_fused2_act(*t, x)
    xq, xd = B.q8_1_quantize_act(x)
    z0, z1 = B.q4_gemv_fused2(*t, xq, xd)
    assert torch.equal(y0, z0) and torch.equal(y1, z1)
    # one matrix only
    e0, e1 = B.q4_gemv_fused2_act(t[0][:0], t[1][:0], t[2], t[3], x)
    assert e0.shape == (M, 0) and torch.equal(e1, z1)


@pytest.mark.parametrize("M,rows,K", [(1, (12288, 12288, 12288), 4096), (1, (2048, 512, 512), 2048),
                                      (2, (300, 0, 17, 1000), 4128), (4, (64, 8, 1, 520), 96)])
def test_gemv_multi_bit_identical(M, rows, K):
    """Several matrices in one launch give the bits of one launch per matrix,
    on Q8_1 planes and on the raw activation."""
    say(f"gemv_multi M={M} rows={rows} K={K}")
    rng = np.random.default_rng(sum(rows) + K)
    mats = [tuple(dev(a) for a in oracle.q4_0_quantize(synth.weights(rng, max(n, 1), K)))
            for n in rows]
    mats = [(q[:n], d[:n]) for (q, d), n in zip(mats, rows)]
    x = bf16_dev(synth.activations(rng, M, K))
    xq, xd = B.q8_1_quantize_act(x)
    ys = B.q4_gemv_multi(mats, xq, xd)
    ya = B.q4_gemv_multi_act(mats, x)
    for (q, d), y, y2 in zip(mats, ys, ya):
        if d.shape[0] == 0:
            assert y.shape == (M, 0)
            continue
        want = B.q4_gemv(q, d, xq, xd)
        assert torch.equal(y, want) and torch.equal(y2, want)


def test_gemv_deterministic_and_row_permutation():
    wqs, wd, xqs, xds = _gemv_case(2, 3000, 4096, seed=77)
    t = [dev(a) for a in (wqs, wd, xqs, xds)]
    hashes = set()
    for _ in range(20):
        y = B.q4_gemv(*t)
        hashes.add(hashlib.sha256(host(y).tobytes()).hexdigest())
    assert len(hashes) == 1
    perm = np.random.default_rng(3).permutation(3000)
    yp = B.q4_gemv(dev(wqs[perm]), dev(wd[perm]), t[2], t[3])
    assert np.array_equal(host(yp), host(y)[:, perm])


# ---------------------------------------------------------------------------
# GEMM paths
# ---------------------------------------------------------------------------

def _q4_gemm_ref(qs, d, Xf64):
    return oracle.matmul_f64(Xf64, oracle.q4_0_dequantize(qs, d))


def test_gemm_tiny_config_f32():
    """The tiny configuration: W f32 [256,512] -> Q4_0, X f32 [4,512], fp32 output."""
    wl = synth.TINY
    W, X = synth.workload_inputs(wl)
    qs, d = oracle.q4_0_quantize(W)
    gq, gd = B.q4_quantize(dev(W))
    assert np.array_equal(host(gq), qs) and np.array_equal(host(gd, np.uint16), d)
    ref = _q4_gemm_ref(qs, d, X.astype(np.float64))
    for path in (-1, B.Q4_PATH_SKINNY, B.Q4_PATH_MFMA):
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, path)
        try:
            y = B.q4_gemm(gq, gd, dev(X), y_dtype=torch.float32)
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
        e = rel(out_f64(y), ref)
        say(f"tiny path {path}: rel {e:.3e}")
        assert e <= BAR
    # and through the integer-dot GEMV on Q8_1 activations (M = 4)
    xq, xd = B.q8_1_quantize_act(dev(X))
    y = B.q4_gemv(gq, gd, xq, xd)
    xqs, xds = oracle.q8_1_quantize(X)
    assert rel(host(y).astype(np.float64), oracle.q4q8_gemv(qs, d, xqs, xds)) <= GEMV_TIGHT


_BOUNDARY_M = [1, 2, 3, 4, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 511, 512, 513]


def _workspace_every_path(M, N, K, fmt=B.Q4_FMT_Q4_0):
    """A workspace large enough for the forced MFMA and DEQUANT_GEMM paths."""
    sizes = []
    for path in (B.Q4_PATH_MFMA, B.Q4_PATH_DEQUANT_GEMM):
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, path)
        try:
            sizes.append(B.q4_gemm_workspace_size(M, N, K, fmt))
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    return torch.empty(max(sizes), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("M", _BOUNDARY_M)
def test_q4_gemm_every_path_boundary_m(M):
    N, K = 300, 2048
    rng = np.random.default_rng(M + 11)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    qs, d = oracle.q4_0_quantize(W)
    xb = synth.bf16_bits(X)
    ref = _q4_gemm_ref(qs, d, synth.bf16_bits_to_f32(xb).astype(np.float64))
    tq, td, tx = dev(qs), dev(d), dev(xb).view(torch.bfloat16)
    ws = _workspace_every_path(M, N, K)
    auto = B.q4_gemm(tq, td, tx, y_dtype=torch.bfloat16)
    assert rel(out_f64(auto), ref) <= BAR
    # (path, workspace): the MFMA path runs on the packed X image with a
    # workspace and converts X in the GEMM without one
    cases = [(B.Q4_PATH_MFMA, ws), (B.Q4_PATH_MFMA, None), (B.Q4_PATH_DEQUANT_GEMM, ws)]
    cases += [(B.Q4_PATH_SKINNY, None)] if M <= 64 else []
    for path, w in cases:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, path)
        try:
            for ydt in (torch.bfloat16, torch.float32):
                y = B.q4_gemm(tq, td, tx, y_dtype=ydt, workspace=w)
                e = rel(out_f64(y), ref)
                assert e <= BAR, (M, path, w is None, ydt, e)
                if ydt == torch.float32:
                    assert e <= 1e-3, (M, path, w is None, e)   # fp16 operands, fp32 output
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 160, 640, 1024), ("q4_0", 129, 300, 96), ("q4_0", 1, 257, 4096),
                                       ("q4_0", 300, 700, 2048), ("q4_0", 200, 1000, 320),
                                       ("affine", 160, 640, 1024), ("affine", 129, 300, 128),
                                       ("affine8", 160, 640, 1024), ("affine8", 129, 300, 128),
                                       ("affine8", 1, 257, 4096)])
def test_gemm_image_equals_mfma_path(fmt, M, N, K):
    """A prepacked weight image gives the bits of q4_gemm / affine4_gemm /
    affine8_gemm on the matrix-core path with a workspace, call after call
    with new activations (these shapes have few tiles, so both split K)."""
    say(f"gemm_image {fmt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    W = synth.weights(rng, N, K)
    if fmt == "q4_0":
        planes = [dev(a) for a in oracle.q4_0_quantize(W)]
        run = lambda x, ws, ydt: B.q4_gemm(*planes, x, y_dtype=ydt, workspace=ws)
        f = B.Q4_FMT_Q4_0
    elif fmt == "affine":
        planes = [dev(a) for a in oracle.affine4_quantize(synth.bf16_bits(W), 64)]
        run = lambda x, ws, ydt: B.affine4_gemm(*planes, x, y_dtype=ydt, workspace=ws)
        f = B.Q4_FMT_AFFINE4
    else:
        planes = [dev(a) for a in oracle.affine8_quantize(synth.bf16_bits(W), 64)]
        run = lambda x, ws, ydt: B.affine8_gemm(*planes, x, y_dtype=ydt, workspace=ws)
        f = B.Q4_FMT_AFFINE8
        assert B.q4_pack_weight_image(*planes).numel() == B.lib().q4_weight_image_size(N, K, f)   # format inferred
    image = B.q4_pack_weight_image(*planes, fmt=f)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)
    try:
        ws = torch.empty(B.lib().q4_gemm_workspace_size(M, N, K, f), dtype=torch.uint8, device="cuda")
        for call in range(2):
            x = bf16_dev(synth.activations(rng, M, K))
            for ydt in (torch.bfloat16, torch.float32):
                want = run(x, ws, ydt)
                # the same workspace size: room for the split-K partial results
                # of small tile counts, so both paths split alike
                got = B.q4_gemm_image(image, x, N, fmt=f, y_dtype=ydt, workspace=ws)
                assert torch.equal(got, want), (fmt, M, N, K, call, ydt)
        # room for the two images only: both run the packed kernel unsplit
        nimg = B.lib().q4_gemm_image_workspace_size(M, K) + B.lib().q4_weight_image_size(N, K, f)
        ws2 = torch.empty(nimg, dtype=torch.uint8, device="cuda")
        xws = torch.empty(max(B.lib().q4_gemm_image_workspace_size(M, K), 16), dtype=torch.uint8, device="cuda")
        x = bf16_dev(synth.activations(rng, M, K))
        want = run(x, ws2, torch.float32)
        got = B.q4_gemm_image(image, x, N, fmt=f, y_dtype=torch.float32, workspace=xws)
        assert torch.equal(got, want), (fmt, M, N, K, "unsplit")
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)


@pytest.mark.parametrize("fmt", ["q4_0", "affine"])
def test_small_m_row_chunks(fmt):
    """Above 32 rows, bf16 X runs the small-M kernel on row chunks of at most
    32 (up to 64 rows, and up to 128 when there is no room for the matrix-core
    GEMM's images): every chunk's rows are bit-identical to a call on those
    rows alone,
    the whole result is within the bar of the oracle, and with binary32 X the
    automatic choice above 16 rows is the matrix-core GEMM (bit-identical to
    it forced) with the workspace the size query asks for, and without a
    workspace the skinny kernel up to 32 rows and the GEMM above."""
    rng = np.random.default_rng(21)
    N, K = 700, 1024
    W = synth.weights(rng, N, K)
    if fmt == "q4_0":
        qs, d = oracle.q4_0_quantize(W)
        planes = [dev(qs), dev(d)]
        ref_w = oracle.q4_0_dequantize(qs, d)
        run = lambda x, **kw: B.q4_gemm(*planes, x, **kw)
        f = B.Q4_FMT_Q4_0
    else:
        ap = oracle.affine4_quantize(synth.bf16_bits(W), 64)
        planes = [dev(a) for a in ap]
        ref_w = oracle.affine4_dequantize(*ap, 64)
        run = lambda x, **kw: B.affine4_gemm(*planes, x, **kw)
        f = B.Q4_FMT_AFFINE4
    assert B.q4_dispatch_path(64, N, K, f) == B.Q4_PATH_SKINNY
    for M in (33, 40, 64, 96, 128):
        say(f"small-M row chunks {fmt} M={M}")
        X = synth.activations(rng, M, K)
        x = bf16_dev(X)
        for ydt in (torch.bfloat16, torch.float32):
            y = run(x, y_dtype=ydt, workspace=None)
            for r in range(0, M, 32):
                part = run(x[r:r + 32].contiguous(), y_dtype=ydt, workspace=None)
                assert torch.equal(y[r:r + 32], part), (fmt, M, r, ydt)
            ref = oracle.matmul_f64(synth.bf16_bits_to_f32(synth.bf16_bits(X)).astype(np.float64), ref_w)
            assert rel(out_f64(y), ref) <= BAR, (fmt, M, ydt)
        if M > 64:
            # with room for its images the matrix-core GEMM takes these rows
            ws = torch.empty(B.q4_gemm_workspace_size(M, N, K, f), dtype=torch.uint8, device="cuda")
            auto = run(x, y_dtype=torch.float32, workspace=ws)
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)
            try:
                forced = run(x, y_dtype=torch.float32, workspace=ws)
            finally:
                B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
            assert torch.equal(auto, forced), (fmt, M)
    # binary32 X above 16 rows: the matrix-core GEMM when the workspace holds
    # its images; without them the skinny kernel up to 32 rows, the GEMM above
    for M in (24, 33, 64):
        xf = torch.from_numpy(synth.activations(rng, M, K)).cuda()
        ws = torch.empty(B.q4_gemm_workspace_size(M, N, K, f), dtype=torch.uint8, device="cuda")
        auto = run(xf, y_dtype=torch.float32, workspace=ws)
        auto_none = run(xf, y_dtype=torch.float32, workspace=None)
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)
        try:
            forced = run(xf, y_dtype=torch.float32, workspace=ws)
            forced_none = run(xf, y_dtype=torch.float32, workspace=None)
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_SKINNY)
            skinny = run(xf, y_dtype=torch.float32, workspace=None)
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
        assert torch.equal(auto, forced), (fmt, M)
        assert torch.equal(auto_none, skinny if M <= 32 else forced_none), (fmt, M)


def test_q4_gemm_equals_image_at_prefill_size():
    """q4_gemm with a workspace (the weight image built per call) gives the
    bits of q4_gemm_image on a weight image prepared once, at the prefill
    shape (M = 2048, N = 12288, K = 4096) and on a ragged one."""
    rng = np.random.default_rng(11)
    for M, N, K in ((2048, 12288, 4096), (2000, 12300, 4096)):
        say(f"per-call vs prepared image M={M} N={N} K={K}")
        qs, d = B.q4_quantize(torch.from_numpy(synth.weights(rng, N, K)).cuda())
        x = bf16_dev(synth.activations(rng, M, K))
        ws = torch.empty(B.q4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device="cuda")
        want = B.q4_gemm_image(B.q4_pack_weight_image(qs, d), x, N, workspace=ws)
        got = B.q4_gemm(qs, d, x, workspace=ws)
        assert torch.equal(got, want), (M, N, K)


@pytest.mark.parametrize("M", [1, 17, 64, 65, 300])
def test_affine4_gemm_every_path(M):
    N, K = 257, 1024
    rng = np.random.default_rng(M + 99)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    q, s, b = oracle.affine4_quantize(synth.bf16_bits(W), 64)
    xb = synth.bf16_bits(X)
    ref = oracle.matmul_f64(synth.bf16_bits_to_f32(xb).astype(np.float64), oracle.affine4_dequantize(q, s, b))
    t = [dev(a) for a in (q, s, b)]
    tx = dev(xb).view(torch.bfloat16)
    ws = _workspace_every_path(M, N, K, B.Q4_FMT_AFFINE4)
    cases = [(B.Q4_PATH_MFMA, ws), (B.Q4_PATH_MFMA, None), (B.Q4_PATH_DEQUANT_GEMM, ws)]
    cases += [(B.Q4_PATH_SKINNY, None)] if M <= 64 else []
    for path, w in cases:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, path)
        try:
            for ydt in (torch.bfloat16, torch.float32):
                y = B.affine4_gemm(t[0], t[1], t[2], tx, y_dtype=ydt, workspace=w)
                e = rel(out_f64(y), ref)
                assert e <= BAR, (M, path, w is None, ydt, e)
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)


def test_dequant_path_equals_dequantize_plus_dense_gemm():
    M, N, K = 200, 384, 1024
    rng = np.random.default_rng(8)
    qs, d = oracle.q4_0_quantize(synth.weights(rng, N, K))
    tx = bf16_dev(synth.activations(rng, M, K))
    tq, td = dev(qs), dev(d)
    ws = _workspace_every_path(M, N, K)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
    try:
        y = B.q4_gemm(tq, td, tx, workspace=ws)
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    z = B.dense_gemm(tx, B.q4_dequantize(tq, td, out_dtype=torch.float16))
    assert torch.equal(y, z)


def _sampled_check(y_dev, Xf64, What, seed, count=6000):
    M, N = y_dev.shape
    rng = np.random.default_rng(seed)
    ms = np.concatenate([rng.integers(0, M, count), np.zeros(N, np.int64), np.arange(M) % M])
    ns = np.concatenate([rng.integers(0, N, count), np.arange(N), np.full(M, N - 1)])
    ref = oracle.matmul_f64_sampled(Xf64, What, ms, ns)
    got = out_f64(y_dev)[ms, ns]
    return rel(got, ref)


def test_q4_gemm_prefill_config_sampled():
    wl = synth.PREFILL
    say(f"prefill config M={wl.M} N={wl.N} K={wl.K}")
    W, X = synth.workload_inputs(wl)
    qs, d = oracle.q4_0_quantize(W)
    xb = synth.bf16_bits(X)
    y = B.q4_gemm(dev(qs), dev(d), dev(xb).view(torch.bfloat16), y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    e = _sampled_check(y, synth.bf16_bits_to_f32(xb).astype(np.float64), oracle.q4_0_dequantize(qs, d), 1)
    say(f"  sampled rel err {e:.3e}")
    assert e <= BAR


@pytest.mark.parametrize("M", synth.AFFINE_MS)
def test_affine4_gemm_sweep_sampled(M):
    wl = synth.AFFINE
    say(f"affine sweep M={M}")
    W, X = synth.workload_inputs(wl, M=M)
    q, s, b = oracle.affine4_quantize(synth.bf16_bits(W), 64)
    xb = synth.bf16_bits(X)
    y = B.affine4_gemm(dev(q), dev(s), dev(b), dev(xb).view(torch.bfloat16), y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    e = _sampled_check(y, synth.bf16_bits_to_f32(xb).astype(np.float64), oracle.affine4_dequantize(q, s, b), M)
    say(f"  sampled rel err {e:.3e}")
    assert e <= BAR



_PREFILL_W = {}


def _prefill_weights(fmt):
    """The prefill shape's weights in one format, quantised by the oracle once."""
    if fmt not in _PREFILL_W:
        W, _ = synth.workload_inputs(synth.PREFILL, M=0)
        if fmt == "q4_0":
            planes = oracle.q4_0_quantize(W)
            _PREFILL_W[fmt] = (planes, oracle.q4_0_dequantize(*planes))
        else:
            planes = oracle.affine4_quantize(synth.bf16_bits(W), 64)
            _PREFILL_W[fmt] = (planes, oracle.affine4_dequantize(*planes, 64))
    return _PREFILL_W[fmt]


@pytest.mark.parametrize("fmt,M", [("q4_0", 2), ("q4_0", 16), ("q4_0", 48), ("q4_0", 64),
                                   ("affine4", 16), ("affine4", 48), ("affine4", 64)])
def test_small_m_prefill_shape_sampled(fmt, M):
    """The small-M sweep at N = 12288, K = 4096 as it is timed (bf16 X and Y,
    no workspace; 48 and 64 rows run as 32-row chunks): sampled outputs
    against the binary64 product with the dequantised weights."""
    wl = synth.PREFILL
    say(f"small-M {fmt} M={M} N={wl.N} K={wl.K}")
    planes, What = _prefill_weights(fmt)
    f = B.Q4_FMT_Q4_0 if fmt == "q4_0" else B.Q4_FMT_AFFINE4
    assert B.q4_dispatch_path(M, wl.N, wl.K, f) == B.Q4_PATH_SKINNY
    X = synth.activations(np.random.default_rng(300 + M), M, wl.K)
    xb = synth.bf16_bits(X)
    tx = dev(xb).view(torch.bfloat16)
    gemm = B.q4_gemm if fmt == "q4_0" else B.affine4_gemm
    y = gemm(*[dev(a) for a in planes], tx, y_dtype=torch.bfloat16, workspace=None)
    torch.cuda.synchronize()
    e = _sampled_check(y, synth.bf16_bits_to_f32(xb).astype(np.float64), What, 100 + M)
    say(f"  sampled rel err {e:.3e}")
    assert e <= BAR

def test_gemm_deterministic_and_row_permutation():
    M, N, K = 600, 512, 2048
    rng = np.random.default_rng(44)
    qs, d = oracle.q4_0_quantize(synth.weights(rng, N, K))
    tx = bf16_dev(synth.activations(rng, M, K))
    tq, td = dev(qs), dev(d)
    ys = [B.q4_gemm(tq, td, tx) for _ in range(5)]
    assert all(torch.equal(ys[0], y) for y in ys[1:])
    perm = np.random.default_rng(1).permutation(N)
    yp = B.q4_gemm(dev(qs[perm]), dev(d[perm]), tx)
    assert torch.equal(yp, ys[0][:, torch.from_numpy(perm).cuda()])


def test_empty_inputs_are_noops():
    """M == 0 or N == 0 launches nothing and leaves the outputs alone."""
    K = 64
    qs, d = B.q4_quantize(torch.ones((4, K), dtype=torch.float32, device="cuda"))
    xq, xd = B.q8_1_quantize_act(torch.ones((2, K), dtype=torch.float32, device="cuda"))
    y = torch.full((2, 4), 7.0, device="cuda")
    assert B.lib().q4_gemv(B._p(qs), B._p(d), B._p(xq), B._p(xd), B._p(y), 0, 4, K, None) == B.Q4_OK
    assert B.lib().q4_gemv(B._p(qs), B._p(d), B._p(xq), B._p(xd), B._p(y), 2, 0, K, None) == B.Q4_OK
    e = B.q4_gemv(qs, d, xq[:0], xd[:0])
    assert e.shape == (0, 4)
    y0, y1 = B.q4_gemv_fused2(qs, d, qs[:0], d[:0], xq, xd)
    assert y1.shape == (2, 0)
    assert torch.equal(y0, B.q4_gemv(qs, d, xq, xd))
    xb = torch.zeros((3, K), dtype=torch.bfloat16, device="cuda")
    assert B.q4_gemm(qs[:0], d[:0], xb).shape == (3, 0)
    assert B.q4_gemm(qs, d, xb[:0]).shape == (0, 4)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---------------------------------------------------------------------------
# HIP graph replay: the decode step and the packed prefill GEMM
# ---------------------------------------------------------------------------

def test_graph_replays_match_eager():
    """Capture q8_1_quantize_act + q4_gemv + q4_gemv_fused2 + q4_gemm (packed
    path, caller workspace) + the activation-quantising GEMVs in one graph; every replay, with eager work and
    synchronisations between replays, reproduces the eager results exactly."""
    rng = np.random.default_rng(21)
    N, K, M = 640, 1024, 160
    w = [oracle.q4_0_quantize(synth.weights(rng, N, K)) for _ in range(3)]
    t = [(dev(q), dev(d)) for q, d in w]
    x1 = bf16_dev(synth.activations(rng, 1, K))
    xm = bf16_dev(synth.activations(rng, M, K))
    xq = torch.empty((1, K), dtype=torch.int8, device="cuda")
    xd = torch.empty((1, K // 32, 2), dtype=torch.int16, device="cuda")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y0 = torch.empty_like(y)
    y1 = torch.empty_like(y)
    yg = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.q4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0

    ya = torch.empty_like(y)
    ya0 = torch.empty_like(y)
    ya1 = torch.empty_like(y)
    outs = (xq, xd, y, y0, y1, yg, ya, ya0, ya1)

    def work():
        B.q8_1_quantize_act(x1, xq, xd)
        B.q4_gemv(*t[0], xq, xd, y)
        B.q4_gemv_fused2(*t[1], *t[2], xq, xd, y0, y1)
        B.q4_gemm(*t[0], xm, y=yg, workspace=ws)
        B.q4_gemv_act(*t[0], x1, ya)
        B.q4_gemv_fused2_act(*t[1], *t[2], x1, ya0, ya1)

    work()
    torch.cuda.synchronize()
    assert torch.equal(ya, y) and torch.equal(ya0, y0) and torch.equal(ya1, y1)
    ref = [a.clone() for a in outs]
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        work()
    for rep in range(4):
        for a in outs:
            a.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip(outs, ref):
            assert torch.equal(a, r), f"replay {rep} differs"
        work()                                   # eager work between replays
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# affine 8-bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(64, 128), (33, 192), (12288, 4096)])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
def test_affine8_quantize_bitexact(N, K, wdt):
    say(f"affine8_quantize N={N} K={K} {wdt}")
    rng = np.random.default_rng(N * 7 + K)
    W = synth.weights(rng, N, K)
    W[0, :64] = 0.25                    # constant group: s = 0
    W[-1, -64:] = np.linspace(-1.0, 2.0, 64, dtype=np.float32)
    Wb = synth.bf16_bits(W)
    wt = dev(Wb).view(torch.bfloat16) if wdt == "bf16" else dev(W)
    q, s, b = B.affine8_quantize(wt)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.affine8_quantize(oracle.f32_to_bf16_bits(W), 64)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s, np.uint16), rs)
    assert np.array_equal(host(b, np.uint16), rb)


@pytest.mark.parametrize("N,K", [(37, 64), (12288, 4096)])
def test_affine8_dequantize_bitexact(N, K):
    say(f"affine8_dequantize N={N} K={K}")
    rng = np.random.default_rng(9)
    W = synth.weights(rng, N, K) * np.float32(40.0)
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(W), 64)
    aq, as_, ab = dev(q), dev(s), dev(b)
    for kind, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        got = host(B.affine8_dequantize(aq, as_, ab, out_dtype=dt), np.uint16)
        assert np.array_equal(got, oracle.affine8_dequantize_half(q, s, b, kind)), kind
    got32 = host(B.affine8_dequantize(aq, as_, ab, out_dtype=torch.float32))
    assert np.array_equal(got32, oracle.affine8_dequantize(q, s, b).astype(np.float32))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 11, 16, 17, 32, 33, 130, 300])
@pytest.mark.parametrize("N,K", [(257, 1024), (40, 64), (96, 4160)])
def test_affine8_gemm_parity(M, N, K):
    say(f"affine8_gemm M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 31 + N + K)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(W), 64)
    t = [dev(a) for a in (q, s, b)]
    xb = synth.bf16_bits(X)
    ref = oracle.matmul_f64(synth.bf16_bits_to_f32(xb).astype(np.float64), oracle.affine8_dequantize(q, s, b))
    for ydt in (torch.bfloat16, torch.float32):
        y = B.affine8_gemm(*t, bf16_dev(X), y_dtype=ydt)
        torch.cuda.synchronize()
        e = oracle.rel_frobenius(out_f64(y), ref)
        assert e <= BAR, (M, N, K, ydt, e)
        if ydt == torch.float32:
            # fused (M <= 32 on bf16 X): exact products, binary32 sums; above
            # (the matrix-core GEMM): binary16 weights and X
            assert e <= (GEMV_TIGHT if M <= 32 else 1e-3), (M, N, K, e)
    if M <= 16:
        # a binary32 activation (the same values): binary32 weights times x
        Xf = synth.bf16_bits_to_f32(xb)
        y32 = B.affine8_gemm(*t, dev(Xf), y_dtype=torch.float32)
        torch.cuda.synchronize()
        e = oracle.rel_frobenius(out_f64(y32), ref)
        assert e <= GEMV_TIGHT, (M, N, K, "f32 x", e)


def test_affine8_dispatch_routes():
    """affine8_gemm follows q4_dispatch_path (Q4_FMT_AFFINE8): a forced
    DEQUANT_GEMM gives the bits of affine8_dequantize + dense_gemm; a forced
    MFMA, or Q4_KEY_AFFINE8_FUSED_MAX_M below M, the matrix-core GEMM on
    images (the same bits both ways); the default stays on the fused kernel;
    all within the bar of the binary64 oracle."""
    M, N, K = 8, 300, 256
    rng = np.random.default_rng(88)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(W), 64)
    t = [dev(a) for a in (q, s, b)]
    x = bf16_dev(X)
    ref = oracle.matmul_f64(synth.bf16_bits_to_f32(synth.bf16_bits(X)).astype(np.float64),
                            oracle.affine8_dequantize(q, s, b))
    want_deq = B.dense_gemm(x, B.affine8_dequantize(*t, out_dtype=torch.float16), y_dtype=torch.float32)
    fused = B.affine8_gemm(*t, x, y_dtype=torch.float32)
    assert not torch.equal(fused, want_deq)          # a different path
    got = {}
    for how in ("force_deq", "force_mfma", "key"):
        if how == "force_deq":
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
        elif how == "force_mfma":
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)
        else:
            B.q4_set_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M, 4)
        try:
            wsb = B.affine8_gemm_workspace_size(M, N, K)
            if how == "force_deq":
                assert wsb == N * K * 2
            else:
                assert wsb >= 128 * (K * 2 + 1) + 2 * (K // 64) * 17408
            got[how] = B.affine8_gemm(*t, x, y_dtype=torch.float32)
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
            B.q4_set_dispatch(B.Q4_KEY_AFFINE8_FUSED_MAX_M, 32)
    torch.cuda.synchronize()
    assert torch.equal(got["force_deq"], want_deq)
    assert torch.equal(got["force_mfma"], got["key"])
    assert not torch.equal(got["key"], want_deq)
    for y in (fused, want_deq, got["key"]):
        assert rel(out_f64(y), ref) <= BAR


@pytest.mark.parametrize("M", [33, 64, 130, 300])
@pytest.mark.parametrize("N,K", [(300, 1024), (520, 4096), (1, 64)])
def test_affine8_mfma_path(M, N, K):
    """The matrix-core GEMM on affine 8-bit images against the binary64
    oracle: bf16 and f32 X, bf16 and f32 Y, with the split-K partials room
    (affine8_gemm_workspace_size) and without it (the two images only: K is
    not split), ragged N and M; and against forced dequantise-then-GEMM."""
    say(f"affine8 matrix-core path M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 13 + N * 5 + K)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(W), 64)
    t = [dev(a) for a in (q, s, b)]
    xb = synth.bf16_bits(X)
    xf = synth.bf16_bits_to_f32(xb)
    ref = oracle.matmul_f64(xf.astype(np.float64), oracle.affine8_dequantize(q, s, b))
    images = B.q4_gemm_image_workspace_size(M, K) + (N + 255) // 256 * (K // 64) * 17408
    full = B.affine8_gemm_workspace_size(M, N, K)
    assert full >= images
    outs = {}
    for xname, x in (("bf16", bf16_dev(X)), ("f32", dev(xf))):
        for wsname, nbytes in (("split", full), ("images", images)):
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            y32 = B.affine8_gemm(*t, x, y_dtype=torch.float32, workspace=ws)
            y16 = B.affine8_gemm(*t, x, y_dtype=torch.bfloat16, workspace=ws)
            torch.cuda.synchronize()
            e = oracle.rel_frobenius(out_f64(y32), ref)
            assert e <= 1e-3, (xname, wsname, e)
            # bf16 Y: the same fp32 results rounded to nearest even (bf16
            # rounding alone is up to 2^-9 of each output, so the Frobenius
            # bar is checked only where there are enough outputs to average)
            assert torch.equal(y16, y32.to(torch.bfloat16)), (xname, wsname)
            if M * N >= 1024:
                assert oracle.rel_frobenius(out_f64(y16), ref) <= BAR, (xname, wsname)
            outs[(xname, wsname)] = y32
    # the same values in bf16 and f32 X convert to the same binary16 image
    assert torch.equal(outs[("bf16", "split")], outs[("f32", "split")])
    assert torch.equal(outs[("bf16", "images")], outs[("f32", "images")])
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
    try:
        yd = B.affine8_gemm(*t, bf16_dev(X), y_dtype=torch.float32)
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    torch.cuda.synchronize()
    # both multiply the same binary16 weights and X: only the summation order differs
    assert rel(out_f64(outs[("bf16", "images")]), out_f64(yd)) <= 1e-5


def test_affine8_gemm_full_size_sampled():
    """N=12288, K=4096 at M = 1, 16 and 32 (fused) and M = 64 (matrix-core GEMM): sampled outputs against binary64."""
    N, K = 12288, 4096
    rng = np.random.default_rng(2024)
    W = synth.weights(rng, N, K)
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(W), 64)
    t = [dev(a) for a in (q, s, b)]
    What = oracle.affine8_dequantize(q, s, b)
    for M in (1, 16, 32, 64):
        say(f"affine8_gemm full size M={M}")
        X = synth.activations(rng, M, K)
        xb = synth.bf16_bits(X)
        y = out_f64(B.affine8_gemm(*t, bf16_dev(X), y_dtype=torch.float32))
        ms = rng.integers(0, M, 64)
        ns = rng.integers(0, N, 64)
        want = oracle.matmul_f64_sampled(synth.bf16_bits_to_f32(xb).astype(np.float64), What, ms, ns)
        got = y[ms, ns]
        assert np.linalg.norm(got - want) <= (GEMV_TIGHT if M <= 32 else 1e-3) * np.linalg.norm(want), M


@pytest.mark.parametrize("M", [1, 5, 32, 33])
@pytest.mark.parametrize("N,K", [(1, 64), (17, 128), (3, 4096)])
def test_affine8_gemm_edges_and_determinism(M, N, K):
    """One output row, one group (three of the MFMA kernel's four waves get none), and repeated calls
    giving the same bits (the summation order depends on K only)."""
    say(f"affine8_gemm edges M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 101 + N * 7 + K)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(W), 64)
    t = [dev(a) for a in (q, s, b)]
    xb = synth.bf16_bits(X)
    ref = oracle.matmul_f64(synth.bf16_bits_to_f32(xb).astype(np.float64), oracle.affine8_dequantize(q, s, b))
    x = bf16_dev(X)
    y1 = B.affine8_gemm(*t, x, y_dtype=torch.float32)
    y2 = B.affine8_gemm(*t, x, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), (M, N, K)
    e = oracle.rel_frobenius(out_f64(y1), ref)
    assert e <= (GEMV_TIGHT if M <= 32 else 1e-3), (M, N, K, e)


def test_affine8_graph_replays_match_eager():
    """affine8_gemm on each of its three paths (vector kernel, bf16-MFMA kernel, matrix-core GEMM on
    images in a caller workspace) captured in one graph: every replay, with eager work and synchronisations
    between replays, reproduces the eager results exactly."""
    rng = np.random.default_rng(77)
    N, K = 300, 1024
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(synth.weights(rng, N, K)), 64)
    t = [dev(a) for a in (q, s, b)]
    xs = {M: bf16_dev(synth.activations(rng, M, K)) for M in (1, 20, 40)}
    ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for M in xs}
    ws = torch.empty(B.lib().affine8_gemm_workspace_size(40, N, K), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0

    def work():
        for M, x in xs.items():
            B.affine8_gemm(*t, x, y=ys[M], workspace=ws if M == 40 else None)

    work()
    torch.cuda.synchronize()
    ref = {M: y.clone() for M, y in ys.items()}
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        work()
    for rep in range(4):
        for y in ys.values():
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for M in ys:
            assert torch.equal(ys[M], ref[M]), (rep, M)
        work()                                          # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("case", range(24))
def test_random_shapes_every_entry_point(case):
    """Seeded random shapes through the automatic dispatch of q4_gemm, affine4_gemm and affine8_gemm
    (with and without a workspace), bf16 output, against the binary64 oracle."""
    rng = np.random.default_rng(9000 + case)
    M = int(rng.choice([1, 2, 3, 5, 8, 13, 17, 31, 32, 33, 64, 65, 128, 129, 200, 300]))
    N = int(rng.integers(1, 700))
    K = 64 * int(rng.integers(1, 40))
    say(f"random shapes case {case}: M={M} N={N} K={K}")
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    xb = synth.bf16_bits(X)
    x = bf16_dev(X)
    xf64 = synth.bf16_bits_to_f32(xb).astype(np.float64)
    qs, d = oracle.q4_0_quantize(W)
    aq, as_, ab = oracle.affine4_quantize(synth.bf16_bits(W), 64)
    eq, es, eb = oracle.affine8_quantize(synth.bf16_bits(W), 64)
    refs = {
        "q4_0": oracle.matmul_f64(xf64, oracle.q4_0_dequantize(qs, d)),
        "affine4": oracle.matmul_f64(xf64, oracle.affine4_dequantize(aq, as_, ab)),
        "affine8": oracle.matmul_f64(xf64, oracle.affine8_dequantize(eq, es, eb)),
    }
    calls = {
        "q4_0": lambda ws: B.q4_gemm(dev(qs), dev(d), x, workspace=ws),
        "affine4": lambda ws: B.affine4_gemm(dev(aq), dev(as_), dev(ab), x, workspace=ws),
        "affine8": lambda ws: B.affine8_gemm(dev(eq), dev(es), dev(eb), x, workspace=ws),
    }
    for fmt, call in calls.items():
        for ws in ("auto", None):
            if fmt == "affine8" and ws is None and M > 32:
                continue                                 # that path needs its workspace
            y = call(ws)
            torch.cuda.synchronize()
            e = oracle.rel_frobenius(out_f64(y), refs[fmt])
            assert e <= BAR, (fmt, ws, M, N, K, e)


@pytest.mark.parametrize("case", range(16))
def test_random_shapes_gemv(case):
    """Seeded random shapes through q4_gemv (M up to 16) against the Q8_1 oracle, and through
    q4_gemv_act / q4_gemv_fused2_act (M up to 4), bit-identical to quantise-then-GEMV."""
    rng = np.random.default_rng(7000 + case)
    M = int(rng.integers(1, 17))
    N = int(rng.integers(1, 3000))
    N1 = int(rng.integers(1, 3000))
    K = 32 * int(rng.integers(1, 200))
    say(f"random gemv case {case}: M={M} N={N} N1={N1} K={K}")
    wqs, wd = oracle.q4_0_quantize(synth.weights(rng, N, K))
    w1qs, w1d = oracle.q4_0_quantize(synth.weights(rng, N1, K))
    X = synth.activations(rng, M, K)
    x = bf16_dev(X)
    xq, xd = B.q8_1_quantize_act(x)
    t0, t1 = (dev(wqs), dev(wd)), (dev(w1qs), dev(w1d))
    y = B.q4_gemv(*t0, xq, xd)
    xqs, xds = oracle.q8_1_quantize(synth.bf16_bits_to_f32(synth.bf16_bits(X)))
    assert np.array_equal(host(xq), xqs) and np.array_equal(host(xd, np.uint16), xds)
    assert rel(host(y).astype(np.float64), oracle.q4q8_gemv(wqs, wd, xqs, xds)) <= GEMV_TIGHT, (M, N, K)
    y0, y1 = B.q4_gemv_fused2(*t0, *t1, xq, xd)
    assert torch.equal(y0, y) and torch.equal(y1, B.q4_gemv(*t1, xq, xd))
    if M <= 4:
        assert torch.equal(B.q4_gemv_act(*t0, x), y)
        a0, a1 = B.q4_gemv_fused2_act(*t0, *t1, x)
        assert torch.equal(a0, y0) and torch.equal(a1, y1)


# ---------------------------------------------------------------------------
# the large-M configuration of the in-kernel-converting GEMM (no workspace)
# and of the dense binary16 GEMM, at the prefill sizes: MLX issue #4621,
# Repro (2048 and 8192 tokens against W 12288 x 4096)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def prefill_q4():
    wl = synth.PREFILL
    W, X = synth.workload_inputs(wl)
    qs, d = oracle.q4_0_quantize(W)
    xb = synth.bf16_bits(X)
    return dict(qs=qs, d=d, xb=xb, Xf64=synth.bf16_bits_to_f32(xb).astype(np.float64),
                What=oracle.q4_0_dequantize(qs, d))


def test_q4_gemm_no_workspace_prefill_sampled(prefill_q4):
    p = prefill_q4
    say("q4_gemm M=2048 without a workspace (in-kernel X conversion)")
    y = B.q4_gemm(dev(p["qs"]), dev(p["d"]), dev(p["xb"]).view(torch.bfloat16), workspace=None)
    torch.cuda.synchronize()
    e = _sampled_check(y, p["Xf64"], p["What"], 5)
    say(f"  sampled rel err {e:.3e}")
    assert e <= BAR


def test_dense_and_dequant_path_prefill_sampled(prefill_q4):
    p = prefill_q4
    M, N, K = p["xb"].shape[0], p["d"].shape[0], p["xb"].shape[1]
    tq, td, tx = dev(p["qs"]), dev(p["d"]), dev(p["xb"]).view(torch.bfloat16)
    say("dense_gemm M=2048 on dequantised binary16 weights")
    w16 = B.q4_dequantize(tq, td, out_dtype=torch.float16)
    z = B.dense_gemm(tx, w16)
    torch.cuda.synchronize()
    e = _sampled_check(z, p["Xf64"], p["What"], 6)
    say(f"  dense sampled rel err {e:.3e}")
    assert e <= BAR
    say("q4_gemm M=2048 forced dequantise-then-GEMM")
    ws = torch.empty(N * K * 2, dtype=torch.uint8, device="cuda")
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
    try:
        y = B.q4_gemm(tq, td, tx, workspace=ws)
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    torch.cuda.synchronize()
    assert torch.equal(y, z)


@pytest.mark.parametrize("M", [2048, 8192])
def test_affine_large_m_no_workspace_and_affine8_sampled(M):
    wl = synth.AFFINE
    say(f"affine4 / affine8 M={M} N={wl.N} K={wl.K}")
    W, X = synth.workload_inputs(wl, M=M)
    wb = synth.bf16_bits(W)
    xb = synth.bf16_bits(X)
    Xf64 = synth.bf16_bits_to_f32(xb).astype(np.float64)
    tx = dev(xb).view(torch.bfloat16)
    q, s, b = oracle.affine4_quantize(wb, 64)
    y = B.affine4_gemm(dev(q), dev(s), dev(b), tx, workspace=None)
    torch.cuda.synchronize()
    e = _sampled_check(y, Xf64, oracle.affine4_dequantize(q, s, b), M + 1)
    say(f"  affine4 without workspace: sampled rel err {e:.3e}")
    assert e <= BAR
    del y
    q8, s8, b8 = oracle.affine8_quantize(wb, 64)
    y = B.affine8_gemm(dev(q8), dev(s8), dev(b8), tx)
    torch.cuda.synchronize()
    e = _sampled_check(y, Xf64, oracle.affine8_dequantize(q8, s8, b8), M + 2)
    say(f"  affine8: sampled rel err {e:.3e}")
    assert e <= BAR


def test_splitk_odd_output_count():
    """K split over workgroups with M*N odd (the partial sums' scalar tail):
    the same as the unsplit kernel within the bar, against the oracle, and a
    call that takes milliseconds, not seconds."""
    M, N, K = 33, 4095, 4096
    rng = np.random.default_rng(3301)
    qs, d = oracle.q4_0_quantize(synth.weights(rng, N, K))
    xb = synth.bf16_bits(synth.activations(rng, M, K))
    tq, td, tx = dev(qs), dev(d), dev(xb).view(torch.bfloat16)
    full = B.q4_gemm_workspace_size(M, N, K)
    imgs = B.q4_gemm_image_workspace_size(M, K) + B.q4_weight_image_size(N, K)
    assert full > imgs, "this shape should split K"
    ys = {}
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)     # 33 rows would run the small-M kernel
    try:
        for name, nbytes in (("split", full), ("unsplit", imgs)):
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            B.q4_gemm(tq, td, tx, y_dtype=torch.float32, workspace=ws)       # warm
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            ys[name] = B.q4_gemm(tq, td, tx, y_dtype=torch.float32, workspace=ws)
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1)
            say(f"  {name}: {ms:.3f} ms")
            assert ms < 20.0, (name, ms)
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    ref = _q4_gemm_ref(qs, d, synth.bf16_bits_to_f32(xb).astype(np.float64))
    for name, y in ys.items():
        assert rel(out_f64(y), ref) <= 1e-3, name
    assert rel(out_f64(ys["split"]), out_f64(ys["unsplit"])) <= 1e-5


def test_side_stream_auto_workspace_is_not_reused_early():
    """q4_gemm on a side stream with workspace "auto": the scratch tensor
    belongs to that stream, so work on the default stream right after the call
    cannot be handed the same memory while the side stream still uses it."""
    M, N, K = 1024, 4096, 4096
    rng = np.random.default_rng(404)
    qs, d = oracle.q4_0_quantize(synth.weights(rng, N, K))
    tq, td = dev(qs), dev(d)
    x = bf16_dev(synth.activations(rng, M, K))
    want = B.q4_gemm(tq, td, x)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        y = B.q4_gemm(tq, td, x, stream=side)
        # default-stream allocations and writes of the workspace's size
        junk = torch.full((B.q4_gemm_workspace_size(M, N, K),), 255, dtype=torch.uint8, device="cuda")
        junk.fill_(7)
        torch.cuda.synchronize()
        assert torch.equal(y, want)
        del junk


def test_f32_activation_rounds_to_nearest_even():
    """f32 X on the MFMA paths is rounded to binary16 to nearest even on every
    path (with and without a workspace), so the result is the fp32 product of
    the RNE-rounded X with the binary16 weights (q-8)*d: values 1 + 3*2^-12
    round up to 1 + 2^-10 (toward zero they would give 1, a bias of about
    1e-3 on two thirds of the x)."""
    M, N, K = 96, 256, 1024
    rng = np.random.default_rng(55)
    qs, d = oracle.q4_0_quantize(synth.weights(rng, N, K))
    sign = np.where(rng.random((M, K)) < 0.5, -1.0, 1.0).astype(np.float32)
    X = (sign * np.float32(1 + 3 * 2 ** -12) * rng.integers(1, 4, (M, K)).astype(np.float32)).astype(np.float32)
    Xr = oracle.f16_bits_to_f32(oracle.f32_to_f16_bits(X)).astype(np.float64)
    assert not np.array_equal(Xr, X.astype(np.float64))
    W16 = oracle.f16_bits_to_f32(oracle.q4_0_dequantize_half(qs, d, "f16")).astype(np.float64)
    ref = oracle.matmul_f64(Xr, W16)
    tq, td, tx = dev(qs), dev(d), dev(X)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)
    try:
        for ws in ("auto", None):
            y = B.q4_gemm(tq, td, tx, y_dtype=torch.float32, workspace=ws)
            torch.cuda.synchronize()
            e = rel(out_f64(y), ref)
            say(f"  f32 X workspace={ws}: rel {e:.3e} against RNE-rounded X")
            assert e <= 2e-5, (ws, e)
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)


# ---------------------------------------------------------------------------
# the 256 x 256-tile matrix-core kernel (Q4_KEY_TILE_ROWS = 256, at least one
# such tile per CU): ragged edges, determinism, weight images
# ---------------------------------------------------------------------------

@pytest.fixture
def big_tiles():
    B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, 256)
    try:
        yield
    finally:
        B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, 128)


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 4100, 4000, 1056), ("affine", 2050, 8200, 1088),
                                       ("q4_0", 4096, 4096, 4096), ("affine", 256, 65536, 512)])
def test_big_tile_kernel_ragged_against_oracle(big_tiles, fmt, M, N, K):
    """Shapes with at least one 256 x 256 tile per CU, ragged in M and N, and
    K = 32 mod 64 for Q4_0 (a last K step with one block): sampled outputs
    against binary64, the workspace and weight-image entry points giving the
    same bits, and the same bits call after call."""
    say(f"big-tile kernel {fmt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    xb = synth.bf16_bits(X)
    tx = dev(xb).view(torch.bfloat16)
    if fmt == "q4_0":
        planes = oracle.q4_0_quantize(W)
        What = oracle.q4_0_dequantize(*planes)
        f = B.Q4_FMT_Q4_0
        run = lambda ws: B.q4_gemm(*tp, tx, y_dtype=torch.float32, workspace=ws)
    else:
        planes = oracle.affine4_quantize(synth.bf16_bits(W), 64)
        What = oracle.affine4_dequantize(*planes)
        f = B.Q4_FMT_AFFINE4
        run = lambda ws: B.affine4_gemm(*tp, tx, y_dtype=torch.float32, workspace=ws)
    tp = [dev(a) for a in planes]
    ws = torch.empty(B.q4_gemm_workspace_size(M, N, K, f), dtype=torch.uint8, device="cuda")
    y = run(ws)
    torch.cuda.synchronize()
    e = _sampled_check(y, synth.bf16_bits_to_f32(xb).astype(np.float64), What, M, count=4000)
    say(f"  sampled rel err {e:.3e}")
    assert e <= 1e-3
    for _ in range(2):
        assert torch.equal(run(ws), y)
    image = B.q4_pack_weight_image(*tp, fmt=f)
    yi = B.q4_gemm_image(image, tx, N, fmt=f, y_dtype=torch.float32, workspace=ws)
    assert torch.equal(yi, y)
    # the same bf16 output is the RNE of the fp32 one
    yb = B.q4_gemm(*tp, tx, workspace=ws) if fmt == "q4_0" else B.affine4_gemm(*tp, tx, workspace=ws)
    assert torch.equal(yb, y.to(torch.bfloat16))


def test_big_tile_kernel_matches_128_row_kernel(big_tiles):
    """M = 2048, N = 12288, K = 4096 (384 tiles of 256 x 256: one round of
    whole tiles, then the last 128 tiles as 256 x 128 column halves): within
    fp32 rounding of the 128-row kernel (Q4_KEY_TILE_ROWS = 128), on the
    same workspace."""
    M, N, K = 2048, 12288, 4096
    rng = np.random.default_rng(12)
    qs, d = oracle.q4_0_quantize(synth.weights(rng, N, K))
    tq, td = dev(qs), dev(d)
    tx = bf16_dev(synth.activations(rng, M, K))
    ws = torch.empty(B.q4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device="cuda")
    y_big = B.q4_gemm(tq, td, tx, y_dtype=torch.float32, workspace=ws)
    B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, 128)
    try:
        y_pk = B.q4_gemm(tq, td, tx, y_dtype=torch.float32, workspace=ws)
    finally:
        B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, 256)
    torch.cuda.synchronize()
    d_ = (y_big.double() - y_pk.double()).norm() / y_pk.double().norm()
    say(f"  256-row vs 128-row kernel: rel {float(d_):.3e}")
    assert float(d_) <= 1e-5


# ---------------------------------------------------------------------------
# X outside binary16's range on the MFMA path with an X image: the per-row
# power-of-two prescale of k_pack_x and the epilogues' inverse
# ---------------------------------------------------------------------------

def _wide_range_x(rng, M, K):
    """Rows cycling through: N(0,1); x 1e5 (beyond 65504); x 1e-6 (below
    binary16's normal range 2^-14); half the entries x 1e5 and half x 1e-6;
    a row of zeros."""
    X = synth.activations(rng, M, K).astype(np.float32)
    kind = np.arange(M) % 5
    X[kind == 1] *= np.float32(1e5)
    X[kind == 2] *= np.float32(1e-6)
    mix = kind == 3
    scale = np.where(np.arange(K) % 2 == 0, np.float32(1e5), np.float32(1e-6)).astype(np.float32)
    X[mix] *= scale[None, :]
    X[kind == 4] = 0.0
    return X


def _per_row_rel(y, ref):
    """Largest per-row relative Frobenius error (rows with a zero reference
    must be exactly zero)."""
    worst = 0.0
    for m in range(ref.shape[0]):
        den = np.linalg.norm(ref[m])
        num = np.linalg.norm(y[m] - ref[m])
        if den == 0:
            assert num == 0, m
        else:
            worst = max(worst, num / den)
    return worst


@pytest.mark.parametrize("fmt,M,N,K,xdt,tile_rows", [
    ("q4_0", 64, 512, 2048, "bf16", 128),       # 2 x 128-row tiles: a K split
    ("q4_0", 2048, 512, 2048, "bf16", 128),
    ("affine", 2048, 512, 2048, "f32", 128),
    ("q4_0", 2048, 8192, 512, "bf16", 256),     # the 256 x 256-tile kernel
    ("affine", 2048, 8192, 512, "f32", 256),
])
def test_wide_range_x_on_the_image_path(fmt, M, N, K, xdt, tile_rows):
    """Rows holding +-1e5 and +-1e-6 values: every row within 2e-3 of the
    binary64 oracle on its own (bf16 X is converted exactly after the row's
    prescale, f32 X is rounded to 11 bits), zero rows exactly zero, and the
    image entry point giving the same bits."""
    say(f"wide-range X {fmt} M={M} N={N} K={K} x={xdt} tile_rows={tile_rows}")
    rng = np.random.default_rng(M * 7 + N + K)
    W = synth.weights(rng, N, K)
    X = _wide_range_x(rng, M, K)
    if xdt == "bf16":
        xb = synth.bf16_bits(X)
        tx = dev(xb).view(torch.bfloat16)
        Xf64 = synth.bf16_bits_to_f32(xb).astype(np.float64)
    else:
        tx = torch.from_numpy(X).cuda()
        Xf64 = X.astype(np.float64)
    if fmt == "q4_0":
        planes = oracle.q4_0_quantize(W)
        What = oracle.q4_0_dequantize(*planes)
        f = B.Q4_FMT_Q4_0
    else:
        planes = oracle.affine4_quantize(synth.bf16_bits(W), 64)
        What = oracle.affine4_dequantize(*planes)
        f = B.Q4_FMT_AFFINE4
    tp = [dev(a) for a in planes]
    ref = Xf64 @ What.T
    B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, tile_rows)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)     # M = 64 would run the small-M kernel
    try:
        assert B.q4_dispatch_path(M, N, K, f, True) == B.Q4_PATH_MFMA
        ws = torch.empty(B.q4_gemm_workspace_size(M, N, K, f), dtype=torch.uint8, device="cuda")
        if fmt == "q4_0":
            y = B.q4_gemm(*tp, tx, y_dtype=torch.float32, workspace=ws)
        else:
            y = B.affine4_gemm(*tp, tx, y_dtype=torch.float32, workspace=ws)
        image = B.q4_pack_weight_image(*tp, fmt=f)
        yi = B.q4_gemm_image(image, tx, N, fmt=f, y_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
    finally:
        B.q4_set_dispatch(B.Q4_KEY_TILE_ROWS, 128)
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    got = out_f64(y)
    assert np.isfinite(got).all()
    e = _per_row_rel(got, ref)
    say(f"  worst per-row rel err {e:.3e}; whole {rel(got, ref):.3e}")
    assert e <= BAR
    assert torch.equal(yi, y)


# ---------------------------------------------------------------------------
# Q4_0 x Q8_1 on the int8 matrix cores (q4_gemm_q8, path Q4_PATH_INT8)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(130, 300, 4128), (1, 33, 32), (64, 256, 512), (257, 129, 1056)])
def test_gemm_q8_unit_scales_are_exact_integer_sums(M, N, K):
    """d4 = d8 = 1: every output is the integer sum of its block dots, bit for
    bit (ragged M and N, K = 32 mod 64 and a last chunk of scales short)."""
    say(f"gemm_q8 unit scales M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 3 + N + K)
    wqs = rng.integers(0, 256, (N, K // 32, 16), dtype=np.uint8)
    wd = np.full((N, K // 32), 0x3C00, np.uint16)
    xqs = rng.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    xds = np.zeros((M, K // 32, 2), np.uint16)
    xds[..., 0] = 0x3C00
    y = B.q4_gemm_q8(dev(wqs), dev(wd), dev(xqs), dev(xds), y_dtype=torch.float32)
    torch.cuda.synchronize()
    isum = oracle.q4q8_block_dots(wqs, xqs).astype(np.int64).sum(axis=2)   # [M, N]
    assert np.array_equal(host(y).astype(np.int64), isum)
    assert np.array_equal(host(y), isum.astype(np.float32))


def test_gemm_q8_block_dot_extremes():
    """The largest block dots: nibbles 0 or 15 against codes +-127."""
    N, K = 2, 32
    wqs = np.zeros((N, 1, 16), np.uint8)
    wqs[1] = 0xFF
    wd = np.full((N, 1), 0x3C00, np.uint16)
    for v, want in ((-127, [32512, -28448]), (127, [-32512, 28448])):
        xqs = np.full((3, K), v, np.int8)
        xds = np.zeros((3, 1, 2), np.uint16)
        xds[..., 0] = 0x3C00
        y = host(B.q4_gemm_q8(dev(wqs), dev(wd), dev(xqs), dev(xds), y_dtype=torch.float32))
        assert y.tolist() == [want] * 3


@pytest.mark.parametrize("M,N,K", [(200, 700, 2048), (33, 4096, 4096), (1, 257, 96)])
def test_gemm_q8_against_oracle(M, N, K):
    """Real scales against the binary64 q4 x q8 oracle: fp32 output within the
    GEMV's 1e-5 (exact block terms, fp32 accumulation), bf16 output its RNE."""
    say(f"gemm_q8 oracle M={M} N={N} K={K}")
    wqs, wd, xqs, xds = _gemv_case(M, N, K, M + N + K)
    ref = oracle.q4q8_gemv(wqs, wd, xqs, xds)
    args = (dev(wqs), dev(wd), dev(xqs), dev(xds))
    y = B.q4_gemm_q8(*args, y_dtype=torch.float32)
    yb = B.q4_gemm_q8(*args, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    e = rel(out_f64(y), ref)
    say(f"  rel err {e:.3e}")
    assert e <= GEMV_TIGHT
    assert torch.equal(yb, y.to(torch.bfloat16))


def test_gemm_q8_prefill_config_sampled():
    """M = 2048, N = 12288, K = 4096 with X quantised to Q8_1 on the GPU (bit-
    exact with the oracle's codes, checked): 24 whole rows against the oracle."""
    wl = synth.PREFILL
    M, N, K = wl.M, wl.N, wl.K
    say(f"gemm_q8 prefill M={M} N={N} K={K}")
    rng = np.random.default_rng(5)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    wqs, wd = oracle.q4_0_quantize(W)
    xb = synth.bf16_bits(X)
    tx = dev(xb).view(torch.bfloat16)
    xq, xds = B.q8_1_quantize_act(tx)
    rows = np.random.default_rng(6).choice(M, 24, replace=False)
    rows.sort()
    rxq, rxd = oracle.q8_1_quantize(synth.bf16_bits_to_f32(xb)[rows])
    assert np.array_equal(host(xq)[rows], rxq) and np.array_equal(host(xds, np.uint16)[rows], rxd)
    y = B.q4_gemm_q8(dev(wqs), dev(wd), xq, xds, y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.q4q8_gemv(wqs, wd, rxq, rxd)
    e = rel(out_f64(y)[rows], ref)
    say(f"  sampled rows rel err {e:.3e}")
    assert e <= GEMV_TIGHT


@pytest.mark.parametrize("M", [1, 4, 77, 2048])
def test_forced_q8_paths_equal_their_two_steps(M):
    """q4_gemm with Q4_KEY_FORCE_PATH = INT8: the bits of q8_1_quantize_act +
    q4_gemm_q8; with GEMV (M <= 4, f32 out): the bits of q4_gemv_act."""
    N, K = 1024, 4096
    say(f"forced Q8_1 paths M={M}")
    rng = np.random.default_rng(M)
    qs, d = (dev(a) for a in oracle.q4_0_quantize(synth.weights(rng, N, K)))
    tx = bf16_dev(synth.activations(rng, M, K))
    xq, xds = B.q8_1_quantize_act(tx)
    want = B.q4_gemm_q8(qs, d, xq, xds, y_dtype=torch.float32)
    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_INT8)
    try:
        got = B.q4_gemm(qs, d, tx, y_dtype=torch.float32)
        gotb = B.q4_gemm(qs, d, tx, y_dtype=torch.bfloat16)
    finally:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert torch.equal(gotb, want.to(torch.bfloat16))
    if M <= B.Q4_GEMV_ACT_MAX_M:
        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_GEMV)
        try:
            g = B.q4_gemm(qs, d, tx, y_dtype=torch.float32)
        finally:
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
        assert torch.equal(g, B.q4_gemv_act(qs, d, tx))
