"""Pins for the CPU oracle: each test checks it against something other than itself.

Sources of truth used here (never the oracle's own formulas retyped):
  * numpy's float16 and torch's bfloat16 conversions (library routines);
  * hand-worked blocks under tests/golden/ (worked by hand from the stated
    conventions; each file cites the page that names the format);
  * exact rational arithmetic (fractions) on tiny shapes;
  * numpy float64 BLAS products, closed forms (one-hot inputs), linearity;
  * invariants: quantise -> dequantise error bounds, code ranges.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gemv_q4_affine_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            yield [p.strip() for p in line.split("|")]


def _f16_frac(bits):
    """Exact rational value of a binary16 bit pattern, via numpy's decoding."""
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def _unpack_q4(qs_block16):
    """Codes of a 16-byte block, split-half order, with numpy bit operations."""
    b = np.asarray(qs_block16, np.uint8)
    return np.concatenate([b & 0x0F, b >> 4]).astype(np.int64)


# --------------------------------------------------------------------------
# 16-bit float conversions vs library routines
# --------------------------------------------------------------------------

def _conversion_probe_values():
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(200_000).astype(np.float32) * np.float32(1e-3),
        rng.standard_normal(200_000).astype(np.float32) * np.float32(100.0),
        (rng.standard_normal(200_000) * 1e-6).astype(np.float32),   # f16 subnormal range
        rng.integers(0, 2**32, 400_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    # every binary16 value, and the midpoints between neighbours +- 1 binary32 ulp
    all16 = np.arange(0, 0x7C01, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = ((all16[:-1].astype(np.float64) + all16[1:].astype(np.float64)) / 2).astype(np.float32)
    parts += [all16, -all16, mids, np.nextafter(mids, np.float32(np.inf)),
              np.nextafter(mids, np.float32(-np.inf)), -mids]
    parts.append(np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.996, 65520, 1e30, -1e30,
                           2**-24, 2**-25, 2**-26, 3 * 2**-26, 1.4e-45], np.float32))
    x = np.concatenate(parts)
    return x[np.isfinite(x) | np.isinf(x)]


def test_f32_to_f16_matches_numpy():
    x = _conversion_probe_values()
    x = x[~np.isnan(x)]
    got = oracle.f32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_f16_to_f32_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_bits_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_f32_to_bf16_matches_torch():
    x = _conversion_probe_values()
    x = x[~np.isnan(x)]
    got = oracle.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_bf16_to_f32_matches_torch():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_bits_to_f32(b)
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


# --------------------------------------------------------------------------
# Q4_0 hand-worked blocks and invariants
# --------------------------------------------------------------------------

def _q4_golden():
    for name, ws, dhex, qhex in _golden_lines("q4_0_blocks.txt"):
        w = np.zeros(32, np.float32)
        if ws:
            for item in ws.split(","):
                i, v = item.split("=")
                w[int(i)] = np.float32(float(v))
        yield name, w, int(dhex, 16), bytes.fromhex(qhex.replace(" ", ""))


@pytest.mark.parametrize("case", list(_q4_golden()), ids=lambda c: c[0])
def test_q4_0_golden_blocks(case):
    name, w, d_bits, qs_bytes = case
    qs, d = oracle.q4_0_quantize(w.reshape(1, 32))
    assert int(d[0, 0]) == d_bits, f"{name}: d {int(d[0,0]):04x} != {d_bits:04x}"
    assert bytes(qs[0, 0]) == qs_bytes, f"{name}: qs {bytes(qs[0,0]).hex(' ')}"


def test_q4_0_golden_blocks_in_a_matrix():
    """The same blocks placed at different (row, block) positions of one matrix."""
    cases = list(_q4_golden())
    N, nb = 3, len(cases)
    W = np.zeros((N, nb * 32), np.float32)
    for r in range(N):
        for b in range(nb):
            W[r, b * 32:(b + 1) * 32] = cases[(b + r) % nb][1]
    qs, d = oracle.q4_0_quantize(W)
    for r in range(N):
        for b in range(nb):
            _, _, d_bits, q_bytes = cases[(b + r) % nb]
            assert int(d[r, b]) == d_bits
            assert bytes(qs[r, b]) == q_bytes


def test_q4_0_dequant_all_codes_exact():
    """Every code 0..15 times several scales, against exact rationals."""
    for d_bits in [0x3C00, 0xB000, 0x2E66, 0x0001, 0x03FF, 0x7BFF, 0x8000, 0x1A3B, 0xC123]:
        codes = np.arange(32) % 16
        blk = (codes[:16] | (codes[16:] << 4)).astype(np.uint8)
        got = oracle.q4_0_dequantize(blk.reshape(1, 1, 16), np.array([[d_bits]], np.uint16))
        dv = _f16_frac(d_bits)
        for j in range(32):
            assert Fraction(got[0, j]) == (codes[j] - 8) * dv


def test_q4_0_all_eights_is_zero_and_impulses():
    rng = np.random.default_rng(3)
    d = rng.integers(0, 0x7C00, (4, 2), dtype=np.uint16)
    qs = np.full((4, 2, 16), 0x88, np.uint8)
    assert np.all(oracle.q4_0_dequantize(qs, d) == 0.0)
    for j in range(32):
        qs = np.full((1, 1, 16), 0x88, np.uint8)
        if j < 16:
            qs[0, 0, j] = 0x89
        else:
            qs[0, 0, j - 16] = 0x98
        dd = np.array([[0x3555]], np.uint16)
        got = oracle.q4_0_dequantize(qs, dd)[0]
        want = np.zeros(32)
        want[j] = float(_f16_frac(0x3555))
        assert np.array_equal(got, want), j


def _block_reference_scale(W):
    """d32 of each block recomputed with numpy: first largest-magnitude weight / -8."""
    N, K = W.shape
    blocks = W.reshape(N, K // 32, 32)
    idx = np.argmax(np.abs(blocks), axis=2)          # first index on ties
    mx = np.take_along_axis(blocks, idx[..., None], 2)[..., 0]
    return (mx / np.float32(-8.0)).astype(np.float32), idx


def test_q4_0_roundtrip_bound_and_codes():
    """|w - w^| <= |d|/2 (+ scale rounding) unclamped, <= |d| clamped (both signs of max)."""
    rng = np.random.default_rng(7)
    W = synth.weights(rng, 257, 1024)
    W[:3] *= -1  # both signs of extreme are exercised anyway; flip some rows for variety
    qs, d = oracle.q4_0_quantize(W)
    What = oracle.q4_0_dequantize(qs, d).reshape(W.shape[0], -1, 32)
    d32, idx = _block_reference_scale(W)
    d16 = np.array([[float(_f16_frac(v)) for v in row] for row in d], np.float64)
    Wb = W.reshape(W.shape[0], -1, 32).astype(np.float64)
    err = np.abs(Wb - What)
    ad32 = np.abs(d32.astype(np.float64))[..., None]
    slack = 8 * np.abs(d16 - d32)[..., None] + 1e-6 * ad32
    codes = np.stack([_unpack_q4(qs[n, b]) for n in range(qs.shape[0]) for b in range(qs.shape[1])])
    codes = codes.reshape(Wb.shape)
    assert codes.min() >= 0 and codes.max() <= 15
    # the extreme element gets code 0 (it is reproduced up to the scale's rounding)
    assert np.all(np.take_along_axis(codes, idx[..., None], 2) == 0)
    clamped = (Wb / d32.astype(np.float64)[..., None] + 8.5) >= 16
    assert np.all(err[~clamped] <= ad32.repeat(32, 2)[~clamped] / 2 + slack.repeat(32, 2)[~clamped])
    assert np.all(err[clamped] <= ad32.repeat(32, 2)[clamped] + slack.repeat(32, 2)[clamped])
    assert np.all(codes[clamped] == 15)
    # clamping only happens opposite in sign to the extreme, above 15/16 of its magnitude
    frac = clamped.mean()
    assert 0.0 < frac < 0.02


# --------------------------------------------------------------------------
# Q8_1
# --------------------------------------------------------------------------

def _q8_golden():
    for name, xs, dhex, shex, qs in _golden_lines("q8_1_blocks.txt"):
        x = np.zeros(32, np.float32)
        if xs:
            for item in xs.split(","):
                i, v = item.split("=")
                x[int(i)] = np.float32(float(v))
        q = np.zeros(32, np.int8)
        if qs:
            for item in qs.split(","):
                i, v = item.split("=")
                q[int(i)] = int(v)
        yield name, x, int(dhex, 16), int(shex, 16), q


@pytest.mark.parametrize("case", list(_q8_golden()), ids=lambda c: c[0])
def test_q8_1_golden_blocks(case):
    name, x, d_bits, s_bits, q = case
    qs, ds = oracle.q8_1_quantize(x.reshape(1, 32))
    assert int(ds[0, 0, 0]) == d_bits, f"{name}: d {int(ds[0,0,0]):04x}"
    assert int(ds[0, 0, 1]) == s_bits, f"{name}: s {int(ds[0,0,1]):04x}"
    assert np.array_equal(qs[0], q)


def test_q8_1_invariants():
    rng = np.random.default_rng(11)
    X = synth.activations(rng, 33, 512) * np.float32(3.0)
    qs, ds = oracle.q8_1_quantize(X)
    blocks = X.reshape(33, -1, 32).astype(np.float64)
    q = qs.reshape(33, -1, 32).astype(np.int64)
    assert np.abs(q).max() <= 127
    amax = np.abs(blocks).max(axis=2)
    d32 = (amax / 127.0)
    # the largest-magnitude element maps to +-127
    idx = np.argmax(np.abs(blocks), axis=2)
    assert np.all(np.abs(np.take_along_axis(q, idx[..., None], 2)) == 127)
    # |x - q d| <= d/2 (+ binary32 slack)
    err = np.abs(blocks - q * d32[..., None])
    assert np.all(err <= d32[..., None] * (0.5 + 1e-5))
    # s is binary16(d * sum q), checked against numpy's conversions
    d16 = ds[..., 0].view(np.float16).astype(np.float64)
    assert np.allclose(d16, d32, rtol=2 ** -11)
    s_want = (d32.astype(np.float32) * q.sum(axis=2).astype(np.float32)).astype(np.float32).astype(np.float16)
    assert np.array_equal(ds[..., 1], s_want.view(np.uint16))


# --------------------------------------------------------------------------
# Integer block dots and the decode GEMV, vs exact integer / rational arithmetic
# --------------------------------------------------------------------------

def test_block_dots_brute_force():
    rng = np.random.default_rng(5)
    M, N, K = 3, 5, 96
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K)
    wqs, wd = oracle.q4_0_quantize(W)
    xqs, xds = oracle.q8_1_quantize(X)
    got = oracle.q4q8_block_dots(wqs, xqs)
    for m in range(M):
        for n in range(N):
            for b in range(K // 32):
                c = _unpack_q4(wqs[n, b]) - 8
                a = xqs[m, b * 32:(b + 1) * 32].astype(np.int64)
                assert got[m, n, b] == int(sum(int(c[j]) * int(a[j]) for j in range(32)))


def test_block_dots_extremes():
    wqs = np.zeros((2, 1, 16), np.uint8)           # all codes 0  -> -8
    wqs[1] = 0xFF                                 # all codes 15 -> +7
    xqs = np.full((1, 32), -127, np.int8)
    got = oracle.q4q8_block_dots(wqs, xqs)
    assert got[0, 0, 0] == 32512 and got[0, 1, 0] == -28448
    xqs = np.full((1, 32), 127, np.int8)
    got = oracle.q4q8_block_dots(wqs, xqs)
    assert got[0, 0, 0] == -32512 and got[0, 1, 0] == 28448


def test_q4q8_gemv_exact_rational():
    rng = np.random.default_rng(9)
    for (M, N, K) in [(1, 3, 32), (2, 5, 64), (3, 2, 96)]:
        W = synth.weights(rng, N, K)
        X = synth.activations(rng, M, K)
        wqs, wd = oracle.q4_0_quantize(W)
        xqs, xds = oracle.q8_1_quantize(X)
        got = oracle.q4q8_gemv(wqs, wd, xqs, xds)
        for m in range(M):
            for n in range(N):
                acc = Fraction(0)
                for b in range(K // 32):
                    c = _unpack_q4(wqs[n, b]) - 8
                    for j in range(32):
                        acc += (int(c[j]) * _f16_frac(wd[n, b])) * (int(xqs[m, b * 32 + j]) * _f16_frac(xds[m, b, 0]))
                assert abs(Fraction(got[m, n]) - acc) <= abs(acc) * Fraction(1, 2**50) + Fraction(1, 2**80)


def test_q4q8_gemv_is_dequant_product():
    """The integer path equals dequant(W) . dequant(Q8_1(x)) (BLAS, float64)."""
    rng = np.random.default_rng(12)
    W = synth.weights(rng, 300, 1024)
    X = synth.activations(rng, 4, 1024)
    wqs, wd = oracle.q4_0_quantize(W)
    xqs, xds = oracle.q8_1_quantize(X)
    y = oracle.q4q8_gemv(wqs, wd, xqs, xds)
    ref = oracle.q8_1_dequantize(xqs, xds) @ oracle.q4_0_dequantize(wqs, wd).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_unit_scales_give_integer_sums():
    """With every d = 1 the GEMV output is the plain integer sum of block dots."""
    rng = np.random.default_rng(13)
    N, K, M = 7, 256, 2
    wqs = rng.integers(0, 256, (N, K // 32, 16), dtype=np.uint8)
    wd = np.full((N, K // 32), 0x3C00, np.uint16)
    xqs = rng.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    xds = np.zeros((M, K // 32, 2), np.uint16)
    xds[..., 0] = 0x3C00
    y = oracle.q4q8_gemv(wqs, wd, xqs, xds)
    for m in range(M):
        for n in range(N):
            c = np.concatenate([_unpack_q4(wqs[n, b]) for b in range(K // 32)]) - 8
            assert y[m, n] == float(np.dot(c, xqs[m].astype(np.int64)))


# --------------------------------------------------------------------------
# binary64 matmul
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (5, 2, 96), (3, 5, 32)])
def test_matmul_exact_rational(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    got = oracle.matmul_f64(x, w)
    assert got.shape == (M, N)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(x[m, k]) * Fraction(w[n, k]) for k in range(K))
            assert abs(Fraction(got[m, n]) - exact) <= Fraction(K * 2 ** -50) * sum(
                abs(Fraction(x[m, k]) * Fraction(w[n, k])) for k in range(K))


def test_matmul_blas_one_hot_and_linearity():
    rng = np.random.default_rng(21)
    W = synth.weights(rng, 129, 512)
    wqs, wd = oracle.q4_0_quantize(W)
    What = oracle.q4_0_dequantize(wqs, wd)
    X = synth.bf16_bits_to_f32(synth.bf16_bits(synth.activations(rng, 6, 512))).astype(np.float64)
    y = oracle.matmul_f64(X, What)
    assert np.allclose(y, X @ What.T, rtol=1e-12, atol=1e-13)
    # one-hot rows pick columns of W^: Y[:, n] = W^[n, k]
    ks = [0, 1, 31, 32, 257, 511]
    E = np.zeros((len(ks), 512))
    E[np.arange(len(ks)), ks] = 1.0
    yE = oracle.matmul_f64(E, What)
    assert np.array_equal(yE, What[:, ks].T)
    # linearity
    y2 = oracle.matmul_f64(2.0 * X[:2] + X[2:4], What)
    assert np.allclose(y2, 2.0 * y[:2] + y[2:4], rtol=1e-12, atol=1e-13)
    # sampled form agrees with the full one
    ms = np.array([0, 5, 3, 3])
    ns = np.array([128, 0, 64, 7])
    assert np.array_equal(oracle.matmul_f64_sampled(X, What, ms, ns), y[ms, ns])


# --------------------------------------------------------------------------
# affine 4-bit
# --------------------------------------------------------------------------

def _rle(spec, conv):
    out = []
    for item in spec.split(","):
        v, c = item.split("*")
        out += [conv(v)] * int(c)
    return out


@pytest.mark.parametrize("case", list(_golden_lines("affine4_groups.txt")), ids=lambda c: c[0])
def test_affine4_golden_groups(case):
    name, vals, shex, bhex, codes = case
    w = np.array(_rle(vals, float), np.float32)
    assert w.size == 64
    wb = synth.bf16_bits(w).reshape(1, 64)
    q, s, b = oracle.affine4_quantize(wb, 64)
    assert int(s[0, 0]) == int(shex, 16) and int(b[0, 0]) == int(bhex, 16), name
    c = np.array(_rle(codes, int))
    packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)
    assert np.array_equal(q[0], packed), name


def test_affine4_ramp_codes():
    """w_j = j/64: min 0, max 63/64, s = bfloat16(63/960) = 67/1024, q_j = round(16 j / 67)."""
    j = np.arange(64)
    w = (j / 64.0).astype(np.float32)
    q, s, b = oracle.affine4_quantize(synth.bf16_bits(w).reshape(1, 64), 64)
    assert _bf16_frac(s[0, 0]) == Fraction(67, 1024) and int(b[0, 0]) == 0
    codes = np.stack([q[0] & 0x0F, q[0] >> 4], axis=1).reshape(-1)
    want = [int(Fraction(16 * i, 67) + Fraction(1, 2)) for i in range(64)]
    assert codes.tolist() == want


def _bf16_frac(bits):
    return Fraction(float(torch.tensor([int(bits)], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()))


def test_affine4_roundtrip_bound_and_dequant_exact():
    rng = np.random.default_rng(17)
    W = synth.bf16_bits(synth.weights(rng, 64, 512))
    q, s, b = oracle.affine4_quantize(W, 64)
    What = oracle.affine4_dequantize(q, s, b, 64)
    Wf = synth.bf16_bits_to_f32(W).astype(np.float64).reshape(64, -1, 64)
    s64 = np.vectorize(lambda v: float(_bf16_frac(v)))(s)
    b64 = np.vectorize(lambda v: float(_bf16_frac(v)))(b)
    mn, mx = Wf.min(axis=2), Wf.max(axis=2)
    assert np.array_equal(b64, mn)                      # bias is the exact group minimum
    s32 = (mx - mn) / 15.0
    err = np.abs(Wf - What.reshape(Wf.shape))
    assert np.all(err <= (s64 / 2 + 15 * np.abs(s32 - s64) + 1e-9)[..., None])
    # exact dequant: q*s + b with codes unpacked here
    codes = np.stack([q & 0x0F, q >> 4], axis=2).reshape(64, 512).astype(np.int64)
    for n in (0, 17, 63):
        for k in (0, 1, 63, 64, 200, 511):
            assert Fraction(What[n, k]) == codes[n, k] * _bf16_frac(s[n, k // 64]) + _bf16_frac(b[n, k // 64])


# --------------------------------------------------------------------------
# affine 8-bit
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", list(_golden_lines("affine8_groups.txt")), ids=lambda c: c[0])
def test_affine8_golden_groups(case):
    name, vals, shex, bhex, codes = case
    w = np.array(_rle(vals, float), np.float32)
    assert w.size == 64
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(w).reshape(1, 64), 64)
    assert int(s[0, 0]) == int(shex, 16) and int(b[0, 0]) == int(bhex, 16), name
    assert q[0].tolist() == _rle(codes, int), name


def test_affine8_ramp_codes():
    """w_j = j/64: min 0, max 63/64, s = bfloat16(63/16320) = 253/65536, q_j = round(1024 j / 253)."""
    j = np.arange(64)
    w = (j / 64.0).astype(np.float32)
    q, s, b = oracle.affine8_quantize(synth.bf16_bits(w).reshape(1, 64), 64)
    assert _bf16_frac(s[0, 0]) == Fraction(253, 65536) and int(b[0, 0]) == 0
    want = [int(Fraction(1024 * i, 253) + Fraction(1, 2)) for i in range(64)]
    assert q[0].tolist() == want


def test_affine8_roundtrip_bound_and_dequant_exact():
    rng = np.random.default_rng(19)
    W = synth.bf16_bits(synth.weights(rng, 48, 512))
    q, s, b = oracle.affine8_quantize(W, 64)
    What = oracle.affine8_dequantize(q, s, b, 64)
    Wf = synth.bf16_bits_to_f32(W).astype(np.float64).reshape(48, -1, 64)
    s64 = np.vectorize(lambda v: float(_bf16_frac(v)))(s)
    b64 = np.vectorize(lambda v: float(_bf16_frac(v)))(b)
    mn, mx = Wf.min(axis=2), Wf.max(axis=2)
    assert np.array_equal(b64, mn)                      # bias is the exact group minimum
    s32 = (mx - mn) / 255.0
    err = np.abs(Wf - What.reshape(Wf.shape))
    assert np.all(err <= (s64 / 2 + 255 * np.abs(s32 - s64) + 1e-9)[..., None])
    assert err.max() < np.abs(Wf).max() / 200           # 8 bits: far finer than 4
    for n in (0, 17, 47):
        for k in (0, 1, 63, 64, 200, 511):
            assert Fraction(What[n, k]) == int(q[n, k]) * _bf16_frac(s[n, k // 64]) + _bf16_frac(b[n, k // 64])
    ex = What.astype(np.float32)                        # q*s + b is exact in binary32 here
    assert np.array_equal(ex.astype(np.float64), What)
    assert np.array_equal(oracle.affine8_dequantize_half(q, s, b, "f16"), ex.astype(np.float16).view(np.uint16))
    want_bf = torch.from_numpy(ex).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.affine8_dequantize_half(q, s, b, "bf16"), want_bf)


# --------------------------------------------------------------------------
# dequantise to 16-bit dense types: RNE of the binary32 value
# --------------------------------------------------------------------------

def test_dequant_half_matches_library_rounding():
    rng = np.random.default_rng(23)
    W = synth.weights(rng, 40, 256)
    qs, d = oracle.q4_0_quantize(W)
    exact = oracle.q4_0_dequantize(qs, d).astype(np.float32)   # exact in binary32
    assert np.array_equal(oracle.q4_0_dequantize_half(qs, d, "f16"), exact.astype(np.float16).view(np.uint16))
    want_bf = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.q4_0_dequantize_half(qs, d, "bf16"), want_bf)
    Wb = synth.bf16_bits(W * np.float32(50.0))
    q, s, b = oracle.affine4_quantize(Wb, 64)
    ex = oracle.affine4_dequantize(q, s, b, 64).astype(np.float32)
    assert np.array_equal(oracle.affine4_dequantize_half(q, s, b, "f16"), ex.astype(np.float16).view(np.uint16))
    want_bf = torch.from_numpy(ex).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.affine4_dequantize_half(q, s, b, "bf16"), want_bf)


# --------------------------------------------------------------------------
# Error budget of the 2e-3 bar (relative Frobenius vs the binary64 oracle)
# --------------------------------------------------------------------------

def test_error_budget_bf16_output_and_weights():
    """bf16 output rounding alone fits the bar; bf16-rounded weights plus bf16 output do not."""
    rng = np.random.default_rng(0)
    N, K, M = 1024, 4096, 64
    W = synth.weights(rng, N, K)
    X = synth.bf16_bits_to_f32(synth.bf16_bits(synth.activations(rng, M, K))).astype(np.float64)
    qs, d = oracle.q4_0_quantize(W)
    What = oracle.q4_0_dequantize(qs, d)
    Y = X @ What.T

    def bf16_round(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()

    e_out = oracle.rel_frobenius(bf16_round(Y), Y)
    W16 = oracle.f16_bits_to_f32(oracle.q4_0_dequantize_half(qs, d, "f16")).astype(np.float64)
    Wbf = oracle.bf16_bits_to_f32(oracle.q4_0_dequantize_half(qs, d, "bf16")).astype(np.float64)
    e_f16w = oracle.rel_frobenius(bf16_round(X @ W16.T), Y)
    e_bfw = oracle.rel_frobenius(bf16_round(X @ Wbf.T), Y)
    assert 1.4e-3 < e_out < 1.9e-3
    assert e_f16w < 1.9e-3
    assert e_bfw > 2e-3
