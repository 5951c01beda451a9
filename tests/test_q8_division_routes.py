"""The Q8_1 quantiser's two binary32 divisions (d = amax / 127, then 1 / d;
"2026-05-06 Q4 sync-after focused repro", Important source touch points: the
q8_1 activation blocks) run on the GPU through binary64: amax * RN64(1/127)
rounded to binary32, and a binary64 reciprocal refined by two Newton steps
rounded to binary32.  Both must give exactly what binary32 division gives.

This is a property of IEEE arithmetic, checked here on the host with numpy
(binary32 division as the reference).  The reciprocal is emulated with a
start 2^-22 away from 1/d in either direction (the device instruction is
closer) and without fused multiply-add (the device uses it), so the checked
error is larger than the device's.  The full sweep over every non-negative
finite binary32 value found no mismatch (Q4_EXHAUSTIVE=1 runs it, about
3 minutes); by default a sample of it runs: every 61st bit pattern, and
every pattern in the binades around the subnormal boundary, around 1 and
below the largest finite value.
"""
import os

import numpy as np
import pytest

INV127 = np.float64(1.0) / np.float64(127.0)


def _check(bits: np.ndarray) -> tuple[int, int]:
    a = bits.view(np.float32)
    ref = a / np.float32(127.0)
    got = (a.astype(np.float64) * INV127).astype(np.float32)
    bad127 = int(np.count_nonzero(ref.view(np.uint32) != got.view(np.uint32)))
    d = a[a > 0]
    badr = 0
    with np.errstate(over="ignore", divide="ignore"):
        refr = np.float32(1.0) / d
        x = d.astype(np.float64)
        for sgn in (1.0, -1.0):
            r = (1.0 / x) * (1.0 + sgn * 2.0 ** -22)
            for _ in range(2):
                e = 1.0 - x * r
                r = r + r * e
            badr += int(np.count_nonzero(refr.view(np.uint32) != r.astype(np.float32).view(np.uint32)))
    return bad127, badr


def _ranges():
    if os.environ.get("Q4_EXHAUSTIVE") == "1":
        step = 1 << 26
        for lo in range(0, 0x7F800000, step):
            yield np.arange(lo, min(lo + step, 0x7F800000), dtype=np.uint32)
        return
    yield np.arange(0, 0x7F800000, 61, dtype=np.uint32)
    for lo, hi in ((0x00000000, 0x01000000),      # subnormals and the first normal binades
                   (0x3F000000, 0x40000000),      # [0.5, 2)
                   (0x7E800000, 0x7F800000)):     # the last two finite binades
        yield np.arange(lo, hi, dtype=np.uint32)


def test_binary64_routes_equal_binary32_division():
    bad127 = badr = 0
    for bits in _ranges():
        b1, b2 = _check(bits)
        bad127 += b1
        badr += b2
    assert bad127 == 0, f"{bad127} inputs where amax * RN64(1/127) rounds differently from amax / 127"
    assert badr == 0, f"{badr} inputs where the refined binary64 reciprocal rounds differently from 1 / d"


@pytest.mark.parametrize("mutant", ["one_newton_step", "binary32_constant"])
def test_the_check_catches_weaker_routes(mutant):
    """A route with one Newton step, or with the binary32 constant 1/127,
    does differ from binary32 division somewhere: the check can tell."""
    bits = np.arange(0x3F000000, 0x40000000, 7, dtype=np.uint32)
    a = bits.view(np.float32)
    if mutant == "binary32_constant":
        got = a * np.float32(1.0 / 127.0)
        ref = a / np.float32(127.0)
    else:
        x = a.astype(np.float64)
        r = (1.0 / x) * (1.0 + 2.0 ** -22)
        e = 1.0 - x * r
        r = r + r * e
        got = r.astype(np.float32)
        ref = np.float32(1.0) / a
    assert np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)) > 0
