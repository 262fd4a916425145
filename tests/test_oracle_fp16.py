"""Pins for the oracle's binary16 conversions.

The oracle writes its own fp16 encode/decode from the format's definition; numpy's float16
(a correctly rounded, round-half-even library conversion) is the independent reference.
"""
import numpy as np

import oracle


def test_decode_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    for b in bits[finite][::97]:
        assert oracle.half_to_double(int(b)) == float(np.uint16(b).view(np.float16))
    # every pattern in a dense stride, including subnormals and both zeros
    for b in list(range(0, 1100)) + list(range(0x8000, 0x8000 + 1100)) + [0x7BFF, 0xFBFF, 0x0400, 0x03FF]:
        assert oracle.half_to_double(b) == float(np.uint16(b).view(np.float16))


def test_encode_matches_numpy_random():
    g = np.random.default_rng(1)
    vals = np.concatenate([
        g.standard_normal(4000) * 10.0 ** g.integers(-8, 5, 4000),
        g.uniform(-70000, 70000, 500),
    ])
    for v in vals:
        assert oracle.double_to_half(float(v)) == int(np.float16(v).view(np.uint16)), v


def test_encode_ties_and_edges():
    # exact midpoints between neighbouring fp16 values must go to the even significand
    for lo_bits in [0x3C00, 0x3C01, 0x0001, 0x0002, 0x03FF, 0x7BFE, 0x5640]:
        lo = float(np.uint16(lo_bits).view(np.float16))
        hi = float(np.uint16(lo_bits + 1).view(np.float16))
        mid = (lo + hi) / 2
        want = lo_bits if lo_bits % 2 == 0 else lo_bits + 1
        assert oracle.double_to_half(mid) == want
        assert oracle.double_to_half(-mid) == want | 0x8000
    assert oracle.double_to_half(65504.0) == 0x7BFF
    assert oracle.double_to_half(65519.99) == 0x7BFF
    assert oracle.double_to_half(65520.0) == 0x7C00  # tie rounds to even -> overflow
    assert oracle.double_to_half(2.0 ** -25) == 0  # half of the smallest subnormal: tie to 0
    assert oracle.double_to_half(2.0 ** -25 * 1.0001) == 1
    assert oracle.double_to_half(-0.0) == 0x8000
