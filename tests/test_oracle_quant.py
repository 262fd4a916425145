"""Pins for the oracle's per-token activation quantisation.

Definition (Quasar Sec. 3.2 and Sec. 3.3 "Online Activation Smoothing and Quantization";
the legible text fixes per-token int8 activations after smoothing; absmax/127 symmetric
scaling with round-half-even is the reading taken where the formulas are missing):
  x' = x * inv_s (fp32), a = max |x'|, s = fl32(a / 127), q = clamp(rne(fl32(x' / s)), -127, 127).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute


def _rand_x(g, M, K, scale=1.0):
    return (g.standard_normal((M, K)) * scale).astype(np.float16)


@pytest.mark.parametrize("seed", range(6))
def test_quant_matches_exact_rational_brute_force(seed):
    g = np.random.default_rng(seed)
    M, K = 3, 24
    x = _rand_x(g, M, K, scale=10.0 ** g.integers(-3, 3))
    q, s = oracle.quant_act(x)
    qb, sb = brute.quant_act(x.view(np.uint16))
    np.testing.assert_array_equal(q, qb)
    np.testing.assert_array_equal(s.view(np.uint32), sb.view(np.uint32))


def test_quant_with_smoothing_matches_brute_force():
    g = np.random.default_rng(7)
    M, K = 2, 20
    x = _rand_x(g, M, K)
    inv = g.uniform(0.1, 4.0, K).astype(np.float32)
    q, s = oracle.quant_act(x, inv)
    qb, sb = brute.quant_act(x.view(np.uint16), inv)
    np.testing.assert_array_equal(q, qb)
    np.testing.assert_array_equal(s, sb)


def test_power_of_two_scale_is_exact_including_ties():
    # x = c * v with c = 2^-3 and max |v| = 127: s = c exactly and x/s = v exactly.
    c = 0.125
    v = np.array([127, -64, 3, 0, -127, 1, 100, -5], np.float64)
    half = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5])  # exact ties
    x = (np.concatenate([v, half]) * c).astype(np.float16)[None, :]
    assert np.all(x.astype(np.float64)[0] == np.concatenate([v, half]) * c)
    q, s = oracle.quant_act(x)
    assert s[0] == np.float32(c)
    want_ties = [0, 2, 2, 0, -2, -2, 126, -126]  # round half to even
    np.testing.assert_array_equal(q[0], np.concatenate([v, want_ties]).astype(np.int8))


def test_zero_row_gives_zero_scale_and_codes():
    x = np.zeros((2, 64), np.float16)
    x[1, 5] = -3.0
    q, s = oracle.quant_act(x)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert q[1, 5] == -127 and np.count_nonzero(q[1]) == 1


@pytest.mark.parametrize("seed", range(4))
def test_quant_invariants(seed):
    g = np.random.default_rng(100 + seed)
    M, K = 16, 4096
    x = _rand_x(g, M, K, scale=float(g.uniform(0.01, 100)))
    q, s = oracle.quant_act(x)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    xd = x.astype(np.float64)
    a = np.max(np.abs(xd), axis=1)
    # s is a/127 rounded once to fp32
    np.testing.assert_allclose(s.astype(np.float64), a / 127, rtol=2.0 ** -24)
    # |q s - x| <= s (1/2 + 2^-17): one fp32 rounding of x/s, then one rounding to an integer
    err = np.abs(q.astype(np.float64) * s.astype(np.float64)[:, None] - xd)
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -17))


def test_unit_smoothing_is_identity_and_power_of_two_smoothing_is_exact():
    g = np.random.default_rng(5)
    x = _rand_x(g, 4, 256)
    q0, s0 = oracle.quant_act(x)
    q1, s1 = oracle.quant_act(x, np.ones(256, np.float32))
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(s0, s1)
    # per-channel powers of two: quantising x*diag(2^e) must equal quantising the exactly
    # scaled fp16 tensor (no fp16 overflow/underflow for these magnitudes)
    e = g.integers(-2, 3, 256)
    inv = (2.0 ** e).astype(np.float32)
    xs = (x.astype(np.float64) * 2.0 ** e).astype(np.float16)
    assert np.all(xs.astype(np.float64) == x.astype(np.float64) * 2.0 ** e)
    q2, s2 = oracle.quant_act(x, inv)
    q3, s3 = oracle.quant_act(xs)
    np.testing.assert_array_equal(q2, q3)
    np.testing.assert_array_equal(s2, s3)


def test_brute_force_rounding_helpers():
    # the exact-rational helpers themselves against numpy's IEEE conversions
    g = np.random.default_rng(9)
    for v in g.standard_normal(300) * 10.0 ** g.integers(-6, 6, 300):
        assert float(brute.to_f32(Fraction(float(v)))) == float(np.float32(v))
        assert brute.fraction_to_f16_bits(brute.to_f16(Fraction(float(v)))) == int(np.float16(v).view(np.uint16))
