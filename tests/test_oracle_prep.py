"""Pins for the offline weight preparation oracle (oracle/prep.py).

W8: brute force with exact rationals (each float32 operation rounded once); s = 1 on values
exact in fp16 reduces to the C oracle's quant_act; scaling a column by inv_s scales it
exactly when inv_s is a power of two; the error bound |q scale - w'| <= scale / 2 inside the
range.  W4: a round trip (quantising exactly dequantised weights whose groups use codes 0
and 15 returns the same codes, scales and zero points); zero is exactly representable;
dequantisation error <= scale / 2; constant and all-zero groups; nibble packing.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.prep import bf16_to_f32, prepare_w4, prepare_w8


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values that are exact in bfloat16 -> their bit patterns."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert not (b & 0xFFFF).any(), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def rand_bf16(rng, shape, scale=0.02):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do


def test_bf16_decode():
    assert bf16_to_f32(np.array([0x3F80, 0xC000, 0x0000, 0x8000], np.uint16)).tolist() == [1.0, -2.0, 0.0, -0.0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_w8_matches_exact_brute_force(seed):
    rng = np.random.default_rng(seed)
    N, K = 3, 40
    wb = rand_bf16(rng, (N, K))
    inv = rng.uniform(0.5, 2.0, K).astype(np.float32)
    q, sc = prepare_w8(wb, inv)
    for n in range(N):
        wp = [brute.to_f32(Fraction(float(bf16_to_f32(wb[n, k]))) * Fraction(float(inv[k]))) for k in range(K)]
        a = max(abs(v) for v in wp)
        s = brute.to_f32(a / 127)
        assert Fraction(float(sc[n])) == s
        for k in range(K):
            t = brute.to_f32(wp[k] / s)
            code = max(-127, min(127, brute._round_half_even_int(t)))
            assert q[n, k] == code


def test_w8_unit_smoothing_reduces_to_quant_act():
    rng = np.random.default_rng(3)
    N, K = 6, 256
    vals = rng.integers(-128, 128, (N, K)).astype(np.float32) / 16  # exact in fp16 and bf16
    q, sc = prepare_w8(f32_to_bf16_bits(vals))
    q2, sc2 = oracle.quant_act(vals.astype(np.float16))
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(sc.view(np.uint32), sc2.view(np.uint32))


def test_w8_power_of_two_smoothing_scales_columns_exactly():
    rng = np.random.default_rng(4)
    N, K = 5, 128
    wb = rand_bf16(rng, (N, K))
    inv = np.full(K, 4.0, np.float32)
    q1, s1 = prepare_w8(wb)
    q4, s4 = prepare_w8(wb, inv)
    np.testing.assert_array_equal(q1, q4)
    np.testing.assert_array_equal(s4, s1 * 4)


def test_w8_error_bound_and_zero_row():
    rng = np.random.default_rng(5)
    wb = rand_bf16(rng, (8, 512))
    wb[3] = 0
    q, sc = prepare_w8(wb)
    w = bf16_to_f32(wb).astype(np.float64)
    err = np.abs(q * sc[:, None].astype(np.float64) - w)
    # |q - w/scale| <= 1/2 + the rounding of the float32 quotient (|w/scale| <= 127)
    assert (err <= sc[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -24)).all()
    assert sc[3] == 0 and not q[3].any()
    assert (np.abs(q).max(axis=1)[sc > 0] == 127).all()


def _pack(codes):
    N, K = codes.shape
    c = codes.reshape(N, K // 8, 8).astype(np.uint32)
    return np.bitwise_or.reduce(c << (4 * np.arange(8, dtype=np.uint32)), axis=2).astype(np.uint32)


def test_w4_round_trip_of_exact_weights():
    rng = np.random.default_rng(6)
    N, K = 4, 512
    G = K // 128
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    codes[:, ::128] = 0
    codes[:, 1::128] = 15                               # every group spans codes 0 .. 15
    zeros = rng.integers(0, 16, (N, G)).astype(np.uint8)
    scales = (2.0 ** rng.integers(-10, -4, (N, G))).astype(np.float16)
    w = (codes.astype(np.float32) - np.repeat(zeros, 128, 1)) * np.repeat(scales.astype(np.float32), 128, 1)
    q, s, z = prepare_w4(f32_to_bf16_bits(w))
    np.testing.assert_array_equal(q, _pack(codes))
    np.testing.assert_array_equal(s, scales)
    np.testing.assert_array_equal(z, zeros)


def test_w4_error_bound_and_zero_exact():
    rng = np.random.default_rng(7)
    N, K = 6, 1024
    wb = rand_bf16(rng, (N, K))
    q, s, z = prepare_w4(wb)
    w = bf16_to_f32(wb)
    codes = ((q[:, :, None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF).reshape(N, K)
    deq = (codes.astype(np.float64) - np.repeat(z, 128, 1)) * np.repeat(s.astype(np.float64), 128, 1)
    err = np.abs(deq - w)
    bound = np.repeat(s.astype(np.float64), 128, 1) * 0.5 * (1 + 2 ** -10)
    assert (err <= bound + 1e-12).all()
    assert (np.repeat(z, 128, 1) >= 0).all()              # code z dequantises to exactly 0


def test_w4_constant_and_zero_groups():
    K = 384
    w = np.zeros((3, K), np.float32)
    w[0, :128] = 0.5                                      # constant positive group
    w[1, 128:256] = -0.25                                 # constant negative group
    q, s, z = prepare_w4(f32_to_bf16_bits(w))
    codes = ((q[:, :, None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF).reshape(3, K)
    assert s[0, 0] == np.float16(0.5 / 15) and z[0, 0] == 0 and (codes[0, :128] == 15).all()
    assert z[1, 1] == 15 and (codes[1, 128:256] == 0).all()
    assert s[2, 0] == 1 and z[2, 0] == 0 and not codes[2].any()   # all-zero group: scale 1


def test_w4_packing_low_nibble_first():
    w = np.zeros((1, 128), np.float32)
    w[0, 1] = 1.0                                         # range [0, 1]: scale 1/15, zero 0
    q, s, z = prepare_w4(f32_to_bf16_bits(w))
    assert q[0, 0] == 0xF0 and z[0, 0] == 0
