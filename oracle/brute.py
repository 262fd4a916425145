"""Exact-rational brute force for tiny inputs (test infrastructure).

A second, independent route to the oracle's results: every quantity is a
``fractions.Fraction`` and every IEEE rounding the method performs is done explicitly
from the definition of round-to-nearest-even on the target format's grid.  It shares no
code with ``qv_oracle.c`` (which works in C floats) and none with the GPU path.  Pure
Python loops: only for inputs of a few hundred elements.

Passages followed are the same as the oracle's: Quasar Sec. 3.2-3.3 (per-token int8
activations, int8 GEMM, dequantisation), the W4A16 verify forward of the Speculative
Decoding Meets Quantization review page, and greedy acceptance (Quasar Sec. 4.2, 4.5).
"""
from __future__ import annotations

from fractions import Fraction
from math import floor

import numpy as np


# ---- rounding on a binary floating-point grid, from the definition ----------------------

def _round_half_even_int(q: Fraction) -> int:
    """Nearest integer to q, ties to the even integer."""
    f = floor(q)
    r = q - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def _exponent(a: Fraction) -> int:
    """e with 2^e <= a < 2^(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_format(v: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction | float:
    """Round v to nearest-even on the grid of a binary format with `mant_bits` fraction
    bits, smallest normal exponent `emin` and largest exponent `emax`.  Returns a Fraction,
    or +-inf on overflow."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_exponent(a), emin)
    quantum = Fraction(2) ** (e - mant_bits)
    r = _round_half_even_int(a / quantum) * quantum
    if r >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * r


def to_f32(v: Fraction):
    return round_to_format(v, 23, -126, 127)


def to_f16(v: Fraction):
    return round_to_format(v, 10, -14, 15)


def f16_bits_to_fraction(bits: int) -> Fraction:
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    assert e != 31, "non-finite input"
    if e == 0:
        return sign * Fraction(f, 2 ** 24)
    return sign * Fraction(1024 + f, 1024) * Fraction(2) ** (e - 15)


def fraction_to_f16_bits(v) -> int:
    """Encode an exactly representable binary16 value (or +-inf)."""
    if isinstance(v, float):
        assert v in (float("inf"), float("-inf"))
        return 0x7C00 | (0x8000 if v < 0 else 0)
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    if a < Fraction(2) ** -14:
        m = a * 2 ** 24
        assert m.denominator == 1
        return sign | int(m)
    e = _exponent(a)
    m = a / Fraction(2) ** (e - 10) - 1024
    assert m.denominator == 1 and 0 <= m < 1024
    return sign | ((e + 15) << 10) | int(m)


def f32_to_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


# ---- the method, exactly --------------------------------------------------------------------

def quant_act(x_bits: np.ndarray, inv_smooth=None):
    """Per-token symmetric int8: s = fl32(a / 127), q = clamp(rne(fl32(x' / s)), +-127)."""
    M, K = x_bits.shape
    xq = np.zeros((M, K), np.int8)
    sx = np.zeros((M,), np.float32)
    for m in range(M):
        xs = []
        for k in range(K):
            v = f16_bits_to_fraction(x_bits[m, k])
            if inv_smooth is not None:
                v = to_f32(v * f32_to_fraction(inv_smooth[k]))
            xs.append(v)
        a = max(abs(v) for v in xs)
        s = to_f32(a / 127)
        sx[m] = np.float32(float(s))
        for k in range(K):
            if a == 0:
                q = 0
            else:
                t = to_f32(xs[k] / s)
                q = _round_half_even_int(t)
                q = max(-127, min(127, q))
            xq[m, k] = q
    return xq, sx


def linear_w8a8(x_q, x_scale, w, w_scale):
    """acc = exact integer dot product; y = fl16(fl32(fl32(fl32(acc) * s_x) * s_w))."""
    M, K = x_q.shape
    N = w.shape[0]
    acc = np.zeros((M, N), np.int64)
    y = np.zeros((M, N), np.uint16)
    for m in range(M):
        for n in range(N):
            a = sum(int(x_q[m, k]) * int(w[n, k]) for k in range(K))
            acc[m, n] = a
            t = to_f32(Fraction(a))
            t = to_f32(t * f32_to_fraction(x_scale[m]))
            t = to_f32(t * f32_to_fraction(w_scale[n]))
            y[m, n] = fraction_to_f16_bits(to_f16(t))
    return y, acc


def w4_dequant(qweight, scales_bits, zeros, K, group_size=128):
    """Exact dequantised weights W[n][k] = (q - z) * s as Fractions."""
    N = qweight.shape[0]
    W = [[None] * K for _ in range(N)]
    for n in range(N):
        for k in range(K):
            word = int(qweight[n, k // 8])
            q = (word >> (4 * (k % 8))) & 0xF
            g = k // group_size
            z = int(zeros[n, g])
            s = f16_bits_to_fraction(scales_bits[n, g])
            W[n][k] = (q - z) * s
    return W


def linear_w4a16(x_bits, qweight, scales_bits, zeros, group_size=128):
    """y = fl16(exact sum over k of x * (q - z) * s)."""
    M, K = x_bits.shape
    N = qweight.shape[0]
    W = w4_dequant(qweight, scales_bits, zeros, K, group_size)
    y = np.zeros((M, N), np.uint16)
    for m in range(M):
        xs = [f16_bits_to_fraction(x_bits[m, k]) for k in range(K)]
        for n in range(N):
            s = sum(xs[k] * W[n][k] for k in range(K))
            y[m, n] = fraction_to_f16_bits(to_f16(s))
    return y


def linear_w4a8(x_q, x_scale, qweight, scales_bits, zeros, group_size=128):
    """y = fl16(s_x * exact sum over k of x_q * (q - z) * s)."""
    M, K = x_q.shape
    N = qweight.shape[0]
    W = w4_dequant(qweight, scales_bits, zeros, K, group_size)
    y = np.zeros((M, N), np.uint16)
    for m in range(M):
        sx = f32_to_fraction(x_scale[m])
        for n in range(N):
            s = sum(int(x_q[m, k]) * W[n][k] for k in range(K))
            y[m, n] = fraction_to_f16_bits(to_f16(sx * s))
    return y


def argmax(logit_bits):
    M, V = logit_bits.shape
    out = np.zeros((M,), np.int32)
    for m in range(M):
        vals = [f16_bits_to_fraction(logit_bits[m, v]) for v in range(V)]
        best = max(vals)
        out[m] = min(v for v in range(V) if vals[v] == best)
    return out


def accept(draft, argmax_rows):
    """Length of the longest prefix of the draft that equals the verifier's argmax."""
    M = len(argmax_rows)
    best = 0
    for j in range(M):  # candidate lengths 0..M-1; keep the largest whose prefix matches
        if all(int(draft[i]) == int(argmax_rows[i]) for i in range(j)):
            best = j
    return best
