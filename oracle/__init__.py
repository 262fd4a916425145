"""CPU oracle for the quantized speculative-verify path.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product library never does.  It shares no code with
the GPU path.  The arithmetic lives in ``qv_oracle.c`` (plain C, built with gcc by
``oracle/build.py``); this module only marshals numpy arrays into it.  ``brute.py`` holds a
second, exact-rational implementation for tiny inputs that pins the C code.

Functions and the passages they follow:

* :func:`quant_act`    -- Quasar, Sec. 3.2 and Sec. 3.3 "Online Activation Smoothing and
  Quantization" (per-token symmetric int8, optional smoothing prescale).
* :func:`linear_w8a8`  -- Quasar, Sec. 3.3 "INT8 Gemm and Dequantization".
* :func:`linear_w4a16` -- Speculative Decoding Meets Quantization (review page): the W4A16
  target's verify forward; group-wise asymmetric 4-bit weights.
* :func:`linear_w4a8`  -- Speculative Decoding Meets Quantization (review page): the W4A8
  target (4-bit weights in the W4A16 format, per-token int8 activations as quant_act).
* :func:`argmax`, :func:`accept` -- Quasar, Sec. 4.5 (top-1 decides) and Sec. 4.2 / Table 1
  (mean acceptance length; T=0 is greedy).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqv_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_quant_act.argtypes = [P, P, I, I, P, P]
    lib.oracle_quant_act.restype = None
    lib.oracle_linear_w8a8.argtypes = [P, P, I, I, P, P, I, P, P]
    lib.oracle_linear_w8a8.restype = I
    lib.oracle_linear_w4a16.argtypes = [P, I, I, P, P, P, I, I, P]
    lib.oracle_linear_w4a16.restype = None
    lib.oracle_linear_w4a8.argtypes = [P, P, I, I, P, P, P, I, I, P]
    lib.oracle_linear_w4a8.restype = None
    lib.oracle_argmax.argtypes = [P, I, I, P]
    lib.oracle_argmax.restype = None
    lib.oracle_accept.argtypes = [P, P, I]
    lib.oracle_accept.restype = I
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_double_to_half.argtypes = [ctypes.c_double]
    lib.oracle_double_to_half.restype = ctypes.c_uint16
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    lib.oracle_set_num_threads.argtypes = [I]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits16(x: np.ndarray) -> np.ndarray:
    """fp16 array (or its uint16 bit pattern) -> contiguous uint16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    assert x.dtype == np.uint16, x.dtype
    return x


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Host threads of the OpenMP loops from now on (timing only; results do not depend on it)."""
    _load().oracle_set_num_threads(n)


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits))


def double_to_half(v: float) -> int:
    return _load().oracle_double_to_half(float(v))


def quant_act(x: np.ndarray, inv_smooth: np.ndarray | None = None):
    """x fp16 [M][K] -> (x_q int8 [M][K], x_scale fp32 [M])."""
    xb = _bits16(x)
    M, K = xb.shape
    inv = None if inv_smooth is None else np.ascontiguousarray(inv_smooth, dtype=np.float32)
    xq = np.empty((M, K), np.int8)
    sx = np.empty((M,), np.float32)
    _load().oracle_quant_act(_ptr(xb), _ptr(inv), M, K, _ptr(xq), _ptr(sx))
    return xq, sx


def linear_w8a8(x_q: np.ndarray, x_scale: np.ndarray, w: np.ndarray, w_scale: np.ndarray):
    """-> (y fp16 [M][N], acc int32 [M][N]).  Raises if a dot product leaves int32."""
    x_q = np.ascontiguousarray(x_q, dtype=np.int8)
    x_scale = np.ascontiguousarray(x_scale, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.int8)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = x_q.shape
    N, K2 = w.shape
    assert K == K2 and x_scale.shape == (M,) and w_scale.shape == (N,)
    y = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.int32)
    ovf = _load().oracle_linear_w8a8(_ptr(x_q), _ptr(x_scale), M, K, _ptr(w), _ptr(w_scale), N,
                                     _ptr(y), _ptr(acc))
    if ovf:
        raise OverflowError("int32 accumulator overflow")
    return y.view(np.float16), acc


def linear_w4a16(x: np.ndarray, qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                 group_size: int = 128):
    """x fp16 [M][K], qweight uint32 [N][K/8], scales fp16 [N][K/G], zeros uint8 [N][K/G]
    -> y fp16 [M][N]."""
    xb = _bits16(x)
    M, K = xb.shape
    qweight = np.ascontiguousarray(qweight, dtype=np.uint32)
    N = qweight.shape[0]
    assert qweight.shape == (N, K // 8) and K % group_size == 0
    sb = _bits16(scales)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    assert sb.shape == (N, K // group_size) and zeros.shape == sb.shape
    y = np.empty((M, N), np.uint16)
    _load().oracle_linear_w4a16(_ptr(xb), M, K, _ptr(qweight), _ptr(sb), _ptr(zeros), N,
                                group_size, _ptr(y))
    return y.view(np.float16)


def linear_w4a8(x_q: np.ndarray, x_scale: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                zeros: np.ndarray, group_size: int = 128):
    """x_q int8 [M][K], x_scale fp32 [M], qweight uint32 [N][K/8], scales fp16 [N][K/G],
    zeros uint8 [N][K/G] -> y fp16 [M][N] = fp16(x_scale * sum_g s_g * sum_{k in g} x_q (q - z))."""
    xq = np.ascontiguousarray(x_q, dtype=np.int8)
    M, K = xq.shape
    sx = np.ascontiguousarray(x_scale, dtype=np.float32)
    assert sx.shape == (M,)
    qweight = np.ascontiguousarray(qweight, dtype=np.uint32)
    N = qweight.shape[0]
    assert qweight.shape == (N, K // 8) and K % group_size == 0
    sb = _bits16(scales)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    assert sb.shape == (N, K // group_size) and zeros.shape == sb.shape
    y = np.empty((M, N), np.uint16)
    _load().oracle_linear_w4a8(_ptr(xq), _ptr(sx), M, K, _ptr(qweight), _ptr(sb), _ptr(zeros), N,
                               group_size, _ptr(y))
    return y.view(np.float16)


def argmax(logits: np.ndarray) -> np.ndarray:
    """logits fp16 [M][V] -> int32 [M], lowest index on ties."""
    lb = _bits16(logits)
    M, V = lb.shape
    out = np.empty((M,), np.int32)
    _load().oracle_argmax(_ptr(lb), M, V, _ptr(out))
    return out


def accept(draft: np.ndarray, argmax_rows: np.ndarray) -> int:
    """draft int32 [M-1], argmax int32 [M] -> n_accept in [0, M-1]."""
    a = np.ascontiguousarray(argmax_rows, dtype=np.int32)
    M = a.shape[0]
    d = np.ascontiguousarray(draft, dtype=np.int32)
    if M > 1:
        assert d.shape == (M - 1,)
    else:
        d = np.zeros((1,), np.int32)
    return int(_load().oracle_accept(_ptr(d), _ptr(a), M))


def verify_greedy(logits: np.ndarray, draft: np.ndarray):
    """-> (argmax int32 [M], n_accept int)."""
    a = argmax(logits)
    return a, accept(draft, a)
