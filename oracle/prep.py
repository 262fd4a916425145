"""Offline weight preparation (TEST INFRASTRUCTURE ONLY; the product library never imports
this).

Quasar, Sec. 3.3 "Offline Weight Preparation": before inference the target's weights are
smoothed and quantised, W_hat = Q(W diag(s)^-1), and stored in device memory.  The page gives
no formula for Q and none for the 4-bit weights of the HierSpec review page; readings taken:

* :func:`prepare_w8` -- W is bf16 [N][K] (rows = output channels); the columns are multiplied
  by the entries of diag(s)^-1, given as a float32 vector inv_s[K] (omitted: 1); then each row
  is quantised as quant_act quantises a token: a = max |w'|, scale = a / 127 (float32
  division), q = clamp(rint(w' / scale), -127, 127) with rint half to even, all in float32
  (q = 0 for an all-zero row).
* :func:`prepare_w4` -- W is bf16 [N][K]; per 128-group the range [lo, hi] is the group's
  min and max widened to include 0; scale = fp16((hi - lo) / 15) (1 if that is 0); zero =
  clamp(rint(-lo / scale), 0, 15); code = clamp(rint(w / scale) + zero, 0, 15), float32
  arithmetic with the fp16 scale; codes packed eight per uint32, lowest k in the low nibble.

Plain numpy float32 (IEEE single, round to nearest even per operation).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact: the upper half of the float32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def prepare_w8(w_bits: np.ndarray, inv_s: np.ndarray | None = None):
    """bf16 bits [N][K] (+ float32 inv_s [K]) -> (int8 codes [N][K], float32 scales [N])."""
    w = bf16_to_f32(w_bits)
    if inv_s is not None:
        w = w * np.asarray(inv_s, dtype=np.float32)[None, :]
    a = np.abs(w).max(axis=1)
    scale = (a / np.float32(127)).astype(np.float32)
    q = np.zeros(w.shape, np.int8)
    nz = scale != 0
    q[nz] = np.clip(np.rint(w[nz] / scale[nz, None]), -127, 127).astype(np.int8)
    return q, scale


def prepare_w4(w_bits: np.ndarray, group_size: int = 128):
    """bf16 bits [N][K] -> (qweight uint32 [N][K/8], scales fp16 [N][K/G], zeros uint8 [N][K/G])."""
    w = bf16_to_f32(w_bits)
    N, K = w.shape
    G = K // group_size
    wg = w.reshape(N, G, group_size)
    lo = np.minimum(wg.min(axis=2), np.float32(0))
    hi = np.maximum(wg.max(axis=2), np.float32(0))
    s16 = ((hi - lo) / np.float32(15)).astype(np.float16)
    s16[s16 == 0] = np.float16(1)
    s = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / s), 0, 15).astype(np.float32)
    codes = np.clip(np.rint(wg / s[:, :, None]) + z[:, :, None], 0, 15).astype(np.uint32)
    codes = codes.reshape(N, K // 8, 8)
    qweight = np.bitwise_or.reduce(codes << (4 * np.arange(8, dtype=np.uint32)), axis=2)
    return qweight.astype(np.uint32), s16, z.astype(np.uint8)
