"""Helpers shared by the GPU parity tests (moving arrays, comparing results)."""
from __future__ import annotations

import numpy as np


def dev(a: np.ndarray):
    """numpy -> contiguous cuda tensor (uint32 is carried as int32 bits)."""
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits16(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint16)


def max_abs_rel(y: np.ndarray, r: np.ndarray) -> float:
    """max |y - r| / max |r| over the tensor (the fp16 output bar of the W4A16 path)."""
    y = y.astype(np.float64)
    r = r.astype(np.float64)
    denom = np.abs(r).max()
    err = np.abs(y - r).max()
    return float(err / denom) if denom > 0 else float(err)


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str) -> None:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if a.dtype.itemsize == 2:
        a, b = a.view(np.uint16), b.view(np.uint16)
    elif a.dtype.itemsize == 4:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} of {a.size} elements differ, first at flat "
                           f"index {bad[0]}: {a.reshape(-1)[bad[0]]} vs {b.reshape(-1)[bad[0]]}")
