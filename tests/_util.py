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


def sentinel(shape, dtype: str):
    """A device tensor whose every element is a sentinel no kernel result can equal: fp16
    NaN (0x7E00) or int32 0x7FFFFFFF (beyond any accumulator the ABI allows) or int32 -7.
    Outputs are pre-filled with it so that an element a kernel leaves unwritten fails the
    comparison instead of passing on a stale allocation."""
    import torch

    if dtype == "f16":
        return torch.full(shape, 0x7E00, dtype=torch.int16, device="cuda").view(torch.float16)
    if dtype == "i32":
        return torch.full(shape, 0x7FFFFFFF, dtype=torch.int32, device="cuda")
    if dtype == "idx":
        return torch.full(shape, -7, dtype=torch.int32, device="cuda")
    raise ValueError(dtype)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits16(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint16)


def max_abs_rel(y: np.ndarray, r: np.ndarray) -> float:
    """max |y - r| / max |r| over the tensor (the fp16 output bar of the W4A16 path).  A NaN
    anywhere in y (an unwritten sentinel) makes the result NaN, which fails every <= bar."""
    y = y.astype(np.float64)
    r = r.astype(np.float64)
    denom = np.abs(r).max()
    d = np.abs(y - r)
    if np.isnan(d).any():
        return float("nan")
    err = d.max()
    return float(err / denom) if denom > 0 else float(err)


def rel_large(y: np.ndarray, r: np.ndarray, frac: float = 0.1) -> float:
    """max |y - r| / |r| over the elements with |r| > frac * max|r| (the element-wise relative
    error reported beside max_abs_rel; NaN if y holds a NaN)."""
    y = y.astype(np.float64)
    r = r.astype(np.float64)
    big = np.abs(r) > frac * np.abs(r).max()
    if np.isnan(y).any():
        return float("nan")
    if not big.any():
        return 0.0
    return float((np.abs(y - r)[big] / np.abs(r)[big]).max())


# (test id, max_abs_rel, element-wise relative error on the large outputs) of every check_fp
# call in this session; the terminal summary (conftest.py) reports the worst of each.
FP_ERRORS: list = []


def assert_all_written(y: np.ndarray, what: str = "y") -> None:
    """Where only sampled columns meet the oracle, every other element must still have been
    written: no fp16 NaN (the sentinel) may remain, since finite inputs give finite results."""
    bad = np.isnan(y.astype(np.float32))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements left unwritten, first at {np.argwhere(bad)[0].tolist()}"


def check_fp(y: np.ndarray, r: np.ndarray, tol: float, what: str = "y") -> None:
    """The fp16 output bar: max_abs_rel <= tol.  The element-wise relative error on the large
    outputs is recorded beside it (and shown in the message on failure)."""
    import os

    e = max_abs_rel(y, r)
    el = rel_large(y, r)
    FP_ERRORS.append((os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], e, el))
    assert e <= tol, f"{what}: max-abs-rel {e:.3e} > {tol} (element-wise rel on |r| > 0.1 max: {el:.3e})"


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
