"""ctypes view of libqv.so (the C ABI declared in include/qv.h).

Only loads the library and declares the signatures; no arithmetic happens here.  Loading
fails loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqv.so")

QV_OK, QV_ERR_NULL, QV_ERR_SHAPE, QV_ERR_ALIGN, QV_ERR_WORKSPACE, QV_ERR_HIP, QV_ERR_SCRATCH = range(7)
QV_OP_W8A8, QV_OP_W4A16, QV_OP_VERIFY, QV_OP_SAMPLE, QV_OP_W4A8 = 1, 2, 3, 4, 5
QV_MAX_M = 64
QV_W8A8_MAX_K = 131008
QV_W4A16_MAX_K = 1 << 20
QV_W4A16_GROUP = 128
QV_WORKSPACE_COUNTER_BYTES = 65536
QV_NOALLOC_SCRATCH_BYTES = 512 * 1024
QV_READ_LINEAR, QV_READ_TILES = 0, 1
QV_READ_MAX_BLOCKS = 65536

# Every symbol include/qv.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_S = ctypes.c_size_t
SIGNATURES = {
    "qv_quant_act": (_I, [_P, _P, _I, _I, _P, _P, _P]),
    "qv_prepare_w8": (_I, [_P, _P, _I, _I, _P, _P, _P]),
    "qv_prepare_w4": (_I, [_P, _I, _I, _I, _P, _P, _P, _P]),
    "qv_linear_w8a8": (_I, [_P, _P, _I, _I, _P, _P, _I, _P, _P, _P, _S, _P]),
    "qv_linear_w4a16": (_I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _S, _P]),
    "qv_linear_w4a8": (_I, [_P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _S, _P]),
    "qv_verify_greedy": (_I, [_P, _I, _I, _P, _P, _P, _P, _S, _P]),
    "qv_verify_greedy_noalloc": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "qv_verify_tree": (_I, [_P, _I, _I, _P, _P, _P, _P, _P, _P, _S, _P]),
    "qv_verify_sample": (_I, [_P, _I, _I, _P, _P, _P, ctypes.c_double, _P, _P, _S, _P]),
    "qv_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "qv_status_str": (ctypes.c_char_p, [_I]),
    "qv_version": (_I, []),
    # qv_test.h: the same calls with a work-split override array (int32[QV_TUNE_COUNT])
    "qv_test_quant_act": (_I, [_P, _P, _I, _I, _P, _P, _P, _P]),
    "qv_test_prepare_w8": (_I, [_P, _P, _I, _I, _P, _P, _P, _P]),
    "qv_test_linear_w8a8": (_I, [_P, _P, _I, _I, _P, _P, _I, _P, _P, _P, _S, _P, _P]),
    "qv_test_linear_w4a16": (_I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _S, _P, _P]),
    "qv_test_linear_w4a8": (_I, [_P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _S, _P, _P]),
    "qv_test_workspace_bytes": (_S, [_I, _I, _I, _I, _P]),
    "qv_test_read_stream": (_I, [_P, _S, _I, _I, _I, _I, _P, _P]),
}

# QV_TUNE_* keys of include/qv_test.h, in order.
TUNE_KEYS = ("W8A8_WAVES", "W8A8_SPLITS", "W8A8_RING", "W8A8_NT", "W8A8_RINGP", "W4A16_CFG",
             "W4A16_SPLITS", "W4A8_NT", "W4A8_WAVES", "W4A8_SPLITS", "W4A8_LDS_KB", "W4A8_CG",
             "W4A8_STAGED", "QUANT_SEGS", "PREP_W8_THREADS", "W4A16_REDUCE",
             "W4A8_REDUCE")


def tune_array(tune: dict | None):
    """A ctypes int32[QV_TUNE_COUNT] from {key: value} (keys as in TUNE_KEYS), or None."""
    if not tune:
        return None
    arr = (ctypes.c_int32 * len(TUNE_KEYS))()
    for key, val in tune.items():
        arr[TUNE_KEYS.index(key)] = int(val)
    return arr

_lib = None


class QVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().qv_status_str(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn: str, status: int) -> None:
    if status != QV_OK:
        raise QVError(fn, status)
