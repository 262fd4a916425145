"""The C ABI on the host, without a GPU: the library loads, exports every function
include/qv.h and include/qv_test.h declare, and rejects bad arguments with the documented
status codes before any HIP call (the pointers below are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from quantized_weight_verification_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qv.h")
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

# Fake, well-aligned device addresses: every call below fails validation first.
A = 0x7F0000000000
A2 = A + 0x100000
MISALIGNED = A + 2


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(qv_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libqv.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ("qv_quant_act", "qv_linear_w8a8", "qv_linear_w4a16", "qv_verify_greedy",
              "qv_workspace_bytes", "qv_status_str"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qv_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    assert set(declared_functions()) == set(B.SIGNATURES), "binding and header disagree"


def test_no_process_state_in_the_public_abi(lib):
    """The calls of qv.h hold no tunable state: there is no setter, qv.h declares no
    qv_test_* call, and a tuned workspace query leaves the public plan unchanged."""
    public = declared_functions([HEADER])
    assert "qv_set_tuning" not in declared_functions()
    assert not [f for f in public if f.startswith("qv_test_")]
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert "qv_set_tuning" not in out
    before = lib.qv_workspace_bytes(B.QV_OP_W4A16, 5, 8192, 8192)
    tuned = lib.qv_test_workspace_bytes(B.QV_OP_W4A16, 5, 8192, 8192,
                                        B.tune_array({"W4A16_CFG": 13, "W4A16_SPLITS": 7}))
    assert tuned != before
    assert lib.qv_workspace_bytes(B.QV_OP_W4A16, 5, 8192, 8192) == before
    assert lib.qv_test_workspace_bytes(B.QV_OP_W4A16, 5, 8192, 8192, None) == before


def test_noalloc_verify_errors(lib):
    """qv_verify_greedy_noalloc rejects bad arguments, and shapes beyond its static scratch,
    before any HIP call."""
    f = lib.qv_verify_greedy_noalloc
    assert f(None, 4, 1000, A, A2, A2, None) == B.QV_ERR_NULL
    assert f(A, 4, 1000, None, A2, A2, None) == B.QV_ERR_NULL
    assert f(A, 0, 1000, A, A2, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 65, 1000, A, A2, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 4, 0, A, A2, A2, None) == B.QV_ERR_SHAPE
    # 64 rows of 2^24 logits need 64 * 1024 chunk keys: more than the static scratch holds.
    assert f(A, 64, 1 << 24, A, A2, A2, None) == B.QV_ERR_SCRATCH
    assert f(MISALIGNED, 4, 1000, A, A2, A2, None) == B.QV_ERR_ALIGN
    assert lib.qv_status_str(B.QV_ERR_SCRATCH)


def test_read_stream_errors(lib):
    """The read-only bandwidth probe validates its arguments before launching anything."""
    f = lib.qv_test_read_stream
    assert f(None, 1 << 20, B.QV_READ_LINEAR, 0, 0, 64, A2, None) == B.QV_ERR_NULL
    assert f(A, 1 << 20, B.QV_READ_LINEAR, 0, 0, 64, None, None) == B.QV_ERR_NULL
    assert f(A, 1 << 20, 2, 0, 0, 64, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 0, B.QV_READ_LINEAR, 0, 0, 64, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 1000, B.QV_READ_LINEAR, 0, 0, 64, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 1 << 20, B.QV_READ_LINEAR, 0, 0, 0, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 1 << 20, B.QV_READ_LINEAR, 0, 0, B.QV_READ_MAX_BLOCKS + 1, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 1 << 20, B.QV_READ_TILES, 0, 0, 64, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 1 << 20, B.QV_READ_TILES, 96, 0, 64, A2, None) == B.QV_ERR_SHAPE
    assert f(A, 16 * 4096 * 3 + 16, B.QV_READ_TILES, 4096, 0, 64, A2, None) == B.QV_ERR_SHAPE
    assert f(MISALIGNED, 1 << 20, B.QV_READ_LINEAR, 0, 0, 64, A2, None) == B.QV_ERR_ALIGN
    assert f(A, 1 << 20, B.QV_READ_LINEAR, 0, 0, 64, A2 + 4, None) == B.QV_ERR_ALIGN


def test_tune_keys_match_the_header():
    text = open(os.path.join(ROOT, "include", "qv_test.h")).read()
    body = text[text.index("enum {"):text.rindex("QV_TUNE_COUNT")]
    keys = re.findall(r"QV_TUNE_([A-Z0-9_]+)", body)
    assert tuple(keys) == B.TUNE_KEYS


def test_status_strings(lib):
    for s in range(7):
        assert lib.qv_status_str(s)
    assert lib.qv_status_str(99) == b"unknown status"
    assert lib.qv_version() >= 100


def test_quant_act_errors(lib):
    f = lib.qv_quant_act
    assert f(None, None, 4, 256, A2, A2, None) == B.QV_ERR_NULL
    assert f(A, None, 0, 256, A2, A2, None) == B.QV_ERR_SHAPE
    assert f(A, None, 65, 256, A2, A2, None) == B.QV_ERR_SHAPE
    assert f(A, None, 4, 12, A2, A2, None) == B.QV_ERR_SHAPE
    assert f(A, None, 4, 0, A2, A2, None) == B.QV_ERR_SHAPE
    assert f(MISALIGNED, None, 4, 256, A2, A2, None) == B.QV_ERR_ALIGN
    assert f(A, A + 1, 4, 256, A2, A2, None) == B.QV_ERR_ALIGN


def test_w8a8_errors(lib):
    f = lib.qv_linear_w8a8

    def call(xq=A, sx=A, M=4, K=256, w=A, sw=A, N=512, y=A2, acc=None, ws=None, wsb=0):
        return f(xq, sx, M, K, w, sw, N, y, acc, ws, wsb, None)

    assert call(xq=None) == B.QV_ERR_NULL
    assert call(y=None) == B.QV_ERR_NULL
    assert call(M=0) == B.QV_ERR_SHAPE
    assert call(M=65) == B.QV_ERR_SHAPE
    assert call(K=96) == B.QV_ERR_SHAPE
    assert call(K=B.QV_W8A8_MAX_K + 64) == B.QV_ERR_SHAPE
    assert call(N=8) == B.QV_ERR_SHAPE
    assert call(N=520) == B.QV_ERR_SHAPE
    assert call(w=MISALIGNED) == B.QV_ERR_ALIGN
    assert call(acc=MISALIGNED) == B.QV_ERR_ALIGN
    # a shape that needs a split-K workspace
    M, N, K = 8, 256, 8192
    need = lib.qv_workspace_bytes(B.QV_OP_W8A8, M, N, K)
    assert need > B.QV_WORKSPACE_COUNTER_BYTES
    assert call(M=M, N=N, K=K) == B.QV_ERR_WORKSPACE
    assert call(M=M, N=N, K=K, ws=A, wsb=need - 1) == B.QV_ERR_WORKSPACE
    assert call(M=M, N=N, K=K, ws=A + 16, wsb=need) == B.QV_ERR_ALIGN


def test_w4a16_errors(lib):
    f = lib.qv_linear_w4a16

    def call(x=A, M=5, K=1024, qw=A, sc=A, z=A, N=256, g=128, y=A2, ws=None, wsb=0):
        return f(x, M, K, qw, sc, z, N, g, y, ws, wsb, None)

    assert call(z=None) == B.QV_ERR_NULL
    assert call(g=64) == B.QV_ERR_SHAPE
    assert call(K=1000) == B.QV_ERR_SHAPE
    assert call(K=64) == B.QV_ERR_SHAPE
    assert call(N=24) == B.QV_ERR_SHAPE
    assert call(M=65) == B.QV_ERR_SHAPE
    assert call(x=MISALIGNED) == B.QV_ERR_ALIGN
    assert call(sc=A + 1) == B.QV_ERR_ALIGN
    need = lib.qv_workspace_bytes(B.QV_OP_W4A16, 5, 256, 1024)
    if need:
        assert call() == B.QV_ERR_WORKSPACE


def test_prepare_errors(lib):
    f8, f4 = lib.qv_prepare_w8, lib.qv_prepare_w4
    assert f8(None, None, 4, 64, A, A2, None) == B.QV_ERR_NULL
    assert f8(A, None, 0, 64, A, A2, None) == B.QV_ERR_SHAPE
    assert f8(A, None, 4, 60, A, A2, None) == B.QV_ERR_SHAPE
    assert f8(A + 8, None, 4, 64, A, A2, None) == B.QV_ERR_ALIGN
    assert f8(A, A + 2, 4, 64, A, A2, None) == B.QV_ERR_ALIGN
    assert f4(A, 4, 256, 128, A, A2, None, None) == B.QV_ERR_NULL
    assert f4(A, 4, 200, 128, A, A2, A2, None) == B.QV_ERR_SHAPE
    assert f4(A, 4, 256, 64, A, A2, A2, None) == B.QV_ERR_SHAPE
    assert f4(A, 0, 256, 128, A, A2, A2, None) == B.QV_ERR_SHAPE
    assert f4(A + 2, 4, 256, 128, A, A2, A2, None) == B.QV_ERR_ALIGN
    assert f4(A, 4, 256, 128, A + 2, A2, A2, None) == B.QV_ERR_ALIGN


def test_w4a8_errors(lib):
    f = lib.qv_linear_w4a8

    def call(x=A, sx=A, M=5, K=1024, qw=A, sc=A, z=A, N=256, g=128, y=A2, ws=None, wsb=0):
        return f(x, sx, M, K, qw, sc, z, N, g, y, ws, wsb, None)

    assert call(sx=None) == B.QV_ERR_NULL
    assert call(z=None) == B.QV_ERR_NULL
    assert call(g=64) == B.QV_ERR_SHAPE
    assert call(K=1000) == B.QV_ERR_SHAPE
    assert call(N=24) == B.QV_ERR_SHAPE
    assert call(M=0) == B.QV_ERR_SHAPE
    assert call(M=65) == B.QV_ERR_SHAPE
    assert call(x=A + 8) == B.QV_ERR_ALIGN
    assert call(qw=A + 4) == B.QV_ERR_ALIGN
    assert call(sx=A + 2) == B.QV_ERR_ALIGN
    # M = 48 over a long K splits K, so the call needs partial sums in a workspace
    need = lib.qv_workspace_bytes(B.QV_OP_W4A8, 48, 8192, 28672)
    assert need >= B.QV_WORKSPACE_COUNTER_BYTES + 2 * 48 * 8192 * 4
    assert call(M=48, K=28672, N=8192) == B.QV_ERR_WORKSPACE
    assert call(M=48, K=28672, N=8192, ws=A, wsb=need - 1) == B.QV_ERR_WORKSPACE
    assert call(M=48, K=28672, N=8192, ws=A + 16, wsb=need) == B.QV_ERR_ALIGN


def test_verify_errors(lib):
    f = lib.qv_verify_greedy

    def call(lg=A, M=8, V=151936, d=A, am=A2, na=A2, ws=A, wsb=1 << 30):
        return f(lg, M, V, d, am, na, ws, wsb, None)

    assert call(d=None) == B.QV_ERR_NULL
    assert call(na=None) == B.QV_ERR_NULL
    assert call(M=0) == B.QV_ERR_SHAPE
    assert call(V=0) == B.QV_ERR_SHAPE
    assert call(lg=MISALIGNED) == B.QV_ERR_ALIGN
    assert call(wsb=100) == B.QV_ERR_WORKSPACE
    assert call(ws=None) == B.QV_ERR_WORKSPACE
    assert call(ws=A + 8) == B.QV_ERR_ALIGN


def test_verify_tree_errors(lib):
    f = lib.qv_verify_tree

    def call(lg=A, M=48, V=128256, tok=A, par=A, am=A2, path=A2, acc=A2, ws=A, wsb=1 << 30):
        return f(lg, M, V, tok, par, am, path, acc, ws, wsb, None)

    assert call(tok=None) == B.QV_ERR_NULL
    assert call(par=None) == B.QV_ERR_NULL
    assert call(acc=None) == B.QV_ERR_NULL
    assert call(M=65) == B.QV_ERR_SHAPE
    assert call(V=0) == B.QV_ERR_SHAPE
    assert call(lg=MISALIGNED) == B.QV_ERR_ALIGN
    assert call(par=A + 2) == B.QV_ERR_ALIGN
    assert call(wsb=100) == B.QV_ERR_WORKSPACE


def test_verify_sample_errors(lib):
    f = lib.qv_verify_sample

    def call(lg=A, M=8, V=151936, dl=A, dr=A, u=A, T=0.8, res=A2, ws=A, wsb=1 << 30):
        return f(lg, M, V, dl, dr, u, T, res, ws, wsb, None)

    assert call(dr=None) == B.QV_ERR_NULL
    assert call(u=None) == B.QV_ERR_NULL
    assert call(res=None) == B.QV_ERR_NULL
    assert call(M=65) == B.QV_ERR_SHAPE
    assert call(V=0) == B.QV_ERR_SHAPE
    for T in (0.0, -0.5, float("inf"), float("nan")):
        assert call(T=T) == B.QV_ERR_SHAPE
    assert call(lg=MISALIGNED) == B.QV_ERR_ALIGN
    assert call(dl=A + 8) == B.QV_ERR_ALIGN
    assert call(u=A + 4) == B.QV_ERR_ALIGN
    assert call(wsb=100) == B.QV_ERR_WORKSPACE
    assert call(ws=A + 16) == B.QV_ERR_ALIGN


def test_workspace_sizes(lib):
    ws = lib.qv_workspace_bytes
    assert ws(B.QV_OP_W8A8, 8, 24576, 4096) == 0          # enough tiles: no split
    assert ws(B.QV_OP_W8A8, 4, 512, 256) >= 0
    assert ws(B.QV_OP_W8A8, 4, 500, 256) == 0             # rejected shape
    v = ws(B.QV_OP_VERIFY, 8, 151936, 0)
    # counters, one 64-bit key per (row, 16384-logit chunk), and the rows' argmax
    assert v >= B.QV_WORKSPACE_COUNTER_BYTES + 8 * 8 * ((151936 + 16383) // 16384) + 8 * 4
    s = ws(B.QV_OP_SAMPLE, 8, 151936, 0)
    # counters, (max, sum) per (row, 4096-logit chunk) over 15 rows, the draft tokens'
    # logits, and two sums per 2048-logit chunk
    assert s >= (B.QV_WORKSPACE_COUNTER_BYTES + 15 * 16 * ((151936 + 4095) // 4096) + 15 * 8
                 + 16 * ((151936 + 2047) // 2048))
    assert ws(B.QV_OP_SAMPLE, 65, 100, 0) == 0
    assert ws(99, 1, 16, 64) == 0
