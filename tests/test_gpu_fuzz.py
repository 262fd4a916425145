"""Fuzzed-shape GPU parity: hypothesis draws shapes (and input seeds) across the shape rules of
each call, so that the planners' branches are reached by routes a hand-picked matrix misses
(ragged channel blocks, odd token counts, K ranges that split unevenly, the W8A8 fall-back to
the direct kernel when the LDS-staged ring would overflow).  Each example is compared with the
oracle to the call's own bar: bit-exact for integer results and the W8A8 fp16 epilogue, within
2e-3 max-abs-rel for the W4A16/W4A8 fp16 outputs.  Examples are derandomised (the same shapes on
every run) and bounded in number and size so the file runs in seconds."""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from quantized_weight_verification_amd import ops, synth
from _util import assert_bits_equal, check_fp, dev, host, sentinel

pytestmark = pytest.mark.gpu

TOL = 2e-3
FUZZ = settings(max_examples=25, deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])

m_st = st.integers(1, 64)
seed_st = st.integers(0, 2 ** 16)


@FUZZ
@given(M=m_st, k8=st.integers(1, 1536), seed=seed_st)
def test_fuzz_quant_act(gpu_lib, M, k8, seed):
    K = 8 * k8
    x = synth.activations(40, seed, 0, M, K)
    q_o, s_o = oracle.quant_act(x)
    q, s = ops.quant_act(dev(x))
    assert_bits_equal(host(q), q_o, "x_q")
    assert_bits_equal(host(s), s_o, "x_scale")


@FUZZ
@given(M=m_st, n16=st.integers(1, 160), k64=st.integers(1, 96), seed=seed_st)
def test_fuzz_w8a8(gpu_lib, M, n16, k64, seed):
    N, K = 16 * n16, 64 * k64
    x = synth.activations(41, seed, 0, M, K)
    w, sw = synth.w8a8_weights(41, seed, 0, N, K)
    xq, sx = oracle.quant_act(x)
    y_o, acc_o = oracle.linear_w8a8(xq, sx, w, sw)
    y, acc = sentinel((M, N), "f16"), sentinel((M, N), "i32")
    ops.linear_w8a8(dev(xq), dev(sx), dev(w), dev(sw), out=y, acc_out=acc)
    assert_bits_equal(host(acc), acc_o, "acc")
    assert_bits_equal(host(y), y_o, "y")


@pytest.mark.parametrize("M,N,K", [(64, 16400, 128), (64, 24576, 256), (33, 17408, 192)])
def test_w8a8_many_tiles_at_large_m(gpu_lib, M, N, K):
    """Over 1024 channel tiles at M > 32: the planner's LDS budget for the staged ring is
    exceeded and the direct kernel runs; every output bit-exact."""
    x = synth.activations(42, M, N, M, K)
    w, sw = synth.w8a8_weights(42, M, N, N, K)
    xq, sx = oracle.quant_act(x)
    y_o, acc_o = oracle.linear_w8a8(xq, sx, w, sw)
    y, acc = sentinel((M, N), "f16"), sentinel((M, N), "i32")
    ops.linear_w8a8(dev(xq), dev(sx), dev(w), dev(sw), out=y, acc_out=acc)
    assert_bits_equal(host(acc), acc_o, "acc")
    assert_bits_equal(host(y), y_o, "y")


@FUZZ
@given(M=m_st, n16=st.integers(1, 96), kg=st.integers(1, 48), seed=seed_st)
def test_fuzz_w4a16(gpu_lib, M, n16, kg, seed):
    N, K = 16 * n16, 128 * kg
    x = synth.activations(43, seed, 0, M, K)
    qw, sc, z = synth.w4a16_weights(43, seed, 0, N, K)
    r = oracle.linear_w4a16(x, qw, sc, z)
    y = sentinel((M, N), "f16")
    ops.linear_w4a16(dev(x), dev(qw), dev(sc), dev(z), out=y)
    check_fp(host(y), r, TOL)


@FUZZ
@given(M=m_st, n16=st.integers(1, 96), kg=st.integers(1, 48), seed=seed_st)
def test_fuzz_w4a8(gpu_lib, M, n16, kg, seed):
    N, K = 16 * n16, 128 * kg
    x = synth.activations(44, seed, 0, M, K)
    qw, sc, z = synth.w4a16_weights(44, seed, 0, N, K)
    xq, sx = oracle.quant_act(x)
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    y = sentinel((M, N), "f16")
    ops.linear_w4a8(dev(xq), dev(sx), dev(qw), dev(sc), dev(z), out=y)
    check_fp(host(y), r, TOL)


@FUZZ
@given(M=m_st, V=st.integers(1, 300000), seed=seed_st, keep=st.integers(0, 64))
def test_fuzz_verify_greedy(gpu_lib, M, V, seed, keep):
    """Drafts copy the oracle's argmax for `keep` positions, then miss once (when V > 1), then
    are uniform: every accept length from 0 to M - 1 is reachable."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((M, V)).astype(np.float16)
    am = oracle.argmax(logits)
    draft = rng.integers(0, V, size=max(M - 1, 0)).astype(np.int32)
    draft[:keep] = am[:M - 1][:keep]
    if keep < M - 1 and V > 1:
        draft[keep] = (am[keep] + 1) % V
    a_o, n_o = oracle.verify_greedy(logits, draft)
    a, n = ops.verify_greedy(dev(logits), dev(draft) if M > 1 else None)
    assert_bits_equal(host(a), np.asarray(a_o, np.int32), "argmax")
    assert int(host(n)[0]) == int(n_o)
