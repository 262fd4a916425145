"""GPU parity: offline weight preparation (qv_prepare_w8, qv_prepare_w4) against the oracle.

Bar: bit-exact codes, fp32 / fp16 scales and zero points (both sides take every rounding in
fp32 with correctly rounded divisions and round-half-to-even).  Rows are independent, so
full-size matrices are checked on sampled rows.
"""
import numpy as np
import pytest

from oracle import prep
from quantized_weight_verification_amd import ops, synth
from _util import assert_bits_equal, dev, host, max_abs_rel

pytestmark = pytest.mark.gpu


def bf16_rows(seed, N, K, scale=0.02):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((N, K)) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _w8(wb, inv=None, tune=None):
    q, s = ops.prepare_w8(dev(wb.view(np.int16)), dev(inv) if inv is not None else None, tune=tune)
    return host(q), host(s)


def _w4(wb):
    qw, sc, z = ops.prepare_w4(dev(wb.view(np.int16)))
    return host(qw).view(np.uint32), host(sc), host(z)


@pytest.mark.parametrize("N,K,smooth", [(1, 8, False), (3, 40, True), (17, 4096, False),
                                        (64, 4096, True), (5, 12288, True), (2, 28672, False),
                                        (4, 40000, True)])
def test_w8_random(gpu_lib, N, K, smooth):
    wb = bf16_rows(N * 7 + K, N, K)
    inv = np.random.default_rng(K).uniform(0.25, 4.0, K).astype(np.float32) if smooth else None
    q, s = _w8(wb, inv)
    q_o, s_o = prep.prepare_w8(wb, inv)
    assert_bits_equal(q, q_o, "w_q")
    assert_bits_equal(s, s_o, "w_scale")


@pytest.mark.parametrize("threads", [128, 256, 512])
@pytest.mark.parametrize("N,K", [(17, 4096), (5, 12288), (4, 40000)])
def test_w8_every_workgroup_size(gpu_lib, threads, N, K):
    """Each workgroup size of the W8 preparation (registers or two passes) gives the
    oracle's codes and scales bit for bit."""
    wb = bf16_rows(N * 11 + K, N, K)
    inv = np.random.default_rng(K + 1).uniform(0.25, 4.0, K).astype(np.float32)
    q, s = _w8(wb, inv, {"PREP_W8_THREADS": threads})
    q_o, s_o = prep.prepare_w8(wb, inv)
    assert_bits_equal(q, q_o, "codes")
    assert_bits_equal(s, s_o, "scales")


def test_w8_zero_row_ties_and_extremes(gpu_lib):
    N, K = 4, 1024
    w = np.zeros((N, K), np.float32)
    w[1, :] = np.arange(K, dtype=np.float32) / 8 - 64        # many w / scale ties at .5
    w[2, :] = -1.0
    w[2, 7] = 3.0
    w[3, :] = 2.0 ** -120                                       # tiny: scale is subnormal
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    q, s = _w8(wb)
    q_o, s_o = prep.prepare_w8(wb)
    assert_bits_equal(q, q_o, "w_q")
    assert_bits_equal(s, s_o, "w_scale")
    assert s[0] == 0 and not q[0].any()


def test_w8_lm_head_sampled(gpu_lib):
    """Qwen3-8B LM head shape (151936 x 4096) with smoothing multipliers; 512 sampled rows."""
    N, K = synth.QWEN3_8B_VOCAB, 4096
    wb = bf16_rows(3, N, K)
    inv = np.random.default_rng(4).uniform(0.5, 2.0, K).astype(np.float32)
    q, s = _w8(wb, inv)
    rows = np.sort(np.random.default_rng(5).choice(N, 512, replace=False))
    q_o, s_o = prep.prepare_w8(wb[rows], inv)
    assert_bits_equal(q[rows], q_o, "w_q")
    assert_bits_equal(s[rows], s_o, "w_scale")


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (16, 8192), (129, 1024), (7, 28672)])
def test_w4_random(gpu_lib, N, K):
    wb = bf16_rows(N * 11 + K, N, K)
    qw, sc, z = _w4(wb)
    qw_o, sc_o, z_o = prep.prepare_w4(wb)
    assert_bits_equal(qw, qw_o, "qweight")
    assert_bits_equal(sc, sc_o, "scales")
    assert_bits_equal(z, z_o, "zeros")


def test_w4_special_groups(gpu_lib):
    K = 128 * 6
    w = np.zeros((2, K), np.float32)
    w[0, 128:256] = 0.5                       # constant positive
    w[0, 256:384] = -0.25                     # constant negative
    w[0, 384:512] = np.linspace(-1, 3, 128)   # asymmetric range
    w[0, 512:640] = 2.0 ** -30                # scale underflows to 0 in fp16 -> 1
    w[1, :] = np.random.default_rng(6).standard_normal(K)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    qw, sc, z = _w4(wb)
    qw_o, sc_o, z_o = prep.prepare_w4(wb)
    assert_bits_equal(qw, qw_o, "qweight")
    assert_bits_equal(sc, sc_o, "scales")
    assert_bits_equal(z, z_o, "zeros")


def test_w4_llama_gate_up_sampled(gpu_lib):
    K, N = synth.LLAMA3_70B_LINEARS["gate_up"]
    wb = bf16_rows(7, N, K)
    qw, sc, z = _w4(wb)
    rows = np.sort(np.random.default_rng(8).choice(N, 256, replace=False))
    qw_o, sc_o, z_o = prep.prepare_w4(wb[rows])
    assert_bits_equal(qw[rows], qw_o, "qweight")
    assert_bits_equal(sc[rows], sc_o, "scales")
    assert_bits_equal(z[rows], z_o, "zeros")


def test_prepared_weights_feed_the_linears(gpu_lib):
    """prepare_w8 -> linear_w8a8 and prepare_w4 -> linear_w4a16 / linear_w4a8 on the device,
    against the oracle linears on the oracle-prepared weights."""
    import oracle

    M, K, N = 8, 4096, 1024
    wb = bf16_rows(9, N, K)
    x = synth.activations(9, 0, 0, M, K)
    xq, sx = oracle.quant_act(x)
    wq, ws = ops.prepare_w8(dev(wb.view(np.int16)))
    y8 = host(ops.linear_w8a8(dev(xq), dev(sx), wq, ws))
    wq_o, ws_o = prep.prepare_w8(wb)
    assert_bits_equal(y8, oracle.linear_w8a8(xq, sx, wq_o, ws_o)[0], "w8a8 on prepared weights")
    qw, sc, z = ops.prepare_w4(dev(wb.view(np.int16)))
    qw_o, sc_o, z_o = prep.prepare_w4(wb)
    y16 = host(ops.linear_w4a16(dev(x), qw, sc, z))
    assert max_abs_rel(y16, oracle.linear_w4a16(x, qw_o, sc_o, z_o)) <= 2e-3
    y4 = host(ops.linear_w4a8(dev(xq), dev(sx), qw, sc, z))
    assert max_abs_rel(y4, oracle.linear_w4a8(xq, sx, qw_o, sc_o, z_o)) <= 2e-3
