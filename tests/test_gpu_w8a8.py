"""GPU parity: W8A8 linear (qv_linear_w8a8) against the oracle.

Bar: int32 accumulators bit-exact; fp16 outputs bit-exact as well, since both sides apply
y = fp16(f32(f32(acc) * s_x) * s_w) in the same order with round-to-nearest-even (Quasar,
Sec. 3.3 "INT8 Gemm and Dequantization"), which is stricter than the 2e-3 fp bar.
"""
import numpy as np
import pytest

import oracle
from quantized_weight_verification_amd import _binding as B, ops, synth
from _util import assert_bits_equal, dev, host, sentinel

pytestmark = pytest.mark.gpu

QWEN = synth.QWEN3_8B_LINEARS


def _run(xq, sx, w, sw, tune=None):
    """The GPU call with outputs pre-filled with sentinels (an unwritten element fails)."""
    M, N = xq.shape[0], w.shape[0]
    y, acc = sentinel((M, N), "f16"), sentinel((M, N), "i32")
    ops.linear_w8a8(dev(xq), dev(sx), dev(w), dev(sw), out=y, acc_out=acc, tune=tune)
    return host(y), host(acc)


def _check(x, w, sw, tune=None):
    xq, sx = oracle.quant_act(x)
    y_o, acc_o = oracle.linear_w8a8(xq, sx, w, sw)
    y, acc = _run(xq, sx, w, sw, tune)
    assert_bits_equal(acc, acc_o, "acc")
    assert_bits_equal(y, y_o, "y")


def test_tiny_verify_linear(gpu_lib):
    """M = 4 (3 drafts + 1), K = 256, N = 512: every output."""
    x = synth.activations(1, 0, 0, 4, 256)
    w, sw = synth.w8a8_weights(1, 0, 0, 512, 256)
    _check(x, w, sw)


@pytest.mark.parametrize("name", list(QWEN))
@pytest.mark.parametrize("M", [1, 4, 6, 8, 10])
def test_qwen3_8b_layer(gpu_lib, name, M):
    """One Qwen3-8B-shaped layer, every linear and every gamma: all outputs."""
    K, N = QWEN[name]
    lid = synth.LINEAR_IDS[name]
    x = synth.activations(2, 0, lid, M, K)
    w, sw = synth.w8a8_weights(2, 0, lid, N, K)
    _check(x, w, sw)


@pytest.mark.parametrize("layer", [0, 35])
@pytest.mark.parametrize("name", list(QWEN))
def test_qwen3_8b_verify_step_layers(gpu_lib, layer, name):
    """The timed step's workload (M = 8, gamma = 7): the first and the last of its 36 layers,
    each linear with that layer's own seeded input and weights (quant_act on the device, as in
    the step): every quantised code, scale, accumulator and output bit-exact."""
    K, N = QWEN[name]
    lid = synth.LINEAR_IDS[name]
    x = synth.activations(5, layer, lid, 8, K)
    w, sw = synth.w8a8_weights(5, layer, lid, N, K)
    xq_o, sx_o = oracle.quant_act(x)
    y_o, acc_o = oracle.linear_w8a8(xq_o, sx_o, w, sw)
    xq, sx = ops.quant_act(dev(x))
    assert_bits_equal(host(xq), xq_o, "x_q")
    assert_bits_equal(host(sx), sx_o, "x_scale")
    y, acc = sentinel((8, N), "f16"), sentinel((8, N), "i32")
    ops.linear_w8a8(xq, sx, dev(w), dev(sw), out=y, acc_out=acc)
    assert_bits_equal(host(acc), acc_o, "acc")
    assert_bits_equal(host(y), y_o, "y")


@pytest.mark.parametrize("M,N,K", [
    (1, 16, 64),        # one tile, one K step
    (15, 48, 192),      # K steps not a multiple of the unroll
    (16, 64, 4096 + 64),
    (17, 32, 640),      # two token tiles
    (33, 80, 1088),     # three token tiles, ragged
    (64, 16, 128),      # maximum M
    (5, 512, 12288),    # few tiles, long K: split-K path
    (7, 16, 64 * 333),  # one tile, odd step count, many splits
])
def test_ragged_shapes(gpu_lib, M, N, K):
    x = synth.activations(9, M, N, M, K)
    w, sw = synth.w8a8_weights(9, M, N, N, K)
    _check(x, w, sw)


def test_split_k_counters_rearm(gpu_lib):
    """Two split-K calls in a row on one workspace give identical results."""
    M, N, K = 8, 256, 8192
    assert ops.workspace_bytes(B.QV_OP_W8A8, M, N, K) > 0, "shape should take the split path"
    x = synth.activations(10, 0, 0, M, K)
    w, sw = synth.w8a8_weights(10, 0, 0, N, K)
    xq, sx = oracle.quant_act(x)
    y1, a1 = _run(xq, sx, w, sw)
    y2, a2 = _run(xq, sx, w, sw)
    assert_bits_equal(a1, a2, "acc rerun")
    assert_bits_equal(y1, y2, "y rerun")
    y_o, acc_o = oracle.linear_w8a8(xq, sx, w, sw)
    assert_bits_equal(a2, acc_o, "acc")


def test_int32_bound_at_max_k(gpu_lib):
    """|acc| reaches 128 * 128 * K (every code -128) at the largest K the ABI accepts: still
    exact int32."""
    M, N, K = 2, 16, B.QV_W8A8_MAX_K
    xq = np.full((M, K), -128, np.int8)
    xq[1] = 127
    sx = np.array([1.0, 0.5], np.float32)
    w = np.full((N, K), -128, np.int8)
    w[1::2] = 127
    sw = np.full(N, 1e-9, np.float32)
    y_o, acc_o = oracle.linear_w8a8(xq, sx, w, sw)
    assert int(acc_o[0, 0]) == 128 * 128 * K < 2 ** 31
    y, acc = _run(xq, sx, w, sw)
    assert_bits_equal(acc, acc_o, "acc")
    assert_bits_equal(y, y_o, "y")


def test_without_acc_out(gpu_lib):
    x = synth.activations(11, 0, 0, 6, 4096)
    w, sw = synth.w8a8_weights(11, 0, 0, 1024, 4096)
    xq, sx = oracle.quant_act(x)
    y = sentinel((6, 1024), "f16")
    ops.linear_w8a8(dev(xq), dev(sx), dev(w), dev(sw), out=y)
    y_o, _ = oracle.linear_w8a8(xq, sx, w, sw)
    assert_bits_equal(host(y), y_o, "y")


def test_golden_tiny(gpu_lib):
    """The worked example: acc = [[6, 0], [126, -2]], y = [[0.375, 0], [3.9375, -1]]; the
    shapes are padded to the ABI's K % 64 and N % 16 rules with zeros."""
    xq = np.zeros((2, 64), np.int8)
    xq[:, :3] = [[1, 2, 3], [-1, 0, 127]]
    w = np.zeros((16, 64), np.int8)
    w[:2, :3] = [[1, 1, 1], [2, -1, 0]]
    sx = np.array([0.5, 0.25], np.float32)
    sw = np.full(16, 1.0, np.float32)
    sw[:2] = [0.125, 2.0]
    y, acc = _run(xq, sx, w, sw)
    assert acc[:, :2].tolist() == [[6, 0], [126, -2]]
    assert y[:, :2].astype(np.float32).tolist() == [[0.375, 0.0], [3.9375, -1.0]]


@pytest.mark.parametrize("kernel", ["direct", "ring1", "ring2", "ring4"])
@pytest.mark.parametrize("waves", [2, 4, 8, 16])
@pytest.mark.parametrize("M,N,K,splits", [(8, 4096, 4096, 0), (10, 256, 12288, 3), (33, 48, 640, 0),
                                          (1, 32, 64 * 37, 2), (20, 160, 64 * 70, 2)])
def test_every_kernel_configuration(gpu_lib, kernel, waves, M, N, K, splits):
    """Both W8A8 kernels (activations from L2, or staged in LDS with a weight ring shared by
    1, 2 or 4 output tiles per workgroup) at 2 (ring only), 4, 8 and 16 waves per tile, with
    and without split-K: bit-exact against the oracle.  Tile counts that the tiles per
    workgroup do not divide fall back to fewer tiles per workgroup."""
    x = synth.activations(12, M, N, M, K)
    w, sw = synth.w8a8_weights(12, M, N, N, K)
    direct = kernel == "direct"
    tune = {"W8A8_RING": 2 if direct else 1, "W8A8_WAVES": waves, "W8A8_SPLITS": splits,
            "W8A8_NT": 1 if direct else int(kernel[4:])}
    _check(x, w, sw, tune)


@pytest.mark.parametrize("waves", [2, 4, 16])
@pytest.mark.parametrize("nt", [1, 2, 4])
@pytest.mark.parametrize("ringp", [8, 12, 16])
@pytest.mark.parametrize("M,N,K", [(8, 4096, 4096), (2, 128, 64 * 45), (16, 64, 12288)])
def test_ring_depths(gpu_lib, waves, nt, ringp, M, N, K):
    """The weight ring at 8, 12 and 16 K-steps in flight, for 2-, 4- and 16-wave tiles shared
    1, 2 or 4 to a workgroup (the step counts per wave include ones that are not a multiple of
    the ring): bit-exact against the oracle."""
    x = synth.activations(13, M, N, M, K)
    w, sw = synth.w8a8_weights(13, M, N, N, K)
    _check(x, w, sw, {"W8A8_RING": 1, "W8A8_WAVES": waves, "W8A8_NT": nt, "W8A8_RINGP": ringp})


@pytest.mark.parametrize("M,N,K", [(8, 16400, 4096), (1, 16400, 1024), (3, 16432, 640)])
def test_default_plan_odd_tile_count(gpu_lib, M, N, K):
    """Default plans with an odd number (>= 1024) of 16-channel tiles: the LDS-staged ring
    with 2-wave tiles must fall back to one tile per workgroup and still write every output
    (the sentinel-filled outputs fail on a dropped tile)."""
    x = synth.activations(14, M, N, M, K)
    w, sw = synth.w8a8_weights(14, M, N, N, K)
    _check(x, w, sw)
