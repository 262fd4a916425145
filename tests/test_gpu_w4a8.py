"""GPU parity: W4A8 linear (qv_linear_w4a8) against the oracle.

Bar: max |y - y_oracle| / max |y_oracle| <= 2e-3 per output tensor (the oracle adds exact
group terms in double and rounds once; the kernel's group terms are exact int32, scaled and
summed in fp32).  Repeated calls are bitwise identical (fixed-order reductions).  Inputs:
the oracle's own quant_act codes of seeded fp16 activations, and W4A16-format weights.
"""
import numpy as np
import pytest

import oracle
from quantized_weight_verification_amd import ops, synth
from _util import assert_all_written, assert_bits_equal, check_fp, dev, host, max_abs_rel, sentinel

pytestmark = pytest.mark.gpu

TOL = 2e-3
LLAMA = synth.LLAMA3_70B_LINEARS


def _inputs(seed, layer, lid, M, N, K):
    x = synth.activations(seed, layer, lid, M, K)
    xq, sx = oracle.quant_act(x)
    qw, sc, z = synth.w4a16_weights(seed, layer, lid, N, K)
    return xq, sx, qw, sc, z


def _gpu(xq, sx, qw, sc, z, tune=None):
    y = sentinel((xq.shape[0], qw.shape[0]), "f16")
    ops.linear_w4a8(dev(xq), dev(sx), dev(qw), dev(sc), dev(z), out=y, tune=tune)
    return host(y)


@pytest.mark.parametrize("M,N,K", [
    (1, 16, 128),       # one tile, one group
    (5, 48, 384),       # three tiles, odd group count
    (16, 256, 1024),
    (17, 272, 640),     # two token tiles, ragged tile groups (17 tiles: one per workgroup)
    (48, 512, 1024),    # tree-sized batch
    (64, 128, 256),     # maximum M
    (33, 144, 1152),    # three token tiles, 9 groups
    (8, 1024, 28672),   # long K (224 groups): split-K with a short last slice
    (3, 32, 128 * 27),  # 27 groups over 16 waves: waves with one and two groups
])
def test_small_and_ragged(gpu_lib, M, N, K):
    xq, sx, qw, sc, z = _inputs(40, M, N, M, N, K)
    y = _gpu(xq, sx, qw, sc, z)
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    check_fp(y, r, TOL)


@pytest.mark.parametrize("name", list(LLAMA))
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5])
def test_llama3_70b_layer0(gpu_lib, name, M):
    """Sequence verify on the 70B-shaped layer 0, every linear, all outputs (2..4 tokens take
    one-tile workgroups on the linears of at most 128 groups, as at one token)."""
    K, N = LLAMA[name]
    lid = synth.LINEAR_IDS[name]
    xq, sx, qw, sc, z = _inputs(5, 0, lid, M, N, K)
    y = _gpu(xq, sx, qw, sc, z)
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    check_fp(y, r, TOL)


@pytest.mark.parametrize("name", list(LLAMA))
@pytest.mark.parametrize("M", [16, 24, 48, 64])
def test_llama3_70b_tree_sampled(gpu_lib, name, M):
    """Tree-sized batches at full 70B shapes; the oracle computes 512 sampled channels."""
    K, N = LLAMA[name]
    lid = synth.LINEAR_IDS[name]
    xq, sx, qw, sc, z = _inputs(6, 79, lid, M, N, K)
    y = _gpu(xq, sx, qw, sc, z)
    cols = np.sort(np.random.default_rng(M * 10 + lid).choice(N, size=512, replace=False))
    r = oracle.linear_w4a8(xq, sx, qw[cols], sc[cols], z[cols])
    check_fp(y[:, cols], r, TOL)
    assert_all_written(y)


def test_code_equals_zero_gives_zero(gpu_lib):
    """q = z everywhere: each group's corrected product is exactly 0, so y = 0 exactly."""
    M, N, K = 5, 64, 512
    xq, sx, _, _, _ = _inputs(41, 0, 0, M, N, K)
    z = np.full((N, K // 128), 9, np.uint8)
    qw = np.full((N, K // 8), 0x99999999, np.uint32)
    sc = np.full((N, K // 128), 0.01, np.float16)
    y = _gpu(xq, sx, qw, sc, z)
    assert np.all(y.view(np.uint16) & 0x7FFF == 0)


def test_golden_two_groups(gpu_lib):
    """x_q = 1 everywhere with x_scale 1; codes 0..15 repeating (eight runs per group):
    group 0 (scale 0.5, zero 8) gives 8 * (120 - 128) * 0.5 = -32 and group 1 (scale 0.25,
    zero 0) 8 * 120 * 0.25 = 240, so y = 208."""
    xq = np.ones((1, 256), np.int8)
    sx = np.ones((1,), np.float32)
    words = np.tile(np.array([0x76543210, 0xFEDCBA98], np.uint32), 16)
    qw = np.tile(words, (16, 1))
    sc = np.tile(np.array([0.5, 0.25], np.float16), (16, 1))
    z = np.tile(np.array([8, 0], np.uint8), (16, 1))
    assert np.all(oracle.linear_w4a8(xq, sx, qw, sc, z) == np.float16(208.0))
    y = _gpu(xq, sx, qw, sc, z)
    assert np.all(y == np.float16(208.0))


def test_extreme_codes_and_activations(gpu_lib):
    """x_q = +-127 and codes 0 / 15 with zero points 0 / 15: the largest group sums
    (|acc_g| = 128 * 127 * 15) stay exact through the zero-point correction."""
    M, N, K = 4, 32, 1024
    g = np.random.default_rng(42)
    xq = np.where(g.random((M, K)) < 0.5, -127, 127).astype(np.int8)
    sx = np.full((M,), 1e-2, np.float32)
    codes = np.where(g.random((N, K)) < 0.5, 0, 15).astype(np.uint32)
    qw = np.bitwise_or.reduce(codes.reshape(N, K // 8, 8) << (4 * np.arange(8, dtype=np.uint32)),
                              axis=2).astype(np.uint32)
    z = np.where(g.random((N, K // 128)) < 0.5, 0, 15).astype(np.uint8)
    sc = np.full((N, K // 128), 1e-3, np.float16)
    y = _gpu(xq, sx, qw, sc, z)
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    check_fp(y, r, TOL)


def test_repeat_is_bitwise_identical(gpu_lib):
    M, N, K = 48, 8192, 8192
    xq, sx, qw, sc, z = _inputs(43, 0, 0, M, N, K)
    args = (dev(xq), dev(sx), dev(qw), dev(sc), dev(z))
    y1 = host(ops.linear_w4a8(*args))
    y2 = host(ops.linear_w4a8(*args))
    assert_bits_equal(y1, y2, "rerun")


@pytest.mark.parametrize("nt,waves,splits", [(1, 4, 1), (1, 8, 1), (1, 16, 1), (1, 4, 3), (1, 16, 5),
                                             (1, 8, 64), (2, 4, 1), (2, 4, 4), (4, 2, 1), (4, 2, 3),
                                             (4, 4, 1), (4, 4, 7)])
@pytest.mark.parametrize("M,N,K", [(1, 272, 1152), (5, 512, 2048), (16, 144, 3072), (33, 256, 1536)])
def test_every_kernel_configuration(gpu_lib, nt, waves, splits, M, N, K):
    """Each (tiles per workgroup, waves per tile) instantiation, with and without split-K
    (the planner caps the split count so that every wave keeps at least one group, and
    halves the tiles per workgroup until they divide the tile count)."""
    xq, sx, qw, sc, z = _inputs(44, M, N, M, N, K)
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    # the staged-slice kernel also at M > 16
    tune = {"W4A8_STAGED": 1, "W4A8_NT": nt, "W4A8_WAVES": waves, "W4A8_SPLITS": splits}
    check_fp(_gpu(xq, sx, qw, sc, z, tune), r, TOL)


def test_quant_act_then_w4a8(gpu_lib):
    """The W4A8 verify path end to end on the device: quant_act, then the linear."""
    M, K, N = 8, 8192, 10240
    x = synth.activations(45, 0, 0, M, K)
    qw, sc, z = synth.w4a16_weights(45, 0, 0, N, K)
    xq_d, sx_d = ops.quant_act(dev(x))
    y = host(ops.linear_w4a8(xq_d, sx_d, dev(qw), dev(sc), dev(z)))
    xq, sx = oracle.quant_act(x)
    assert_bits_equal(host(xq_d), xq, "x_q")
    assert max_abs_rel(y, oracle.linear_w4a8(xq, sx, qw, sc, z)) <= TOL


@pytest.mark.parametrize("nt,cg,splits", [(8, 4, 1), (8, 8, 1), (8, 4, 3), (8, 8, 2), (16, 4, 1),
                                          (16, 8, 5)])
@pytest.mark.parametrize("M,N,K", [(17, 256, 1536), (48, 512, 128 * 27), (64, 256, 2048),
                                   (33, 128, 128 * 5)])
def test_chunked_configurations(gpu_lib, nt, cg, splits, M, N, K):
    """The chunked kernel of tree-sized batches: 8 or 16 tiles per workgroup, chunks of 4 or
    8 groups (with a partial last chunk), with and without split-K."""
    xq, sx, qw, sc, z = _inputs(46, M, N, M, N, K)
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    check_fp(_gpu(xq, sx, qw, sc, z, {"W4A8_NT": nt, "W4A8_CG": cg, "W4A8_SPLITS": splits}), r, TOL)


@pytest.mark.parametrize("cg,splits", [(4, 1), (8, 1), (4, 3), (8, 2)])
@pytest.mark.parametrize("M,N,K", [(17, 896, 1536), (48, 1792, 128 * 27), (64, 896, 2048),
                                   (33, 896, 128 * 5)])
def test_chunked_fourteen_tiles(gpu_lib, cg, splits, M, N, K):
    """Workgroups of 14 tiles (the plan for gate_up-sized linears up to 48 tokens, so that they
    fill every CU), with partial last chunks and split-K."""
    xq, sx, qw, sc, z = _inputs(44, M, N, M, N, K)
    y = _gpu(xq, sx, qw, sc, z, {"W4A8_NT": 14, "W4A8_CG": cg, "W4A8_SPLITS": splits})
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    check_fp(y, r, TOL)


@pytest.mark.parametrize("cg,splits", [(4, 1), (8, 1), (4, 4), (8, 2)])
@pytest.mark.parametrize("M,N,K", [(17, 640, 1536), (48, 1280, 128 * 27), (64, 640, 2048),
                                   (33, 1280, 128 * 5)])
def test_chunked_ten_tiles(gpu_lib, cg, splits, M, N, K):
    """Workgroups of 10 tiles (the plan for qkv-sized linears, 640 tiles: 64 workgroups x 4
    splits fill the 256 CUs), with partial last chunks and split-K."""
    xq, sx, qw, sc, z = _inputs(48, M, N, M, N, K)
    y = _gpu(xq, sx, qw, sc, z, {"W4A8_NT": 10, "W4A8_CG": cg, "W4A8_SPLITS": splits})
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    check_fp(y, r, TOL)


@pytest.mark.parametrize("nt,cg,splits", [(8, 4, 3), (16, 8, 5), (16, 4, 2)])
@pytest.mark.parametrize("M,N,K", [(17, 256, 1536), (48, 512, 128 * 27), (64, 256, 2048)])
def test_split_reduce_launch_matches_in_kernel_finish(gpu_lib, nt, cg, splits, M, N, K):
    """The chunked kernel's split-K finish as its own launch (the default) adds the same fp32
    partials in the same order and scales them by the same per-token factor as the last
    workgroup of each tile block does: bit-identical outputs, within the bar of the oracle."""
    xq, sx, qw, sc, z = _inputs(47, M, N, M, N, K)
    r = oracle.linear_w4a8(xq, sx, qw, sc, z)
    base = {"W4A8_NT": nt, "W4A8_CG": cg, "W4A8_SPLITS": splits}
    y1 = _gpu(xq, sx, qw, sc, z, dict(base, W4A8_REDUCE=1))
    y2 = _gpu(xq, sx, qw, sc, z, dict(base, W4A8_REDUCE=2))
    check_fp(y2, r, TOL)
    assert_bits_equal(y2, y1, "reduce launch vs in-kernel finish")
