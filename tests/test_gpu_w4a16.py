"""GPU parity: W4A16 group-128 linear (qv_linear_w4a16) against the oracle.

Bar: max |y - y_oracle| / max |y_oracle| <= 2e-3 per output tensor (the oracle sums exact
products in double; the kernels accumulate in fp32, the small-M kernel with exact per-group
sums scaled in fp32, the others with each dequantised weight rounded to fp16).  Outputs are
pre-filled with NaN sentinels, so an unwritten element fails.  Repeated calls must be
bitwise identical (fixed-order split-K reduction).
"""
import numpy as np
import pytest

import oracle
from quantized_weight_verification_amd import ops, synth
from _util import assert_all_written, assert_bits_equal, check_fp, dev, host, max_abs_rel, sentinel

pytestmark = pytest.mark.gpu

TOL = 2e-3
LLAMA = synth.LLAMA3_70B_LINEARS


def _gpu(x, qw, sc, z, tune=None):
    y = sentinel((x.shape[0], qw.shape[0]), "f16")
    ops.linear_w4a16(dev(x), dev(qw), dev(sc), dev(z), out=y, tune=tune)
    return host(y)


@pytest.mark.parametrize("M,N,K", [
    (1, 16, 128),       # one tile, one group
    (5, 48, 384),       # partial tile block, odd group count
    (16, 256, 1024),
    (17, 272, 640),     # two token tiles, ragged channels
    (48, 512, 1024),    # tree-sized batch
    (64, 128, 256),     # maximum M
    (33, 144, 1152),    # three token tiles, 9 groups
    (8, 1024, 28672),   # long K (224 groups): split-K with a tail chunk
])
def test_small_and_ragged(gpu_lib, M, N, K):
    x = synth.activations(30, M, N, M, K)
    qw, sc, z = synth.w4a16_weights(30, M, N, N, K)
    y = _gpu(x, qw, sc, z)
    r = oracle.linear_w4a16(x, qw, sc, z)
    check_fp(y, r, TOL)


@pytest.mark.parametrize("name", list(LLAMA))
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5])
def test_llama3_70b_layer0(gpu_lib, name, M):
    """Sequence verify on the 70B-shaped layer 0, every linear, all outputs (each M of 1..5
    takes its own default plan)."""
    K, N = LLAMA[name]
    lid = synth.LINEAR_IDS[name]
    x = synth.activations(3, 0, lid, M, K)
    qw, sc, z = synth.w4a16_weights(3, 0, lid, N, K)
    y = _gpu(x, qw, sc, z)
    r = oracle.linear_w4a16(x, qw, sc, z)
    check_fp(y, r, TOL)


@pytest.mark.parametrize("layer", [0, 79])
@pytest.mark.parametrize("name", list(LLAMA))
@pytest.mark.parametrize("M", [1, 12, 16, 24, 48])
def test_llama3_70b_tree_sampled(gpu_lib, layer, name, M):
    """Decode (M = 1), the 9..16-token plans (M = 12, 16) and tree verify (M = 24, 48: the
    staging-wave kernel on gate_up, the chunk kernel on the others) at full 70B shapes; the
    oracle computes 512 sampled output channels one by one."""
    K, N = LLAMA[name]
    lid = synth.LINEAR_IDS[name]
    x = synth.activations(4, layer, lid, M, K)
    qw, sc, z = synth.w4a16_weights(4, layer, lid, N, K)
    y = _gpu(x, qw, sc, z)
    cols = np.sort(np.random.default_rng(layer * 10 + lid).choice(N, size=512, replace=False))
    r = oracle.linear_w4a16(x, qw[cols], sc[cols], z[cols])
    check_fp(y[:, cols], r, TOL)
    assert_all_written(y)


@pytest.mark.parametrize("M", [17, 24, 32, 33, 40, 48, 56, 64])
@pytest.mark.parametrize("N,K", [(32784, 1024), (36864, 2048)])
def test_default_plans_many_channels(gpu_lib, M, N, K):
    """Default plans past 32768 channels at 17..64 tokens: two-tile workgroups of 7 compute
    waves and a staging wave, with 4-group chunks up to 48 tokens and 2-group chunks above
    (N = 32784 leaves a 16-channel remainder after the last full 224-channel block, and
    K = 1024 a split count that the 147-block plan rounds to 2); the oracle computes 512
    sampled channels, the last 16 included."""
    x = synth.activations(41, M, N, M, K)
    qw, sc, z = synth.w4a16_weights(41, M, N, N, K)
    y = _gpu(x, qw, sc, z)
    rng = np.random.default_rng(M * 7 + N)
    cols = np.unique(np.concatenate([rng.choice(N, size=496, replace=False), np.arange(N - 16, N)]))
    r = oracle.linear_w4a16(x, qw[cols], sc[cols], z[cols])
    check_fp(y[:, cols], r, TOL)
    assert_all_written(y)


def test_code_equals_zero_gives_zero(gpu_lib):
    """q = z everywhere: every weight is exactly 0, so y = 0 exactly."""
    M, N, K = 5, 64, 512
    x = synth.activations(31, 0, 0, M, K)
    z = np.full((N, K // 128), 9, np.uint8)
    qw = np.full((N, K // 8), 0x99999999, np.uint32)
    sc = np.full((N, K // 128), 0.01, np.float16)
    y = _gpu(x, qw, sc, z)
    assert np.all(y.view(np.uint16) & 0x7FFF == 0)


def test_single_group_nonzero(gpu_lib):
    """Only group 1 has non-zero weights: y is that group's partial sum alone."""
    M, N, K = 3, 32, 512
    x = synth.activations(32, 0, 0, M, K)
    qw, sc, z = synth.w4a16_weights(32, 0, 0, N, K)
    zsel = z.copy()
    for g in (0, 2, 3):  # codes 0 and zero point 0: every weight of the group is exactly 0
        zsel[:, g] = 0
        qw[:, g * 16:(g + 1) * 16] = 0
    y = _gpu(x, qw, sc, zsel)
    r = oracle.linear_w4a16(x, qw, sc, zsel)
    only = oracle.linear_w4a16(x[:, 128:256].copy(), qw[:, 16:32].copy(), sc[:, 1:2].copy(),
                               zsel[:, 1:2].copy())
    assert_bits_equal(r, only, "oracle: group-1 sum")
    check_fp(y, r, TOL)


def test_golden_two_groups(gpu_lib):
    """The worked example (y = 208), channel replicated to the 16-channel tile."""
    x = np.ones((1, 256), np.float16)
    words = np.tile(np.array([0x76543210, 0xFEDCBA98], np.uint32), 16)
    qw = np.tile(words, (16, 1))
    sc = np.tile(np.array([0.5, 0.25], np.float16), (16, 1))
    z = np.tile(np.array([8, 0], np.uint8), (16, 1))
    y = _gpu(x, qw, sc, z)
    assert np.all(y == np.float16(208.0))


@pytest.mark.parametrize("M,N,K", [(48, 8192, 8192), (48, 33024, 2048)])
def test_repeat_is_bitwise_identical(gpu_lib, M, N, K):
    """Chunk kernel with split-K, and past 32768 channels the kernel with a staging wave."""
    x = synth.activations(33, 0, 0, M, K)
    qw, sc, z = synth.w4a16_weights(33, 0, 0, N, K)
    args = (dev(x), dev(qw), dev(sc), dev(z))
    y1 = host(ops.linear_w4a16(*args))
    y2 = host(ops.linear_w4a16(*args))
    assert_bits_equal(y1, y2, "rerun")


@pytest.mark.parametrize("cfg", [9, 1, 2, 3, 4, 5, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19])
@pytest.mark.parametrize("M,N,K", [(1, 272, 1152), (5, 512, 2048), (17, 144, 640), (48, 400, 3072),
                                   (49, 144, 1024), (64, 400, 3072)])
def test_every_kernel_configuration(gpu_lib, cfg, M, N, K):
    """Each work-split configuration of the fp16-weight W4A16 kernels (LDS-staged chunks = 9,
    register ring = 1..5, chunked ring = 10..17), with ragged channel blocks and split-K,
    against the oracle."""
    x = synth.activations(34, M, N, M, K)
    qw, sc, z = synth.w4a16_weights(34, M, N, N, K)
    r = oracle.linear_w4a16(x, qw, sc, z)
    check_fp(_gpu(x, qw, sc, z, {"W4A16_CFG": cfg}), r, TOL)


@pytest.mark.parametrize("cfg", list(range(100, 104)))
@pytest.mark.parametrize("M,N,K,splits", [
    (17, 144, 1024, 0),    # one 32-token tile, a half-filled last 32-channel tile
    (32, 400, 3072, 0),    # a full token tile, 24 groups split three ways
    (33, 272, 2048, 2),    # two token tiles, the second with one row
    (48, 400, 3072, 3),
    (64, 512, 4096, 0),
    (5, 256, 28672, 0),    # long K (224 groups), few tokens
    (48, 1024, 8192, 1),   # no split: fp16 stored by the GEMM itself
])
def test_wide_configurations(gpu_lib, cfg, M, N, K, splits):
    """Each shape of the wide kernel (32x32x16 MFMAs on 32-channel x 32-token tiles, weights
    as the A operand), with channel counts that leave a half tile, token counts that leave a
    ragged token tile, and split-K through the reduction launch."""
    x = synth.activations(38, M, N, M, K)
    qw, sc, z = synth.w4a16_weights(38, M, N, N, K)
    r = oracle.linear_w4a16(x, qw, sc, z)
    check_fp(_gpu(x, qw, sc, z, {"W4A16_CFG": cfg, "W4A16_SPLITS": splits}), r, TOL)


@pytest.mark.parametrize("cfg", list(range(110, 114)))
@pytest.mark.parametrize("M,N,K,splits", [
    (17, 272, 1024, 0),    # two token tiles (the second with one row), a ragged channel block
    (32, 464, 3072, 0),    # 24 groups, 29 tiles: two blocks, the second with one tile
    (33, 224, 2048, 2),    # three token tiles, one full block, split-K by the second launch
    (48, 480, 3072, 3),
    (64, 448, 4096, 0),    # four token tiles (only the 2-group-chunk shapes take them)
    (5, 256, 28672, 0),    # long K (224 groups), few tokens
    (48, 1024, 8192, 1),   # no split: fp16 stored by the GEMM itself
])
def test_stage_configurations(gpu_lib, cfg, M, N, K, splits):
    """Each shape of the kernel with a staging wave (7 compute waves of one or two 16-channel
    tiles plus one wave that only fills the activation chunks), over ragged channel blocks,
    ragged token tiles and split-K.  A shape that cannot hold a whole chunk in its staging
    wave at this M is refused by the planner, which then runs the default plan."""
    x = synth.activations(43, M, N, M, K)
    qw, sc, z = synth.w4a16_weights(43, M, N, N, K)
    r = oracle.linear_w4a16(x, qw, sc, z)
    check_fp(_gpu(x, qw, sc, z, {"W4A16_CFG": cfg, "W4A16_SPLITS": splits}), r, TOL)


SMALL_CFGS = ([20, 21, 22, 23, 24, 25, 40, 41, 42, 43, 44, 45] + list(range(60, 68)) +
              list(range(80, 88)))


@pytest.mark.parametrize("cfg", SMALL_CFGS)
@pytest.mark.parametrize("M,N,K,splits", [
    (1, 272, 1024, 0),     # 17 tiles: a partial tile block; parts past K (ghost waves)
    (2, 512, 4096, 0),
    (3, 144, 8192, 0),     # three tokens in the four-output lanes
    (4, 1024, 3072, 3),    # 24 groups in 3 splits
    (5, 400, 2048, 0),
    (16, 256, 5120, 0),    # a full token tile, 40 groups
    (9, 64, 28672, 0),     # long K (224 groups), split across workgroups by default
    (1, 160, 8192, 5),     # splits that do not divide the blocks
])
def test_small_m_configurations(gpu_lib, cfg, M, N, K, splits):
    """Each shape of the small-M kernels (activations as the MFMA's A operand, fp32 group
    sums scaled per group): chunk-staged 20..25 (zero point subtracted in fp16) and 40..45
    (with a second MFMA), whole-slice-staged 60..67 and 80..87, with partial tile blocks,
    parts past the end of K and forced split counts.  A slice that cannot fit in LDS falls
    back to the default plan, which is checked the same way."""
    x = synth.activations(35, M, N, M, K)
    qw, sc, z = synth.w4a16_weights(35, M, N, N, K)
    r = oracle.linear_w4a16(x, qw, sc, z)
    tune = {"W4A16_CFG": cfg, "W4A16_SPLITS": splits}
    check_fp(_gpu(x, qw, sc, z, tune), r, TOL)


@pytest.mark.parametrize("cfg", [20, 40, 60, 80])
def test_small_m_exact_integer_case(gpu_lib, cfg):
    """s = 1, z = 8 and activations that are small integers: every product, group sum and
    partial sum (also with the 1024 offsets of the zero-point MFMA) is an integer far below
    2^24, exact in fp32, so the small-M kernel rounds the exact sum to fp16 once, as the
    oracle does: bit-equal results."""
    M, N, K = 3, 64, 2048
    rng = np.random.default_rng(36)
    x = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    qw = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = np.ones((N, K // 128), np.float16)
    z = np.full((N, K // 128), 8, np.uint8)
    r = oracle.linear_w4a16(x, qw, sc, z)
    assert_bits_equal(_gpu(x, qw, sc, z, {"W4A16_CFG": cfg}), r, "y")


@pytest.mark.parametrize("cfg,M,N,K,splits", [
    (10, 17, 144, 2048, 2), (13, 48, 400, 3072, 3), (14, 64, 272, 4096, 4), (14, 48, 8192, 8192, 0),
    (20, 5, 400, 4096, 4), (41, 16, 256, 5120, 5), (45, 9, 64, 28672, 0), (61, 1, 160, 8192, 5),
    (81, 4, 1024, 3072, 3), (87, 3, 144, 8192, 2)])
def test_split_reduce_launch_matches_in_kernel_finish(gpu_lib, cfg, M, N, K, splits):
    """The split-K finish as its own launch adds the same fp32 partials in the same split
    order as the last workgroup of each tile does: bit-identical outputs, both within the bar
    of the oracle."""
    x = synth.activations(37, M, N, M, K)
    qw, sc, z = synth.w4a16_weights(37, M, N, N, K)
    r = oracle.linear_w4a16(x, qw, sc, z)
    base = {"W4A16_CFG": cfg, "W4A16_SPLITS": splits}
    y1 = _gpu(x, qw, sc, z, dict(base, W4A16_REDUCE=1))
    y2 = _gpu(x, qw, sc, z, dict(base, W4A16_REDUCE=2))
    check_fp(y2, r, TOL)
    assert_bits_equal(y2, y1, "reduce launch vs in-kernel finish")
