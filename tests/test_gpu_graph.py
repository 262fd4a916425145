"""The verify path inside a HIP graph: a captured sequence (quantise, split-K W8A8, split-K
W4A16, greedy verify) replayed several times, with eager work and synchronisations between
the replays, matches the eager results bit for bit on every replay.  The split-K arrival
counters re-arm themselves, so no memset node is needed in the graph."""
import numpy as np
import pytest
import torch

from quantized_weight_verification_amd import _binding as B, ops, synth
from _util import assert_bits_equal, dev, host

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_lib):
    M, K, N = 8, 8192, 256          # W8A8 shape that takes the split-K path
    assert ops.workspace_bytes(B.QV_OP_W8A8, M, N, K) > 0
    M4, K4, N4 = 5, 8192, 512       # W4A16 shape that takes the split-K path
    assert ops.workspace_bytes(B.QV_OP_W4A16, M4, N4, K4) > 0
    x = dev(synth.activations(40, 0, 0, M, K))
    w, sw = (dev(a) for a in synth.w8a8_weights(40, 0, 0, N, K))
    x4 = dev(synth.activations(40, 0, 1, M4, K4))
    qw, sc, z = (dev(a) for a in synth.w4a16_weights(40, 0, 1, N4, K4))
    draft = dev(np.arange(M - 1, dtype=np.int32))

    xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    y = torch.empty(M, N, dtype=torch.float16, device="cuda")
    y4 = torch.empty(M4, N4, dtype=torch.float16, device="cuda")
    am = torch.empty(M, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")

    def seq():
        ops.quant_act(x, out=xq, scale_out=sx)
        ops.linear_w8a8(xq, sx, w, sw, out=y)
        ops.linear_w4a16(x4, qw, sc, z, out=y4)
        ops.verify_greedy(y, draft, argmax_out=am, n_accept_out=na)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        seq()
    torch.cuda.synchronize()
    ref = [host(t).copy() for t in (xq, sx, y, y4, am, na)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        seq()
    for rep in range(4):
        for t in (xq, sx, y, y4, am, na):
            t.zero_()
        _ = (x.float() * 2).sum().item()     # unrelated eager work between replays
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("x_q", "x_scale", "y", "y4", "argmax", "n_accept"),
                              (xq, sx, y, y4, am, na), ref):
            assert_bits_equal(host(t), r, f"replay {rep}: {name}")
