"""The verify path inside a HIP graph: a captured sequence (quantise, split-K W8A8, split-K
W4A16, greedy verify) replayed several times, with eager work and synchronisations between
the replays, matches the eager results bit for bit on every replay.  The split-K arrival
counters re-arm themselves, so no memset node is needed in the graph."""
import numpy as np
import pytest
import torch

import oracle
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


def test_graph_replays_of_the_widened_calls(gpu_lib):
    """Tree verification, speculative sampling (two launches sharing a draw counter), the W4A8
    linear with split-K at M = 5 and with the chunked kernel at M = 48, the W4A16 linear at
    M = 1 (whole-slice kernel) and at M = 48 (chunked kernel with its split-K reduction
    launch; past 32768 channels the kernel with a staging wave, also split), and the weight
    preparation passes: captured once, replayed four times with eager
    work in between, every replay bit-identical to the eager results."""
    M, V = 48, 20000
    logits = dev((np.random.default_rng(50).standard_normal((M, V)) * 3).astype(np.float16))
    parent, tokens, _ = synth.draft_tree(50, M, V, 0.8)
    parent, tokens = dev(parent), dev(tokens)
    tgt, dl, dr, u = synth.sampling_inputs(51, 8, 151936, True)
    tgt, dl, dr = dev(tgt), dev(dl), dev(dr)
    u = torch.from_numpy(u).cuda()
    assert ops.workspace_bytes(B.QV_OP_W4A8, 5, 512, 8192) > 0
    x5 = synth.activations(52, 0, 0, 5, 8192)
    x48 = synth.activations(52, 0, 1, 48, 8192)
    qw, sc, z = (dev(a) for a in synth.w4a16_weights(52, 0, 0, 512, 8192))
    xq5, sx5 = ops.quant_act(dev(x5))
    xq48, sx48 = ops.quant_act(dev(x48))
    x1d, x48d = dev(x5[:1]), dev(x48)
    qs, ss, zs = (dev(a) for a in synth.w4a16_weights(54, 0, 0, 33024, 2048))
    x48s = dev(synth.activations(54, 0, 1, 48, 2048))
    wb = dev((np.random.default_rng(53).standard_normal((256, 1024)).astype(np.float32)
              .view(np.uint32) >> 16).astype(np.uint16).view(np.int16))

    am = torch.empty(M, dtype=torch.int32, device="cuda")
    path = torch.empty(M, dtype=torch.int32, device="cuda")
    acc = torch.empty(2, dtype=torch.int32, device="cuda")
    res = torch.empty(2, dtype=torch.int32, device="cuda")
    y5 = torch.empty(5, 512, dtype=torch.float16, device="cuda")
    y48 = torch.empty(48, 512, dtype=torch.float16, device="cuda")
    w1 = torch.empty(1, 512, dtype=torch.float16, device="cuda")
    w48 = torch.empty(48, 512, dtype=torch.float16, device="cuda")
    s48 = torch.empty(48, 33024, dtype=torch.float16, device="cuda")
    outs = {}

    def seq():
        ops.verify_tree(logits, tokens, parent, argmax_out=am, path_out=path, accept_out=acc)
        ops.verify_sample(tgt, dr, u, 0.8, draft_logits=dl, result_out=res)
        ops.linear_w4a8(xq5, sx5, qw, sc, z, out=y5)
        ops.linear_w4a8(xq48, sx48, qw, sc, z, out=y48)
        ops.linear_w4a16(x1d, qw, sc, z, out=w1)
        ops.linear_w4a16(x48d, qw, sc, z, out=w48)
        ops.linear_w4a16(x48s, qs, ss, zs, out=s48)
        outs["w8"] = ops.prepare_w8(wb)
        outs["w4"] = ops.prepare_w4(wb)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        seq()
    torch.cuda.synchronize()
    fixed = (am, path, acc, res, y5, y48, w1, w48, s48)
    ref = [host(t).copy() for t in fixed]
    ref_prep = [host(t).copy() for t in (*outs["w8"], *outs["w4"])]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        seq()
    prep_graph = (*outs["w8"], *outs["w4"])   # the tensors the captured calls write
    for rep in range(4):
        for t in fixed + prep_graph:
            t.zero_()
        _ = (logits.float() * 2).sum().item()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("argmax", "path", "accept", "sample", "w4a8 M5", "w4a8 M48",
                               "w4a16 M1", "w4a16 M48", "w4a16 M48 staged"), fixed, ref):
            assert_bits_equal(host(t), r, f"replay {rep}: {name}")
        for name, t, r in zip(("w8 codes", "w8 scales", "w4 qweight", "w4 scales", "w4 zeros"),
                              prep_graph, ref_prep):
            assert_bits_equal(host(t), r, f"replay {rep}: {name}")


def test_graph_replays_of_the_many_tile_w8a8_ring(gpu_lib):
    """The dominant launch of the verify step (a W8A8 linear with >= 1024 16-channel tiles at
    M = 8: two 2-wave tiles per workgroup, no split-K) captured behind its quant_act launch and
    replayed: every replay equals the eager result and the oracle bit for bit."""
    M, K, N = 8, 4096, 16384
    x_np = synth.activations(41, 0, 0, M, K)
    w_np, sw_np = synth.w8a8_weights(41, 0, 0, N, K)
    x, w, sw = dev(x_np), dev(w_np), dev(sw_np)
    xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    y = torch.empty(M, N, dtype=torch.float16, device="cuda")

    def seq():
        ops.quant_act(x, out=xq, scale_out=sx)
        ops.linear_w8a8(xq, sx, w, sw, out=y)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        seq()
    torch.cuda.synchronize()
    ref = host(y).copy()
    xq_o, sx_o = oracle.quant_act(x_np)
    y_o, _ = oracle.linear_w8a8(xq_o, sx_o, w_np, sw_np)
    assert_bits_equal(ref, y_o, "eager y")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        seq()
    for rep in range(3):
        y.zero_()
        _ = (x.float() * 2).sum().item()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(host(y), ref, f"replay {rep}: y")
