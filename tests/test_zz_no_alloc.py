"""GPU parity of the no-allocation entry point: qv_verify_greedy_noalloc (static per-GPU
scratch inside libqv.so) against qv_verify_greedy (caller workspace) and the oracle, called
through the C ABI, twice in a row with the second call smaller (the scratch keeps the first
call's contents; its counters must be back at zero).  Bar: argmax indices and accept lengths
bit-exact."""
import ctypes

import numpy as np
import pytest

import oracle
from quantized_weight_verification_amd import _binding as B, ops, synth
from _util import dev, host, sentinel

pytestmark = pytest.mark.gpu


def _noalloc(logits_d, draft_d):
    import torch

    M, V = logits_d.shape
    am = sentinel((M,), "idx")
    na = sentinel((1,), "idx")
    st = B.lib().qv_verify_greedy_noalloc(
        logits_d.data_ptr(), M, V, draft_d.data_ptr() if M > 1 else None, am.data_ptr(),
        na.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    B.check("qv_verify_greedy_noalloc", st)
    return host(am), int(host(na)[0])


def _with_workspace(logits_d, draft_d):
    M = logits_d.shape[0]
    am = sentinel((M,), "idx")
    na = sentinel((1,), "idx")
    ops.verify_greedy(logits_d, draft_d if M > 1 else None, argmax_out=am, n_accept_out=na)
    return host(am), int(host(na)[0])


@pytest.mark.parametrize("first,second", [((8, 151936), (3, 4099)), ((64, 128256), (1, 16384)),
                                          ((17, 40000), (16, 39999))])
def test_noalloc_matches_workspace_call(gpu_lib, first, second):
    for call, (M, V) in enumerate((first, second)):
        x = synth.activations(61, call, M, M, V)  # fp16 N(0,1) rows, as logits
        am_o = oracle.argmax(x)
        draft, planned = synth.draft_tokens(62 + call, am_o, V)
        xd, dd = dev(x), dev(draft)
        am_n, na_n = _noalloc(xd, dd)
        am_w, na_w = _with_workspace(xd, dd)
        assert np.array_equal(am_n, am_w), f"call {call}: argmax differs from the workspace call"
        assert na_n == na_w, f"call {call}: n_accept differs from the workspace call"
        assert np.array_equal(am_n, am_o), f"call {call}: argmax differs from the oracle"
        assert na_n == oracle.accept(draft, am_o) == planned
