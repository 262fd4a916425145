"""Seeded synthetic inputs for the verify path.

This module only draws random numbers: it holds none of the method's arithmetic, and both
the GPU tests and the CPU oracle receive their inputs from it.  No trained weights or
evaluation prompts exist here; every tensor has the shape, dtype and value distribution of
the model layers the verify pass runs over:

* activations: fp16 N(0, 1), [M][K], one row per verified position (last accepted token
  plus the draft tokens);
* W8A8 weights: int8 uniform in [-127, 127], [N][K]; per-output-channel fp32 scales
  uniform in [1e-3, 1e-2);
* W4A16 weights: 4-bit codes uniform in 0..15 packed eight per uint32 (low nibble = lowest
  k), [N][K/8]; per-(channel, 128-group) fp16 scales uniform in [1e-3, 2e-2) and zero
  points uniform in 0..15 (stored one per byte);
* draft tokens: each position copies the verifier's argmax with probability 0.6 until the
  first miss, then tokens are uniform over the vocabulary.

Streams come from ``numpy.random.Generator(PCG64(SeedSequence([config, layer, linear,
tensor])))`` so any single tensor of a stack can be regenerated on its own.
"""
from __future__ import annotations

import numpy as np

# tensor ids inside one linear
T_X, T_W, T_WSCALE, T_ZEROS, T_DRAFT = 0, 1, 2, 3, 4

# Layer shapes (K = in_features, N = out_features) of the two model families the pages
# evaluate: Qwen3-8B (hidden 4096, intermediate 12288, vocab 151936) for the W8A8
# verifier and Llama-3-70B (hidden 8192, intermediate 28672) for the W4A16 verifier.
QWEN3_8B_LINEARS = {
    "qkv": (4096, 6144),
    "o": (4096, 4096),
    "gate_up": (4096, 24576),
    "down": (12288, 4096),
}
QWEN3_8B_LAYERS = 36
QWEN3_8B_VOCAB = 151936
LLAMA3_70B_LINEARS = {
    "qkv": (8192, 10240),
    "o": (8192, 8192),
    "gate_up": (8192, 57344),
    "down": (28672, 8192),
}
LLAMA3_70B_LAYERS = 80
LINEAR_IDS = {"qkv": 0, "o": 1, "gate_up": 2, "down": 3, "lm_head": 4}


def rng(config: int, layer: int, linear: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, layer, linear, tensor])))


def activations(config: int, layer: int, linear: int, M: int, K: int) -> np.ndarray:
    """fp16 N(0,1) [M][K]."""
    return rng(config, layer, linear, T_X).standard_normal((M, K), dtype=np.float32).astype(np.float16)


def w8a8_weights(config: int, layer: int, linear: int, N: int, K: int):
    """(w int8 [N][K] uniform in [-127,127], w_scale fp32 [N] uniform in [1e-3, 1e-2))."""
    w = rng(config, layer, linear, T_W).integers(-127, 128, size=(N, K), dtype=np.int8)
    s = rng(config, layer, linear, T_WSCALE).uniform(1e-3, 1e-2, size=N).astype(np.float32)
    return w, s


def w4a16_weights(config: int, layer: int, linear: int, N: int, K: int, group_size: int = 128):
    """(qweight uint32 [N][K/8], scales fp16 [N][K/G], zeros uint8 [N][K/G])."""
    assert K % group_size == 0 and K % 8 == 0
    # Uniform 32-bit words give eight independent uniform 4-bit codes each.
    q = rng(config, layer, linear, T_W).integers(0, 2**32, size=(N, K // 8), dtype=np.uint32)
    s = rng(config, layer, linear, T_WSCALE).uniform(1e-3, 2e-2, size=(N, K // group_size))
    z = rng(config, layer, linear, T_ZEROS).integers(0, 16, size=(N, K // group_size), dtype=np.uint8)
    return q, s.astype(np.float16), z


def draft_tokens(config: int, verifier_argmax: np.ndarray, V: int, p_match: float = 0.6):
    """Draft tokens for rows 1..M-1 given the verifier's argmax of rows 0..M-2.

    Returns (draft int32 [M-1], planned n_accept).  Position i keeps matching with
    probability p_match until the first miss; a miss draws a token different from the
    argmax, and every later position is uniform over the vocabulary.
    """
    a = np.asarray(verifier_argmax, dtype=np.int64)
    M = a.shape[0]
    g = rng(config, 0, LINEAR_IDS["lm_head"], T_DRAFT)
    u = g.random(max(M - 1, 0))
    r = g.integers(0, V - 1, size=max(M - 1, 0))
    tail = g.integers(0, V, size=max(M - 1, 0))
    draft = np.zeros((max(M - 1, 0),), np.int32)
    planned = M - 1
    matching = True
    for i in range(M - 1):
        if matching and u[i] < p_match:
            draft[i] = a[i]
        elif matching:
            draft[i] = (a[i] + 1 + r[i]) % V
            matching = False
            planned = i
        else:
            draft[i] = tail[i]
    return draft, planned


T_TREE = 5  # tensor id of a draft tree's shape and tokens


def draft_tree(config: int, M: int, vocab: int, p_match: float = 0.6,
               argmax: np.ndarray | None = None):
    """A draft tree of M nodes shaped like a dynamic draft tree (node 0 is the root; every
    later node hangs under one of the 8 nodes before it, so depths vary from 1 to M - 1),
    with node tokens that equal the target's argmax at their parent with probability
    p_match and are a different token otherwise.

    argmax: the target's argmax at each node (int [M]); drawn uniformly from [0, vocab) when
    not given.  Returns (parent int32 [M] with parent[0] = -1, tokens int32 [M] with
    tokens[0] = 0, argmax int32 [M]).
    """
    g = rng(config, M, vocab, T_TREE)
    if argmax is None:
        argmax = g.integers(0, vocab, size=M)
    a = np.asarray(argmax, dtype=np.int64)
    parent = np.full((M,), -1, np.int32)
    tokens = np.zeros((M,), np.int32)
    for v in range(1, M):
        parent[v] = int(g.integers(max(0, v - 8), v))
        if g.random() < p_match:
            tokens[v] = a[parent[v]]
        else:
            tokens[v] = (a[parent[v]] + 1 + int(g.integers(0, vocab - 1))) % vocab
    return parent, tokens, a.astype(np.int32)


T_SAMPLE = 6  # tensor id of the stochastic-verification inputs


def sampling_inputs(config: int, M: int, V: int, with_draft_logits: bool = True,
                    noise: float = 0.5, p_top: float = 0.7):
    """Inputs of stochastic verification at one sequence: M target rows (M - 1 drafts and
    the bonus row) over a vocabulary of V.

    Target logits are fp16 N(0, 2.5) with one planted peak per row (+12 at a uniform token),
    so the rows are peaked like a language model's; the drafter's logits are the target's
    plus N(0, noise) and, with probability 0.2 per row, a peak at another token.  Each draft
    token is the drafter's peak with probability p_top, else one of the drafter's 16 largest
    logits at random.  Returns (target fp16 [M][V], draft_logits fp16 [M-1][V] or None,
    draft int32 [M-1], u float64 [M] uniform in [0, 1)).
    """
    g = rng(config, M, V, T_SAMPLE)
    target = g.normal(0.0, 2.5, (M, V)).astype(np.float32)
    peak = g.integers(0, V, M)
    target[np.arange(M), peak] += 12.0
    drafter = target[:M - 1] + g.normal(0.0, noise, (M - 1, V)).astype(np.float32)
    moved = g.random(M - 1) < 0.2
    other = g.integers(0, V, M - 1)
    drafter[np.arange(M - 1)[moved], other[moved]] += 12.0
    target = np.clip(target, -65504, 65504).astype(np.float16)
    drafter = np.clip(drafter, -65504, 65504).astype(np.float16)
    draft = np.zeros((M - 1,), np.int32)
    pick_top = g.random(M - 1) < p_top
    pick = g.integers(0, min(16, V), M - 1)
    for i in range(M - 1):
        order = np.argsort(-drafter[i].astype(np.float32), kind="stable")
        draft[i] = order[0] if pick_top[i] else order[pick[i]]
    u = g.random(M)
    return target, (drafter if with_draft_logits else None), draft, u
