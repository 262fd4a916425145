"""Pins of the greedy tree-acceptance oracle (oracle/tree.py): a chain reduces to the
longest-matching-prefix rule of the chain oracle; a star accepts at most one child; the
forward scan agrees with an independent depth-first search on random trees; a worked
example; and structural invariants of every result."""
import numpy as np
import pytest

import oracle
from oracle.tree import tree_accept, tree_accept_dfs
from quantized_weight_verification_amd import synth


def _check_valid(argmax, tokens, parent, path, L, bonus):
    assert path[0] == 0 and len(path) == L + 1
    for d in range(1, len(path)):
        v, u = path[d], path[d - 1]
        assert parent[v] == u and u < v
        assert tokens[v] == argmax[u]
    assert bonus == argmax[path[-1]]


def test_chain_is_the_longest_matching_prefix():
    rng = np.random.default_rng(1)
    for _ in range(200):
        M = int(rng.integers(1, 65))
        a = rng.integers(0, 5, M).astype(np.int32)
        d = rng.integers(0, 5, max(M - 1, 1)).astype(np.int32)[: M - 1]
        tokens = np.concatenate([[0], d]).astype(np.int32)
        parent = np.arange(-1, M - 1, dtype=np.int32)
        path, L, bonus = tree_accept(a, tokens, parent)
        n = oracle.accept(d if M > 1 else np.zeros(0, np.int32), a)
        assert L == n and path == list(range(n + 1)) and bonus == a[n]


def test_star_accepts_the_lowest_matching_child():
    a = np.array([7, 1, 2, 3, 4, 5], np.int32)
    parent = np.array([-1, 0, 0, 0, 0, 0], np.int32)
    tokens = np.array([0, 3, 7, 9, 7, 1], np.int32)
    assert tree_accept(a, tokens, parent) == ([0, 2], 1, 2)
    tokens = np.array([0, 3, 6, 9, 8, 1], np.int32)
    assert tree_accept(a, tokens, parent) == ([0], 0, 7)


def test_worked_example():
    """Root argmax 5.  Children 1 (token 5, argmax 8) and 2 (token 5, argmax 9) both match;
    node 3 under 1 (token 8) matches, node 4 under 2 (token 9) matches, node 5 under 4
    (token 2, argmax at 4 is 2) matches: the deepest accepted node is 5 at depth 3."""
    a = np.array([5, 8, 9, 1, 2, 6], np.int32)
    tokens = np.array([0, 5, 5, 8, 9, 2], np.int32)
    parent = np.array([-1, 0, 0, 1, 2, 4], np.int32)
    assert tree_accept(a, tokens, parent) == ([0, 2, 4, 5], 3, 6)


def test_invalid_parent_cuts_the_subtree():
    a = np.array([5, 5, 5, 5], np.int32)
    tokens = np.array([0, 5, 5, 5], np.int32)
    parent = np.array([-1, 0, 3, 2], np.int32)   # node 2 points forward: never accepted
    assert tree_accept(a, tokens, parent) == ([0, 1], 1, 5)


@pytest.mark.parametrize("seed", range(40))
def test_forward_scan_equals_dfs_on_random_trees(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 65))
    parent, tokens, a = synth.draft_tree(seed, M, vocab=6, p_match=0.7)
    r1 = tree_accept(a, tokens, parent)
    r2 = tree_accept_dfs(a, tokens, parent)
    assert r1 == r2
    _check_valid(a, tokens, parent, *r1)
