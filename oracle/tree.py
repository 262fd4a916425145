"""Greedy acceptance of a draft tree (TEST INFRASTRUCTURE ONLY; the product library never
imports this).

Speculative Decoding Meets Quantization (review page, "What carries the argument" and "Core
claim"): EAGLE-2 drafts a token tree, the target verifies every node in one forward pass,
and verification turns the tree into the sequential draft that is accepted.  With greedy
decoding the target's top-1 token at a node decides which child may follow it.

Reading taken (the pages give no formula):
  * node 0 is the root (the last accepted token); nodes 1..M-1 are drafts, each with a
    parent index p with 0 <= p < node (a node whose parent index is out of that range is
    never accepted, nor anything below it);
  * a node is accepted iff its parent is accepted and its token equals the target's argmax
    at the parent; the root is accepted;
  * the accepted path ends at the accepted node of greatest depth, the lowest index among
    equals; the step emits the tokens of the path's drafts and then the target's argmax at
    the path's last node (the bonus token).

`tree_accept` follows that definition node by node in index order; `tree_accept_dfs` is an
independent second reading (a depth-first search over accepted children) used to pin it.
"""
from __future__ import annotations

import numpy as np


def tree_accept(argmax: np.ndarray, tokens: np.ndarray, parent: np.ndarray):
    """argmax, tokens, parent: int [M] -> (path list of node indices from the root,
    accept length = len(path) - 1, bonus token = argmax at the path's last node)."""
    a = [int(v) for v in argmax]
    t = [int(v) for v in tokens]
    p = [int(v) for v in parent]
    M = len(a)
    accepted = [False] * M
    depth = [0] * M
    accepted[0] = True
    for v in range(1, M):
        if 0 <= p[v] < v and accepted[p[v]] and t[v] == a[p[v]]:
            accepted[v] = True
            depth[v] = depth[p[v]] + 1
    best = 0
    for v in range(1, M):
        if accepted[v] and depth[v] > depth[best]:
            best = v
    path = [best]
    while path[-1] != 0:
        path.append(p[path[-1]])
    path.reverse()
    return path, len(path) - 1, a[best]


def tree_accept_dfs(argmax: np.ndarray, tokens: np.ndarray, parent: np.ndarray):
    """The same result by a depth-first search from the root over the children whose token
    equals the target's argmax at their parent (visiting children in index order)."""
    a = [int(v) for v in argmax]
    t = [int(v) for v in tokens]
    p = [int(v) for v in parent]
    M = len(a)
    children = {v: [] for v in range(M)}
    for v in range(1, M):
        if 0 <= p[v] < v:
            children[p[v]].append(v)
    best_path = [0]

    def visit(path):
        nonlocal best_path
        if len(path) > len(best_path) or (len(path) == len(best_path) and path[-1] < best_path[-1]):
            best_path = list(path)
        for c in children[path[-1]]:
            if t[c] == a[path[-1]]:
                visit(path + [c])

    visit([0])
    return best_path, len(best_path) - 1, a[best_path[-1]]
