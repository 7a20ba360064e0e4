"""Draft-tree shapes for verification workloads.

A draft tree is a parent array over N nodes: node 0 is the root (the last
committed token, whose query row is verified first), ``parent[0] = -1`` and
``0 <= parent[i] < i`` for every other node, so nodes are in topological order.

The tree generator follows the construction step on the JETFLOW page
(JETFLOW, section 2, "Construção da Árvore"): candidates are ranked by their
cumulative draft log-probability and the best one is expanded first, until a
node budget is reached.  The draft head itself is not available, so the
per-depth log-probabilities are synthetic: at each depth, a softmax over 32
seeded logits drawn from N(0, 2) (variance 2), sorted in decreasing order.
Every node at the same depth shares that depth's candidate list.
"""
from __future__ import annotations

import heapq

import numpy as np


def chain_parents(n: int) -> np.ndarray:
    """Parent array of a linear draft chain: node i's parent is i-1."""
    p = np.arange(-1, n - 1, dtype=np.int32)
    return p


def depth_logprobs(rng: np.random.Generator, max_depth: int, n_cand: int = 32,
                   var: float = 2.0) -> np.ndarray:
    """Per-depth candidate log-probabilities, shape [max_depth + 1][n_cand].

    Row d (1 <= d <= max_depth) is log_softmax of ``n_cand`` logits ~ N(0, var),
    sorted in decreasing order; row 0 is unused (the root is not drafted).
    """
    lp = np.zeros((max_depth + 1, n_cand), dtype=np.float64)
    for d in range(1, max_depth + 1):
        z = rng.normal(0.0, np.sqrt(var), size=n_cand)
        zmax = z.max()
        lse = zmax + np.log(np.exp(z - zmax).sum())
        lp[d] = np.sort(z - lse)[::-1]
    return lp


def best_first_tree(n_nodes: int, lp: np.ndarray, max_depth: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Grow a tree of ``n_nodes`` nodes (root included) by best-first expansion.

    A candidate is (parent node, depth, rank within that depth's list); its score
    is the parent's cumulative log-probability plus ``lp[depth][rank]``.  The
    candidate with the highest score becomes the next node (ties: lower parent
    id, then lower rank).  Popping a candidate pushes its first child (rank 0 at
    the next depth, if the depth limit allows) and its next sibling (rank + 1).
    Because every log-probability is negative, the node set is always closed
    under taking ancestors.

    Returns (parent, depth, rank), each int32[n_nodes] (rank of the root is 0).
    """
    n_cand = lp.shape[1]
    parent = [-1]
    depth = [0]
    rank = [0]
    cum = [0.0]
    heap: list = []
    if n_nodes > 1 and max_depth >= 1:
        heapq.heappush(heap, (-(0.0 + lp[1][0]), 0, 0, 1))
    while len(parent) < n_nodes:
        if not heap:
            raise ValueError("tree budget exceeds the number of reachable nodes")
        neg, p, r, d = heapq.heappop(heap)
        c = -neg
        i = len(parent)
        parent.append(p)
        depth.append(d)
        rank.append(r)
        cum.append(c)
        if d < max_depth:
            heapq.heappush(heap, (-(c + lp[d + 1][0]), i, 0, d + 1))
        if r + 1 < n_cand:
            heapq.heappush(heap, (-(cum[p] + lp[d][r + 1]), p, r + 1, d))
    return (np.asarray(parent, dtype=np.int32), np.asarray(depth, dtype=np.int32),
            np.asarray(rank, dtype=np.int32))
