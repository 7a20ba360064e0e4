"""GPU parity of the device draft-tree builder (sv_build_tree) against the
CPU oracle: parent, depth and rank arrays compared exactly, at the measured
workloads' tree shapes (256 nodes / depth 8 / 32 candidates; 16 trees of 64
nodes / depth 6), on random small cases, on a tie-order case and on the edge
cases (a lone root, one candidate per depth, a budget equal to every
reachable node)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import depth_logprobs

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


def _check(lps, n, max_depth):
    lp_t = torch.from_numpy(np.ascontiguousarray(lps, dtype=np.float64)).cuda()
    parent, depth, rank = (x.cpu().numpy() for x in sv.build_tree(lp_t, n))
    for b in range(lps.shape[0]):
        ref = oracle.build_best_first_tree(lps[b], n, max_depth)
        assert np.array_equal(parent[b], ref[0]), f"tree {b}: parents differ"
        assert np.array_equal(depth[b], ref[1]) and np.array_equal(rank[b], ref[2]), f"tree {b}"


@pytest.mark.parametrize("B,n,depth,n_cand", [(1, 256, 8, 32), (16, 64, 6, 32), (5, 100, 3, 7), (3, 2, 1, 1)])
def test_build_tree_exact(B, n, depth, n_cand):
    r = np.random.default_rng(n + depth)
    lps = np.stack([depth_logprobs(r, depth, n_cand=n_cand) for _ in range(B)])
    _check(lps, n, depth)


def test_build_tree_edges_and_ties():
    # a lone root
    _check(np.zeros((2, 4, 3)), 1, 3)
    # one candidate per depth: a chain
    lps = np.stack([depth_logprobs(np.random.default_rng(1), 40, n_cand=1)])
    _check(lps, 41, 40)
    # every reachable node: 1 + 3 + 9 + 27
    _check(np.stack([depth_logprobs(np.random.default_rng(2), 3, n_cand=3)]), 40, 3)
    # equal log-probabilities everywhere: order decided by parent id, then rank
    _check(np.full((2, 5, 4), -1.0), 60, 4)
    _check(np.array([[[0.0, 0.0], [-1.0, -1.0], [-1.0, -2.0]]]), 5, 2)


def _reachable(nc, depth):
    reach, lev = 1, 1
    for _ in range(depth):
        lev = min(lev * nc, 1 << 20)
        reach += lev
    return reach


@pytest.mark.parametrize("kind", ["plain", "quarter_ties", "fine_ties", "all_equal", "wide", "zero_logprobs"])
def test_build_tree_random_shapes(kind):
    """Random budgets, depths and candidate counts, with log-probabilities
    rounded to coarse and fine grids (many exactly equal scores, also at the
    budget's threshold), constant rows, scores spread over hundreds of units,
    and zero log-probabilities (a child or sibling scoring exactly what its
    parent or elder sibling scores)."""
    r = np.random.default_rng(["plain", "quarter_ties", "fine_ties", "all_equal", "wide",
                               "zero_logprobs"].index(kind) + 500)
    for t in range(12):
        depth = int(r.integers(1, 10))
        nc = int(r.integers(1, 40))
        n = int(r.integers(1, min(256, _reachable(nc, depth)) + 1))
        B = int(r.integers(1, 4))
        lps = []
        for _ in range(B):
            lp = depth_logprobs(r, depth, n_cand=nc)
            if kind == "quarter_ties":
                lp = np.round(lp * 4) / 4
            elif kind == "fine_ties":
                lp = np.round(lp * 64) / 64
            elif kind == "all_equal":
                lp = np.full_like(lp, -0.75)
            elif kind == "wide":
                lp = lp * 30.0
            elif kind == "zero_logprobs":
                lp[1:, 0] = 0.0
            lps.append(lp)
        print(f"[case] {kind} #{t}: B={B} n={n} depth={depth} n_cand={nc}", flush=True)
        _check(np.stack(lps), n, depth)


def test_build_tree_many_large_budgets():
    """Budgets near the 256-node maximum over deep and wide candidate lists
    (up to depth 12 and 64 candidates), with a few exact-tie grids mixed in: the
    trial values then isolate several hundred sequences, near the per-wave list
    limit, and the first round's spacing is exercised on many list shapes."""
    r = np.random.default_rng(777)
    for t in range(60):
        depth = int(r.integers(3, 13))
        nc = int(r.integers(8, 65))
        n = int(r.integers(128, 257))
        lp = depth_logprobs(r, depth, n_cand=nc, var=float(r.uniform(0.5, 4.0)))
        grid = t % 4
        if grid == 1:
            lp = np.round(lp * 16) / 16
        elif grid == 2:
            lp = lp * float(r.uniform(0.05, 0.3))  # scores packed close together
        print(f"[case] many #{t}: n={n} depth={depth} n_cand={nc} grid={grid}", flush=True)
        _check(lp[None], n, depth)
