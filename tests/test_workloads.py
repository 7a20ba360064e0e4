"""Seeded generators: determinism, layouts, and the best-first tree construction
(JETFLOW §2, tree construction) pinned by brute-force enumeration."""
import itertools

import numpy as np
import pytest

from workloads import (best_first_tree, bf16_bits_from_f32, depth_logprobs, f32_from_bf16_bits,
                       make_custom, make_workload)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1.0 + 2 ** -9], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 ties up to 1 + 2^-6
    got = f32_from_bf16_bits(bf16_bits_from_f32(x))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.015625 and got[3] == -2.5
    assert got[5] == 1.0
    assert np.isfinite(got).all()


def test_deterministic_and_seed_sensitive():
    a = make_custom(seed=[1, 2], dtype="bf16", B=2, Hq=8, Hkv=2, D=64, P=[40, 70], N=6, tree="best_first")
    b = make_custom(seed=[1, 2], dtype="bf16", B=2, Hq=8, Hkv=2, D=64, P=[40, 70], N=6, tree="best_first")
    c = make_custom(seed=[1, 3], dtype="bf16", B=2, Hq=8, Hkv=2, D=64, P=[40, 70], N=6, tree="best_first")
    for f in ("q", "k", "v", "parent", "dq"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.k, c.k)


def _rank_sequences(parent, rank):
    seqs = []
    for i in range(1, len(parent)):
        s, a = [], i
        while a > 0:
            s.append(int(rank[a]))
            a = int(parent[a])
        seqs.append(tuple(reversed(s)))
    return seqs


@pytest.mark.parametrize("seed", range(40))
def test_best_first_equals_top_sequences(seed):
    """Best-first expansion by cumulative log-prob keeps exactly the N-1 rank
    sequences with the highest cumulative log-prob (all log-probs are negative,
    so that set is closed under prefixes)."""
    rng = np.random.default_rng(seed)
    n_cand, max_depth = 4, 3
    lp = depth_logprobs(rng, max_depth, n_cand=n_cand)
    allseq = [s for d in range(1, max_depth + 1) for s in itertools.product(range(n_cand), repeat=d)]
    cum = {s: sum(lp[i + 1][r] for i, r in enumerate(s)) for s in allseq}
    N = int(rng.integers(2, len(allseq) + 1))
    parent, depth, rank = best_first_tree(N, lp, max_depth)
    assert parent[0] == -1 and all(0 <= parent[i] < i for i in range(1, N))
    assert depth.max() <= max_depth
    got = set(_rank_sequences(parent, rank))
    want = set(sorted(allseq, key=lambda s: -cum[s])[: N - 1])
    assert got == want


def test_full_size_workloads_shapes():
    w1 = make_workload(1)
    assert w1.q.shape == (1, 5, 4, 64) and w1.q.dtype == np.float32 and w1.k.shape == (517, 1, 64)
    assert w1.k_sel.tolist() == [64] and w1.score_rows.tolist() == [0, 1, 2, 3, 4]
    w3 = make_workload(3)
    assert w3.N == 256 and w3.parent.shape == (1, 256) and w3.score_rows.size == 256
    d = np.zeros(256, int)
    for i in range(1, 256):
        assert 0 <= w3.parent[0, i] < i
        d[i] = d[w3.parent[0, i]] + 1
    assert d.max() <= 8


@pytest.mark.slow
def test_paged_workload_layout():
    w = make_workload(5)
    assert w.B == 16 and w.layout == "paged" and w.page_size == 16
    assert (w.P >= 4096).all() and (w.P <= 65536).all()
    used = w.page_table[w.page_table >= 0]
    assert len(np.unique(used)) == len(used) == w.num_slots // 16     # pages are a permutation of the pool
    assert (w.k_sel == np.maximum(1, w.P // 20)).all()


def test_planted_heavy_keys_rank_high():
    """Soft sanity: planting along the scoring queries' direction makes planted
    keys score high (not a parity check)."""
    w = make_custom(seed=[2, 0], B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=4096, N=8,
                    score_rows="c2q", k_sel=256, heavy_count=40, heavy_c=2.5, window=64, window_c=1.0)
    import oracle
    s = oracle.verify_scores(w.q, "bf16", oracle.KVCache.of(w), w.P, w.score_rows, w.scale, w.Hkv)[0]
    top = set(oracle.topk_select(s, 4096, 256).tolist())
    assert len(top & set(w.heavy.tolist())) >= 36
