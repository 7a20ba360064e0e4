"""Pins of the CPU oracle against things other than itself: hand-derived golden
cases, closed forms, brute force, an independent library routine (torch SDPA in
float64) and invariants.  CPU only."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import KVCache
from workloads import make_custom, make_score_vector
from tests.conftest import load_golden


def f32(x):
    return np.asarray(x, dtype=np.float32)


def torch_bf16_to_f64(x):
    """bfloat16 bit patterns decoded by torch's own bfloat16 type: a decoder
    independent of the oracle's, for the pins that cross-check it."""
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


# ----------------------------------------------------------------------------- storage format

def test_bf16_decoder_format_values():
    """bfloat16 = 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits: values
    the format itself fixes, then every one of the 65536 patterns against torch."""
    fixed = {
        0x3F80: 1.0, 0xC020: -2.5, 0x4049: 3.140625, 0x3E80: 0.25, 0x0000: 0.0, 0x8000: -0.0,
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,      # largest finite
        0x0080: 2.0 ** -126,                         # smallest normal
        0x0001: 2.0 ** -133,                         # smallest subnormal
        0x807F: -(127 / 128) * 2.0 ** -126,          # largest negative subnormal
        0x7F80: np.inf, 0xFF80: -np.inf,
    }
    got = oracle.bf16_bits_to_f64(np.array(list(fixed), dtype=np.uint16))
    for (bits, want), g in zip(fixed.items(), got):
        assert g == want and np.signbit(g) == np.signbit(want), (hex(bits), g, want)
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0, 0xFFC1], dtype=np.uint16))).all()
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    a, b = oracle.bf16_bits_to_f64(every), torch_bf16_to_f64(every)
    nan = np.isnan(b)
    assert (np.isnan(a) == nan).all()
    assert np.array_equal(a[~nan], b[~nan]) and (np.signbit(a[~nan]) == np.signbit(b[~nan])).all()


# ----------------------------------------------------------------------------- golden

def test_golden_attention_three_keys():
    g = load_golden("attention_three_keys.json")
    q = f32(g["q"])[None]                       # [B=1][N][Hq][D]
    k = f32(g["k"])[:, None, :]                 # [slots][Hkv][D]
    v = f32(g["v"])[:, None, :]
    kv = KVCache(k, v, "f32", "contiguous", seq_stride=len(g["k"]))
    P = np.array([g["P"]], dtype=np.int32)
    out = oracle.verify_attention(q, "f32", kv, P, None, g["scale"], 1)
    np.testing.assert_allclose(out[0], np.asarray(g["expect_out"]), rtol=0, atol=2e-6)
    s = oracle.verify_scores(q, "f32", kv, P, [0], g["scale"], 1)
    np.testing.assert_allclose(s[0], g["expect_scores"], rtol=0, atol=2e-6)
    assert oracle.topk_select(s[0], g["P"], g["k_sel"]).tolist() == g["expect_idx"]


def test_golden_tree_uniform():
    g = load_golden("tree_uniform.json")
    parent = np.asarray(g["parent"], dtype=np.int32)
    N, D, P = len(parent), g["D"], g["P"]
    for t, exp in enumerate(g["expect_ancestors"]):
        assert sorted(oracle.ancestors(parent, t)) == exp
    q = np.zeros((1, N, 1, D), dtype=np.float32)
    k = np.ones((P + N, 1, D), dtype=np.float32)
    v = np.zeros((P + N, 1, D), dtype=np.float32)
    for j in range(P + N):
        v[j, 0, j] = 6.0
    kv = KVCache(k, v, "f32", "contiguous", seq_stride=P + N)
    out = oracle.verify_attention(q, "f32", kv, np.array([P], np.int32), parent[None], 0.5, 1)
    np.testing.assert_allclose(out[0, :, 0], np.asarray(g["expect_out"]), rtol=0, atol=1e-12)


def test_golden_scores_small():
    g = load_golden("scores_small.json")
    q = f32(g["q"])[None]
    P, N = g["P"], g["N"]
    k = np.zeros((P + N, 1, g["D"]), dtype=np.float32)
    k[:P, 0] = f32(g["k_prefix"])
    k[P:, 0] = 1e6                               # verify tokens' keys: never scored
    kv = KVCache(k, k, "f32", "contiguous", seq_stride=P + N)
    for case in g["cases"]:
        s = oracle.verify_scores(q, "f32", kv, np.array([P], np.int32), case["rows"], g["scale"], 1)
        np.testing.assert_allclose(s[0], case["expect_scores"], rtol=0, atol=1e-12)
        assert oracle.topk_select(s[0], P, case["k"]).tolist() == case["expect_idx"]


def test_golden_topk_ties():
    g = load_golden("topk_ties.json")
    s = f32(g["scores"])
    for case in g["cases"]:
        assert oracle.topk_select(s, len(s), case["k"]).tolist() == case["expect_idx"], case


def test_golden_sparse_two_keys():
    g = load_golden("sparse_two_keys.json")
    L, D = g["L"], g["D"]
    k = np.tile(f32(g["fill_k"]), (L, 1, 1))
    v = np.tile(f32(g["fill_v"]), (L, 1, 1))
    for p, val in g["k_at"].items():
        k[int(p), 0] = val
    for p, val in g["v_at"].items():
        v[int(p), 0] = val
    kv = KVCache(k, v, "f32", "contiguous", seq_stride=L)
    out = oracle.sparse_draft_attention(f32(g["q"])[None], "f32", kv, [np.array(g["idx"])], g["scale"], 1)
    np.testing.assert_allclose(out[0], np.asarray(g["expect_out"]), rtol=0, atol=2e-6)


# ----------------------------------------------------------------------------- library cross-check

def _reach_mask(parent, N):
    """Ancestor-or-self relation by boolean matrix closure (independent of the oracle's walk)."""
    A = np.eye(N, dtype=bool)
    for i in range(N):
        if parent is None:
            if i > 0:
                A[i, i - 1] = True
        elif parent[i] >= 0:
            A[i, parent[i]] = True
    R = A.copy()
    for _ in range(N):
        R2 = R | ((R.astype(np.int64) @ R.astype(np.int64)) > 0)
        if (R2 == R).all():
            break
        R = R2
    return R   # R[t, a]: a is t or an ancestor of t


def _sdpa_verify(wl, b):
    """torch scaled_dot_product_attention in float64 with an explicit boolean mask."""
    kv = KVCache.of(wl)
    Pb, N, G = int(wl.P[b]), wl.N, wl.Hq // wl.Hkv
    L = Pb + N
    slots = kv.slots(b, np.arange(L))
    to64 = torch_bf16_to_f64 if wl.dtype == "bf16" else (lambda x: x.astype(np.float64))
    K = torch.from_numpy(to64(wl.k[slots])).permute(1, 0, 2)          # [Hkv][L][D]
    V = torch.from_numpy(to64(wl.v[slots])).permute(1, 0, 2)
    K = K.repeat_interleave(G, dim=0)                                 # MHA with repeated K/V
    V = V.repeat_interleave(G, dim=0)
    Q = torch.from_numpy(to64(wl.q[b])).permute(1, 0, 2)              # [Hq][N][D]
    R = _reach_mask(None if wl.parent is None else wl.parent[b], N)
    mask = np.zeros((N, L), dtype=bool)
    mask[:, :Pb] = True
    mask[:, Pb:] = R
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(mask),
                                                         scale=wl.scale)
    return o.permute(1, 0, 2).numpy()                                 # [N][Hq][D]


@pytest.mark.parametrize("case", [
    dict(dtype="f32", B=1, Hq=4, Hkv=1, D=64, P=300, N=5),
    dict(dtype="bf16", B=2, Hq=8, Hkv=2, D=128, P=[200, 333], N=7, tree="best_first", tree_depth=4),
    dict(dtype="bf16", B=1, Hq=4, Hkv=4, D=64, P=100, N=12, tree="best_first", tree_depth=3,
         layout="paged", page_size=16),
    dict(dtype="f32", B=1, Hq=6, Hkv=3, D=64, P=50, N=9, tree="best_first", tree_depth=8, q_std_mult=8.0),
])
def test_verify_matches_torch_sdpa(case):
    wl = make_custom(seed=11, **case)
    out = oracle.verify_attention(wl.q, wl.dtype, KVCache.of(wl), wl.P, wl.parent, wl.scale, wl.Hkv)
    for b in range(wl.B):
        np.testing.assert_allclose(out[b], _sdpa_verify(wl, b), rtol=1e-10, atol=1e-12)


def test_chain_equals_triangular_mask():
    wl = make_custom(seed=3, dtype="f32", Hq=2, Hkv=1, D=64, P=40, N=6, q_std_mult=10.0)
    kv = KVCache.of(wl)
    out = oracle.verify_attention(wl.q, "f32", kv, wl.P, None, wl.scale, 1)
    # separately written causal mask: row t sees positions <= P + t
    L = int(wl.P[0]) + wl.N
    K = kv.keys(0, 0, np.arange(L))
    V = kv.values(0, 0, np.arange(L))
    tri = np.tril(np.ones((wl.N, wl.N), dtype=bool))
    for t in range(wl.N):
        vis = np.concatenate([np.ones(int(wl.P[0]), bool), tri[t]])
        for h in range(2):
            lg = wl.scale * (K[vis] @ wl.q[0, t, h].astype(np.float64))
            w = np.exp(lg - lg.max())
            np.testing.assert_allclose(out[0, t, h], (w / w.sum()) @ V[vis], rtol=1e-12, atol=1e-14)
    # the same chain written as an explicit parent array gives the same result
    out2 = oracle.verify_attention(wl.q, "f32", kv, wl.P, np.arange(-1, wl.N - 1)[None], wl.scale, 1)
    np.testing.assert_array_equal(out, out2)


# ----------------------------------------------------------------------------- closed forms / invariants

@pytest.mark.parametrize("case", [
    dict(dtype="bf16", B=2, Hq=8, Hkv=2, D=64, P=[97, 130], N=6, score_rows=[0, 5]),
    dict(dtype="f32", B=1, Hq=4, Hkv=1, D=64, P=77, N=5, score_rows="all"),
    dict(dtype="bf16", B=1, Hq=8, Hkv=4, D=128, P=64, N=10, tree="best_first", score_rows=[1, 3, 4]),
])
def test_scores_closed_form(case):
    """The sum of logits over rows and heads is linear in q: s_i = scale * sum_g K_g[i] . qbar_g."""
    wl = make_custom(seed=5, **case)
    s = oracle.verify_scores(wl.q, wl.dtype, KVCache.of(wl), wl.P, wl.score_rows, wl.scale, wl.Hkv)
    G = wl.Hq // wl.Hkv
    q = torch_bf16_to_f64(wl.q) if wl.dtype == "bf16" else wl.q.astype(np.float64)
    kall = torch_bf16_to_f64(wl.k) if wl.dtype == "bf16" else wl.k.astype(np.float64)
    for b in range(wl.B):
        Pb = int(wl.P[b])
        qbar = q[b][wl.score_rows].reshape(len(wl.score_rows), wl.Hkv, G, wl.D).sum(axis=(0, 2))
        Kb = kall[b * wl.seq_stride: b * wl.seq_stride + Pb]          # [Pb][Hkv][D]
        ref = wl.scale * np.einsum("igd,gd->i", Kb, qbar)
        np.testing.assert_allclose(s[b, :Pb], ref, rtol=1e-10, atol=1e-12)
        assert np.isnan(s[b, Pb:]).all()
    # the grouped oracle routine (used for full-size checks) is the same sum
    sg = oracle.verify_scores_grouped(wl.q, wl.dtype, KVCache.of(wl), wl.P, wl.score_rows, wl.scale, wl.Hkv)
    np.testing.assert_allclose(sg, s, rtol=1e-10, atol=1e-12)


def test_scores_linear_in_rows_and_c2q_subset():
    wl = make_custom(seed=9, dtype="bf16", Hq=8, Hkv=2, D=64, P=150, N=8)
    kv = KVCache.of(wl)
    f = lambda rows: oracle.verify_scores(wl.q, "bf16", kv, wl.P, rows, wl.scale, 2)  # noqa: E731
    full = f(list(range(8)))
    parts = sum(f([t]) for t in range(8))
    np.testing.assert_allclose(full, parts, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f([0, 7]), f([0]) + f([7]), rtol=1e-10, atol=1e-12)


def test_softmax_rows_sum_to_one():
    wl = make_custom(seed=2, dtype="f32", Hq=4, Hkv=2, D=64, P=60, N=7, tree="best_first", q_std_mult=5.0)
    wl.v[:] = 1.0
    out = oracle.verify_attention(wl.q, "f32", KVCache.of(wl), wl.P, wl.parent, wl.scale, 2)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)
    dr = oracle.sparse_draft_attention(wl.dq[0], "f32", KVCache.of(wl), [np.arange(30)], wl.scale, 2)
    np.testing.assert_allclose(dr, 1.0, rtol=0, atol=1e-13)


def test_single_node_equals_decode_and_full_index_set():
    """N = 1 verification is plain decode over prefix + self; the sparse draft
    over every position reproduces it exactly (k = whole context == dense)."""
    wl = make_custom(seed=4, dtype="bf16", B=2, Hq=8, Hkv=2, D=64, P=[120, 75], N=1, q_std_mult=4.0)
    kv = KVCache.of(wl)
    out = oracle.verify_attention(wl.q, "bf16", kv, wl.P, None, wl.scale, 2)
    idx = [np.arange(int(wl.P[b]) + 1) for b in range(2)]
    dr = oracle.sparse_draft_attention(wl.q[:, 0], "bf16", kv, idx, wl.scale, 2)
    np.testing.assert_allclose(out[:, 0], dr, rtol=1e-12, atol=1e-14)


def test_star_tree_is_prefix_root_self():
    N = 6
    star = np.array([-1] + [0] * (N - 1), dtype=np.int32)
    wl = make_custom(seed=6, dtype="f32", Hq=2, Hkv=1, D=64, P=30, N=N, tree=star, q_std_mult=6.0)
    kv = KVCache.of(wl)
    out = oracle.verify_attention(wl.q, "f32", kv, wl.P, wl.parent, wl.scale, 1)
    P = int(wl.P[0])
    for t in range(N):
        idx = np.concatenate([np.arange(P + 1), [P + t]]) if t else np.arange(P + 1)
        dr = oracle.sparse_draft_attention(wl.q[:, t], "f32", kv, [idx], wl.scale, 1)
        np.testing.assert_allclose(out[0, t], dr[0], rtol=1e-12, atol=1e-14)


def test_sparse_permutation_invariance_and_dense_prefix():
    wl = make_custom(seed=8, dtype="bf16", Hq=8, Hkv=2, D=128, P=200, N=3, q_std_mult=5.0)
    kv = KVCache.of(wl)
    rng = np.random.default_rng(0)
    idx = np.sort(rng.choice(200, 40, replace=False))
    a = oracle.sparse_draft_attention(wl.dq[0], "bf16", kv, [idx], wl.scale, 2)
    b = oracle.sparse_draft_attention(wl.dq[0], "bf16", kv, [rng.permutation(idx)], wl.scale, 2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    # every prefix position selected == dense decode over the prefix (torch SDPA)
    full = oracle.sparse_draft_attention(wl.dq[0], "bf16", kv, [np.arange(200)], wl.scale, 2)
    K = torch.from_numpy(torch_bf16_to_f64(wl.k[:200])).permute(1, 0, 2).repeat_interleave(4, 0)
    V = torch.from_numpy(torch_bf16_to_f64(wl.v[:200])).permute(1, 0, 2).repeat_interleave(4, 0)
    Q = torch.from_numpy(torch_bf16_to_f64(wl.dq[0, 0]))[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=wl.scale)[:, 0].numpy()
    np.testing.assert_allclose(full[0], ref, rtol=1e-10, atol=1e-13)
    # empty index list gives zeros
    z = oracle.sparse_draft_attention(wl.dq[0], "bf16", kv, [np.arange(0)], wl.scale, 2)
    assert (z == 0).all()


def test_gqa_equals_mha_with_repeated_kv():
    wl = make_custom(seed=12, dtype="bf16", B=1, Hq=8, Hkv=2, D=64, P=90, N=6, tree="best_first",
                     q_std_mult=4.0)
    kv = KVCache.of(wl)
    out = oracle.verify_attention(wl.q, "bf16", kv, wl.P, wl.parent, wl.scale, 2)
    k_rep = np.repeat(wl.k, 4, axis=1)
    v_rep = np.repeat(wl.v, 4, axis=1)
    kv2 = KVCache(k_rep, v_rep, "bf16", "contiguous", wl.seq_stride)
    out2 = oracle.verify_attention(wl.q, "bf16", kv2, wl.P, wl.parent, wl.scale, 8)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-15)
    s1 = oracle.verify_scores(wl.q, "bf16", kv, wl.P, wl.score_rows, wl.scale, 2)
    s2 = oracle.verify_scores(wl.q, "bf16", kv2, wl.P, wl.score_rows, wl.scale, 8)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-14)


def test_paged_equals_contiguous():
    wl = make_custom(seed=13, dtype="bf16", B=3, Hq=4, Hkv=2, D=64, P=[50, 17, 80], N=5, tree="best_first")
    kv = KVCache.of(wl)
    # scatter the same logical tokens into a shuffled paged pool (written here, not by the generator)
    ps = 8
    rng = np.random.default_rng(1)
    L = wl.P + wl.N
    npg = (L + ps - 1) // ps
    perm = rng.permutation(int(npg.sum()))
    pt = np.full((3, int(npg.max())), -1, np.int32)
    off = 0
    kp = np.zeros((int(npg.sum()) * ps, 2, 64), np.uint16)
    vp = np.zeros_like(kp)
    for b in range(3):
        pt[b, :npg[b]] = perm[off: off + npg[b]]
        off += npg[b]
        pos = np.arange(L[b])
        sl = pt[b][pos // ps].astype(np.int64) * ps + pos % ps
        kp[sl] = wl.k[b * wl.seq_stride + pos]
        vp[sl] = wl.v[b * wl.seq_stride + pos]
    kv2 = KVCache(kp, vp, "bf16", "paged", page_size=ps, page_table=pt)
    o1 = oracle.verify_attention(wl.q, "bf16", kv, wl.P, wl.parent, wl.scale, 2)
    o2 = oracle.verify_attention(wl.q, "bf16", kv2, wl.P, wl.parent, wl.scale, 2)
    np.testing.assert_array_equal(o1, o2)
    s1 = oracle.verify_scores(wl.q, "bf16", kv, wl.P, wl.score_rows, wl.scale, 2)
    s2 = oracle.verify_scores(wl.q, "bf16", kv2, wl.P, wl.score_rows, wl.scale, 2)
    np.testing.assert_array_equal(s1, s2)


# ----------------------------------------------------------------------------- selection brute force

def _brute_topk(s, k):
    """Explicit argmax over all k-subsets of the summed score (Vegas §2.A);
    among maximisers, the lexicographically smallest ascending tuple."""
    best, best_t = None, None
    for t in itertools.combinations(range(len(s)), k):
        v = sum(float(s[i]) for i in t)
        if best is None or v > best:
            best, best_t = v, t
    return list(best_t) if best_t is not None else []


@pytest.mark.parametrize("seed", range(30))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 13))
    # integer-valued scores force exact ties; sums of integers are exact in float64
    s = rng.integers(-3, 4, size=n).astype(np.float32)
    for k in range(0, min(n, 5) + 1):
        assert oracle.topk_select(s, n, k).tolist() == _brute_topk(s, k), (s, k)


def test_topk_clamps_and_prefix_only():
    s = make_score_vector(3, 50, "normal")
    s[40:] = 1e9                      # entries past P_b must be ignored
    got = oracle.topk_select(s, 40, 100)
    assert got.tolist() == list(range(40))
    got = oracle.topk_select(s, 40, 5)
    assert len(got) == 5 and got.max() < 40 and (np.diff(got) > 0).all()


def test_topk_signed_zero_and_wide():
    s = make_score_vector(4, 200, "signed_zero")
    got = oracle.topk_select(s, 200, 60)
    # -0.0 and +0.0 tie: among zeros the lowest indices are taken regardless of sign
    order = sorted(range(200), key=lambda i: (-float(s[i]), i))
    assert got.tolist() == sorted(order[:60])
    s = make_score_vector(5, 300, "wide")
    got = oracle.topk_select(s, 300, 17)
    thr = np.sort(s)[::-1][16]
    assert (s[got] >= thr).all() and len(got) == 17


# ----------------------------------------------------------------------------- compacted draft loop

def _tail_cache(wl, tail_k, tail_v, steps):
    """Copy of the cache with tail row t of sequence b at logical position P_b + N + t."""
    k2, v2 = wl.k.copy(), wl.v.copy()
    kv = KVCache.of(wl)
    for b in range(wl.B):
        sl = kv.slots(b, int(wl.P[b]) + wl.N + np.arange(steps))
        k2[sl] = tail_k[:steps, b]
        v2[sl] = tail_v[:steps, b]
    return KVCache(k2, v2, wl.dtype, wl.layout, wl.seq_stride, wl.page_size, wl.page_table)


@pytest.mark.parametrize("dtype,layout", [("bf16", "contiguous"), ("f32", "paged")])
def test_compacted_draft_equals_sparse_list(dtype, layout):
    """Rows gathered once and attended densely == the sparse step over the same
    list (the pinned sparse_draft_attention), with and without a tail."""
    from workloads import make_tail_rows
    wl = make_custom(seed=21, dtype=dtype, B=2, Hq=8, Hkv=2, D=64, P=[150, 90], N=3, q_std_mult=4.0,
                     layout=layout, page_size=16, seq_extra=8)
    kv = KVCache.of(wl)
    rng = np.random.default_rng(3)
    idx = [np.sort(rng.choice(int(wl.P[b]), n, replace=False)) for b, n in enumerate((40, 17))]
    n = [len(x) for x in idx]
    cap = 48
    ck, cv = oracle.compact_kv(kv, idx, cap)
    assert (ck[1, 17:] == 0).all() and (cv[0, 40:] == 0).all()
    a = oracle.dense_draft_attention(wl.dq[0], dtype, ck, cv, n, wl.scale, 2)
    b = oracle.sparse_draft_attention(wl.dq[0], dtype, kv, idx, wl.scale, 2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    # a tail of s drafted tokens behind the set == those rows past the prefix, listed
    tail_k, tail_v = make_tail_rows(5, 4, wl.B, 2, 64, dtype)
    for s in (1, 2, 4):
        ck2, cv2 = ck.copy(), cv.copy()
        for bb in range(wl.B):
            ck2[bb, n[bb]: n[bb] + s] = tail_k[:s, bb]
            cv2[bb, n[bb]: n[bb] + s] = tail_v[:s, bb]
        dense = oracle.dense_draft_attention(wl.dq[0], dtype, ck2, cv2, [x + s for x in n], wl.scale, 2)
        kv2 = _tail_cache(wl, tail_k, tail_v, s)
        idx2 = [np.concatenate([idx[bb], int(wl.P[bb]) + wl.N + np.arange(s)]) for bb in range(wl.B)]
        sparse = oracle.sparse_draft_attention(wl.dq[0], dtype, kv2, idx2, wl.scale, 2)
        np.testing.assert_allclose(dense, sparse, rtol=1e-12, atol=1e-15)


def test_dense_draft_single_row_permutation_and_empty():
    wl = make_custom(seed=22, dtype="bf16", B=2, Hq=8, Hkv=2, D=128, P=120, N=2, q_std_mult=4.0)
    kv = KVCache.of(wl)
    idx = [np.arange(0, 120, 3), np.arange(5, 60)]
    ck, cv = oracle.compact_kv(kv, idx, 64)
    # one row: softmax over a single logit is 1, so the output is that row's V exactly
    one = oracle.dense_draft_attention(wl.dq[0], "bf16", ck, cv, [1, 1], wl.scale, 2)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(one[b, h], torch_bf16_to_f64(cv[b, 0, h // 4]))
    # rows in another order give the same output
    n = [40, 55]
    base = oracle.dense_draft_attention(wl.dq[0], "bf16", ck, cv, n, wl.scale, 2)
    rng = np.random.default_rng(1)
    ckp, cvp = ck.copy(), cv.copy()
    for b in range(2):
        perm = rng.permutation(n[b])
        ckp[b, : n[b]] = ck[b, perm]
        cvp[b, : n[b]] = cv[b, perm]
    np.testing.assert_allclose(oracle.dense_draft_attention(wl.dq[0], "bf16", ckp, cvp, n, wl.scale, 2), base,
                               rtol=1e-12, atol=1e-15)
    # no rows: zero output
    z = oracle.dense_draft_attention(wl.dq[0], "bf16", ck, cv, [0, 0], wl.scale, 2)
    assert (z == 0).all()


# ----------------------------------------------------------------------------- acceptance

def _branch_matched(parent, draft, target, v):
    """Every edge on node v's root branch carries the target's token."""
    while v != 0:
        p = (v - 1) if parent is None else int(parent[v])
        if int(draft[v]) != int(target[p]):
            return False
        v = p
    return True


@pytest.mark.parametrize("seed", range(12))
def test_greedy_accept_brute_force(seed):
    """On trees whose siblings carry distinct tokens, the accepted path is the
    root branch of the deepest node whose whole branch matches (brute force
    over every node); on chains, the leading run of matches."""
    from workloads import best_first_tree, depth_logprobs, make_accept_tokens
    rng = np.random.default_rng(seed)
    N = int(rng.integers(2, 80))
    parent = best_first_tree(N, depth_logprobs(rng, 6), 6)[0][None]
    draft, target = make_accept_tokens(seed, parent, match_prob=float(rng.uniform(0.3, 1.0)))
    path = oracle.greedy_accept(parent[0], draft[0], target[0])
    matched = [v for v in range(N) if _branch_matched(parent[0], draft[0], target[0], v)]
    deepest = max(matched, key=lambda v: (len(oracle.ancestors(parent[0], v)), -v))
    assert path == sorted(oracle.ancestors(parent[0], deepest))
    # chain: leading matches
    chain = np.arange(-1, N - 1, dtype=np.int32)[None]
    d2, t2 = make_accept_tokens(seed + 100, chain, match_prob=0.8)
    n_lead = 0
    while n_lead + 1 < N and d2[0, n_lead + 1] == t2[0, n_lead]:
        n_lead += 1
    assert oracle.greedy_accept(None, d2[0], t2[0]) == list(range(n_lead + 1))
    assert oracle.greedy_accept(chain[0], d2[0], t2[0]) == list(range(n_lead + 1))


def test_greedy_accept_golden():
    # root 0 -> {1, 2}; 1 -> {3}; 2 -> {4, 5}.  Target after 0 is token 20 (node 2),
    # after 2 is 51 (node 5), after 5 nothing matches.
    parent = np.array([-1, 0, 0, 1, 2, 2])
    draft = np.array([7, 10, 20, 30, 50, 51])
    target = np.array([20, 30, 51, 0, 0, 99])
    assert oracle.greedy_accept(parent, draft, target) == [0, 2, 5]
    # nothing accepted: the path is the root alone
    assert oracle.greedy_accept(parent, draft, np.array([5, 0, 0, 0, 0, 0])) == [0]


def test_commit_accepted_kv_moves_only_the_path():
    wl = make_custom(seed=31, dtype="bf16", B=2, Hq=4, Hkv=2, D=64, P=[40, 25], N=8)
    kv = KVCache.of(wl)
    k0, v0 = wl.k.copy(), wl.v.copy()
    path = [0, 2, 5, 7]
    oracle.commit_accepted_kv(kv, 1, 25, path)
    for d in range(1, 4):
        assert np.array_equal(wl.k[kv.slots(1, [25 + d])], k0[kv.slots(1, [25 + path[d]])])
        assert np.array_equal(wl.v[kv.slots(1, [25 + d])], v0[kv.slots(1, [25 + path[d]])])
    moved = set(kv.slots(1, 25 + np.arange(1, 4)).tolist())
    other = [s for s in range(wl.k.shape[0]) if s not in moved]
    assert np.array_equal(wl.k[other], k0[other]) and np.array_equal(wl.v[other], v0[other])


# ----------------------------------------------------------------------------- tree construction

def _all_nodes(lp, max_depth):
    """Every node reachable within the depth limit: (score, rank path)."""
    out = []

    def rec(path, score):
        d = len(path)
        if d == max_depth:
            return
        for r in range(lp.shape[1]):
            sc = score + lp[d + 1][r]
            out.append((sc, path + (r,)))
            rec(path + (r,), sc)
    rec((), 0.0)
    return out


@pytest.mark.parametrize("seed", range(10))
def test_best_first_tree_brute_force(seed):
    """Node i (i >= 1) is the i-th best of all reachable nodes (scores are
    continuous, so there are no ties), and its parent is the node of the same
    rank path minus its last step."""
    rng = np.random.default_rng(seed)
    n_cand, max_depth = int(rng.integers(2, 5)), int(rng.integers(1, 4))
    lp = np.zeros((max_depth + 1, n_cand))
    for d in range(1, max_depth + 1):
        z = rng.normal(0, np.sqrt(2), n_cand)
        lp[d] = np.sort(z - np.log(np.exp(z).sum()))[::-1]
    allnodes = sorted(_all_nodes(lp, max_depth), key=lambda x: -x[0])
    n = int(rng.integers(1, min(len(allnodes) + 1, 40) + 1))
    parent, depth, rank = oracle.build_best_first_tree(lp, n, max_depth)
    paths = {(): 0}
    for i in range(1, n):
        sc, path = allnodes[i - 1]
        paths[path] = i
        assert parent[i] == paths[path[:-1]], f"node {i}"
        assert depth[i] == len(path) and rank[i] == path[-1]


def test_best_first_tree_golden_ties_and_generator():
    # two candidate lists with equal entries: ties go to the lower parent id, then the lower rank
    lp = np.array([[0.0, 0.0], [-1.0, -1.0], [-1.0, -2.0]])
    parent, depth, rank = oracle.build_best_first_tree(lp, 5, 2)
    # root -> (0, r0) -1 -> (0, r1) -1 [tie: lower rank first] -> child of node 1 r0: -2, child of node 2 r0: -2
    assert parent.tolist() == [-1, 0, 0, 1, 2] and rank.tolist() == [0, 0, 1, 0, 0] and depth.tolist() == [0, 1, 1, 2, 2]
    # the input generator's trees (configs 3 and 5 shapes) are the same trees
    from workloads import best_first_tree, depth_logprobs
    for seed, n, dmax in ((1, 256, 8), (2, 64, 6), (3, 100, 3)):
        lpg = depth_logprobs(np.random.default_rng(seed), dmax)
        g = best_first_tree(n, lpg, dmax)
        o = oracle.build_best_first_tree(lpg, n, dmax)
        for a, b in zip(g, o):
            assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- selection variants

def test_per_head_scores_sum_to_the_total():
    wl = make_custom(seed=41, dtype="bf16", B=2, Hq=8, Hkv=2, D=64, P=[90, 57], N=4, score_rows="all")
    kv = KVCache.of(wl)
    ph = oracle.verify_scores_per_head(wl.q, "bf16", kv, wl.P, wl.score_rows, wl.scale, 2)
    tot = oracle.verify_scores(wl.q, "bf16", kv, wl.P, wl.score_rows, wl.scale, 2)
    np.testing.assert_allclose(ph.sum(axis=1), tot, rtol=1e-12, atol=1e-12, equal_nan=True)
    # one KV head: the per-head score is the total
    wl1 = make_custom(seed=42, dtype="f32", B=1, Hq=4, Hkv=1, D=64, P=70, N=3, score_rows=[0, 2])
    kv1 = KVCache.of(wl1)
    np.testing.assert_allclose(oracle.verify_scores_per_head(wl1.q, "f32", kv1, wl1.P, wl1.score_rows, wl1.scale, 1)[:, 0],
                               oracle.verify_scores(wl1.q, "f32", kv1, wl1.P, wl1.score_rows, wl1.scale, 1),
                               rtol=1e-12, atol=1e-12, equal_nan=True)


def test_per_head_draft_with_shared_lists_is_the_shared_step():
    wl = make_custom(seed=43, dtype="bf16", B=2, Hq=8, Hkv=2, D=64, P=[120, 80], N=2, q_std_mult=4.0)
    kv = KVCache.of(wl)
    rng = np.random.default_rng(2)
    idx = [np.sort(rng.choice(int(wl.P[b]), 30, replace=False)) for b in range(2)]
    a = oracle.sparse_draft_attention_per_head(wl.dq[0], "bf16", kv, [[i, i] for i in idx], wl.scale, 2)
    b = oracle.sparse_draft_attention(wl.dq[0], "bf16", kv, idx, wl.scale, 2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    # different lists per head: head group g sees only its own list
    other = [np.sort(rng.choice(int(wl.P[b]), 12, replace=False)) for b in range(2)]
    c = oracle.sparse_draft_attention_per_head(wl.dq[0], "bf16", kv, [[idx[b], other[b]] for b in range(2)],
                                               wl.scale, 2)
    d = oracle.sparse_draft_attention(wl.dq[0], "bf16", kv, other, wl.scale, 2)
    np.testing.assert_allclose(c[:, :4], b[:, :4], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(c[:, 4:], d[:, 4:], rtol=1e-12, atol=1e-15)


def test_sink_window_select_by_hand():
    assert oracle.sink_window_select(10, 2, 3).tolist() == [0, 1, 7, 8, 9]
    assert oracle.sink_window_select(4, 2, 3).tolist() == [0, 1, 2, 3]      # overlap
    assert oracle.sink_window_select(0, 2, 3).tolist() == []
    assert oracle.sink_window_select(100, 0, 5).tolist() == [95, 96, 97, 98, 99]


# ---- tokens per time (KnapSpec §2 TPT metric)

def test_tpt_closed_forms_and_series():
    """alpha = 0: one token per round; alpha = 1: gamma + 1 tokens (the
    limit); gamma = 0: one token per target pass; otherwise the token factor
    is the explicit sum of alpha^i over i = 0..gamma."""
    assert oracle.tpt(0.0, 7, 3.0, 50.0) == pytest.approx(1.0 / (7 * 3.0 + 50.0), rel=1e-15)
    assert oracle.tpt(1.0, 7, 3.0, 50.0) == pytest.approx(8.0 / (7 * 3.0 + 50.0), rel=1e-15)
    assert oracle.tpt(0.7, 0, 3.0, 50.0) == pytest.approx(1.0 / 50.0, rel=1e-15)
    for alpha in (0.1, 0.5, 0.8, 0.95, 0.999999):
        for gamma in (1, 3, 7, 15):
            tokens = sum(alpha ** i for i in range(gamma + 1))
            assert oracle.tpt(alpha, gamma, 2.5, 40.0) == pytest.approx(tokens / (gamma * 2.5 + 40.0), rel=1e-9)
    # more acceptance never lowers the rate; a slower draft always lowers it
    assert oracle.tpt(0.9, 7, 3.0, 50.0) > oracle.tpt(0.8, 7, 3.0, 50.0)
    assert oracle.tpt(0.8, 7, 4.0, 50.0) < oracle.tpt(0.8, 7, 3.0, 50.0)
