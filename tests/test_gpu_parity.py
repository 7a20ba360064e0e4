"""GPU parity: the HIP path (through the C ABI binding) against the CPU oracle,
element by element, on seeded inputs small enough for the oracle but spanning
several tiles, chunks and ragged tails, plus the edge cases of the method."""
import numpy as np
import pytest
import torch

import oracle
from oracle import KVCache as OKV
from workloads import make_custom, make_score_vector, make_workload
from tests.gpu_util import (DevWorkload, as_f64, attention_abs, check_out, check_out_derived, check_scores,
                            check_selection_band, i32, score_floor, sparse_abs, to_torch)

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


CASES = {
    "cfg1_full": lambda: make_workload(1),
    "chain8_c2q_bf16_ragged": lambda: make_custom(
        seed=101, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=3001, N=8, score_rows="c2q", k_sel=200,
        heavy_count=30, heavy_c=2.5, window=64, window_c=1.0),
    "chain8_bf16_d64_sharp": lambda: make_custom(
        seed=102, B=1, Hq=16, Hkv=4, D=64, dtype="bf16", P=2222, N=8, score_rows="all", k_sel=100, q_std_mult=8.0),
    "tree256_bf16": lambda: make_custom(
        seed=103, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=777, N=256, tree="best_first", tree_depth=8,
        score_rows="all", k_sel=100, decode_steps=0),
    "tree37_canary": lambda: make_custom(
        seed=104, B=1, Hq=8, Hkv=2, D=128, dtype="bf16", P=1234, N=37, tree="best_first", tree_depth=5,
        score_rows=[0, 3, 36], k_sel=50, q_std_mult=4.0, v_canary=4.0),
    "batch4_chain16": lambda: make_custom(
        seed=105, B=4, Hq=32, Hkv=8, D=128, dtype="bf16", P=[2000, 1500, 3333, 17], N=16, score_rows="c2q",
        k_sel=300, decode_steps=2),
    "paged5_tree64": lambda: make_custom(
        seed=106, B=5, Hq=32, Hkv=8, D=128, dtype="bf16", P=[100, 2500, 999, 40, 3000], N=64, tree="best_first",
        tree_depth=6, score_rows="all", k_sel="5pct", layout="paged", page_size=16),
    "gqa3_d64": lambda: make_custom(
        seed=107, B=2, Hq=12, Hkv=4, D=64, dtype="bf16", P=[700, 301], N=5, score_rows="all", k_sel=64,
        seq_extra=13),
    "mha_f32_d128": lambda: make_custom(
        seed=108, B=1, Hq=8, Hkv=8, D=128, dtype="f32", P=300, N=3, score_rows="all", k_sel=30, q_std_mult=3.0),
    "f32_tree_d64": lambda: make_custom(
        seed=109, B=2, Hq=4, Hkv=1, D=64, dtype="f32", P=[513, 64], N=20, tree="best_first", tree_depth=4,
        score_rows="all", k_sel=40, q_std_mult=5.0, v_canary=2.0),
    "single_node": lambda: make_custom(
        seed=110, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=500, N=1, score_rows="all", k_sel=16),
    "empty_prefix": lambda: make_custom(
        seed=111, B=2, Hq=8, Hkv=2, D=128, dtype="bf16", P=[0, 5], N=4, score_rows="all", k_sel=10),
    "no_scores": lambda: make_custom(
        seed=112, B=1, Hq=8, Hkv=2, D=128, dtype="bf16", P=900, N=6, score_rows=[], k_sel=10, decode_steps=0),
    # head_dim 64 tree kernel (96 rows per KV head), paged, ragged prefixes
    "tree24_bf16_d64_paged": lambda: make_custom(
        seed=113, B=3, Hq=16, Hkv=4, D=64, dtype="bf16", P=[1500, 77, 640], N=24, tree="best_first",
        tree_depth=5, score_rows="all", k_sel=60, layout="paged", page_size=16),
    # small trees on the streaming kernel: 48 and 64 rows per KV head (two row tiles)
    "tree12_stream_g4": lambda: make_custom(
        seed=114, B=2, Hq=16, Hkv=4, D=128, dtype="bf16", P=[2100, 513], N=12, tree="best_first",
        tree_depth=4, score_rows="c2q", k_sel=90),
    "tree64_stream_mha": lambda: make_custom(
        seed=115, B=1, Hq=4, Hkv=4, D=128, dtype="bf16", P=1900, N=64, tree="best_first", tree_depth=6,
        score_rows="all", k_sel=120),
    # mask canaries at full tree width: ancestor-set words 2..7 (nodes >= 64), a
    # prefix over three 2048-key tree chunks, sharpened queries, distinct large V
    # rows on the verify tokens (a one-key leak moves outputs far past the bound)
    "tree256_canary": lambda: make_custom(
        seed=116, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=5000, N=256, tree="best_first", tree_depth=8,
        score_rows="all", k_sel=200, decode_steps=0, q_std_mult=4.0, v_canary=32.0),
    "paged_tree64_canary": lambda: make_custom(
        seed=117, B=3, Hq=32, Hkv=8, D=128, dtype="bf16", P=[3000, 900, 4500], N=64, tree="best_first",
        tree_depth=6, score_rows="all", k_sel="5pct", layout="paged", page_size=16, q_std_mult=4.0,
        v_canary=32.0),
    # page sizes other than 16: one token per page, and a size that is not a
    # power of two (the division path), on the streaming and the tree kernels
    "chain8_paged_ps1": lambda: make_custom(
        seed=118, B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[2500, 700], N=8, score_rows="c2q", k_sel=100,
        layout="paged", page_size=1, q_std_mult=4.0),
    "chain8_paged_ps24": lambda: make_custom(
        seed=119, B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[2500, 701], N=8, score_rows="c2q", k_sel=100,
        layout="paged", page_size=24, q_std_mult=4.0),
    "tree64_paged_ps1": lambda: make_custom(
        seed=120, B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[2100, 333], N=64, tree="best_first", tree_depth=6,
        score_rows="all", k_sel=64, layout="paged", page_size=1, q_std_mult=4.0, v_canary=8.0),
    "tree64_paged_ps24": lambda: make_custom(
        seed=121, B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[2100, 333], N=64, tree="best_first", tree_depth=6,
        score_rows="all", k_sel=64, layout="paged", page_size=24, q_std_mult=4.0, v_canary=8.0),
    # head_dim 64 tree kernel with two row blocks per KV head (400 rows): the
    # prefix stages' scores alternate between the row blocks (eight keys per
    # wave, eight lanes per key), with a subset of scoring rows
    "tree100_bf16_d64_rb2": lambda: make_custom(
        seed=123, B=1, Hq=16, Hkv=4, D=64, dtype="bf16", P=3001, N=100, tree="best_first", tree_depth=7,
        score_rows=[0, 5, 17, 42, 99], k_sel=150, q_std_mult=3.0),
    "f32_chain_paged_ps24": lambda: make_custom(
        seed=122, B=2, Hq=8, Hkv=2, D=64, dtype="f32", P=[900, 250], N=5, score_rows="all", k_sel=40,
        layout="paged", page_size=24, q_std_mult=4.0),
}


def _oracle(wl, with_attention=True):
    kv = OKV.of(wl)
    res = {}
    if with_attention:
        res["out"] = oracle.verify_attention(wl.q, wl.dtype, kv, wl.P, wl.parent, wl.scale, wl.Hkv)
    if len(wl.score_rows):
        res["scores"] = oracle.verify_scores(wl.q, wl.dtype, kv, wl.P, wl.score_rows, wl.scale, wl.Hkv, wl.P_max)
        res["idx"] = [oracle.topk_select(res["scores"][b], int(wl.P[b]), int(wl.k_sel[b])) for b in range(wl.B)]
    return res


@pytest.mark.parametrize("name", list(CASES))
def test_verify_and_step_parity(name):
    print(f"[case] {name}", flush=True)
    check_workload(CASES[name]())


def check_workload(wl):
    """Verification outputs, scores, the selection and the draft steps of one
    workload against the oracle."""
    dw = DevWorkload(wl)
    ref = _oracle(wl)
    out, scores = dw.verify()
    torch.cuda.synchronize()
    check_out(as_f64(out), ref["out"], wl.dtype, "verify out")
    if wl.dtype == "bf16":
        check_out_derived(as_f64(out), ref["out"], attention_abs(wl), "verify", "verify out")
    if not len(wl.score_rows):
        assert scores is None
        return
    worst, by_floor = check_scores(as_f64(scores), ref["scores"], wl.P, score_floor(wl))
    print(f"  scores: worst relative error {worst:.2e}, {by_floor} entries within the fp32 floor only", flush=True)
    idx, count = sv.topk_select(scores, dw.P, dw.k_sel, wl.k_max)
    gi = idx.cpu().numpy()
    kk = np.minimum(wl.k_sel, wl.P)
    assert (count.cpu().numpy() == kk).all()
    check_selection_band(gi, ref["scores"], ref["idx"], wl.P, wl.k_sel)
    for s in range(wl.dq.shape[0]):
        # draft attention over the oracle's selected set (an input from the oracle side)
        oi = np.full((wl.B, max(1, wl.k_max)), -1, np.int32)
        for b in range(wl.B):
            oi[b, : len(ref["idx"][b])] = ref["idx"][b]
        n = np.array([len(x) for x in ref["idx"]], np.int32)
        d = sv.sparse_draft_attn(dw.dq[s], dw.kv, i32(oi), i32(n), max_idx=max(1, wl.k_max))
        dref = oracle.sparse_draft_attention(wl.dq[s], wl.dtype, OKV.of(wl), ref["idx"], wl.scale, wl.Hkv)
        check_out(as_f64(d), dref, wl.dtype, f"draft step {s}")
        if wl.dtype == "bf16":
            check_out_derived(as_f64(d), dref, sparse_abs(wl, wl.dq[s], ref["idx"]), "sparse", f"draft step {s}")


def test_page_table_longer_than_the_cached_slice():
    """One token per page and over a million positions: a verify chunk spans
    more pages than its LDS copy of the page table holds, and the pages past
    it are read from memory.  Sampled rows against the oracle, every score."""
    print("[case] paged ps=1, P=1050000", flush=True)
    wl = make_custom(seed=130, B=1, Hq=4, Hkv=1, D=64, dtype="bf16", P=1_050_000, N=4, score_rows="all",
                     k_sel=64, decode_steps=0, layout="paged", page_size=1, q_std_mult=4.0)
    dw = DevWorkload(wl)
    out, scores = dw.verify()
    torch.cuda.synchronize()
    rows = [(0, t, h) for t in (0, 3) for h in range(4)]
    ref = oracle.verify_attention(wl.q, wl.dtype, OKV.of(wl), wl.P, None, wl.scale, wl.Hkv, rows=rows)
    got = as_f64(out)
    ab = attention_abs(wl, rows=rows)
    for (b, t, h) in rows:
        check_out(got[b, t, h], ref[b, t, h], "bf16", f"verify out t={t} h={h}")
        check_out_derived(got[b, t, h], ref[b, t, h], ab[b, t, h], "verify", f"verify out t={t} h={h}")
    ref_s = oracle.verify_scores_grouped(wl.q, wl.dtype, OKV.of(wl), wl.P, wl.score_rows, wl.scale, wl.Hkv, wl.P_max)
    check_scores(as_f64(scores), ref_s, wl.P, score_floor(wl))


@pytest.mark.parametrize("name", ["batch4_chain16", "tree256_bf16", "paged5_tree64", "tree256_canary"])
def test_verify_is_deterministic(name):
    """No float atomics anywhere: reruns are bit-identical (scores compared where written, i < P_b)."""
    wl = CASES[name]()
    dw = DevWorkload(wl)
    o1, s1 = dw.verify()
    o2, s2 = dw.verify()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for b in range(wl.B):
        Pb = int(wl.P[b])
        assert torch.equal(s1[b, :Pb], s2[b, :Pb])


def test_scores_untouched_past_prefix():
    wl = CASES["gqa3_d64"]()
    dw = DevWorkload(wl)
    scores = torch.full((wl.B, wl.P_max), 7.25, dtype=torch.float32, device="cuda")
    dw.verify(scores=scores)
    s = scores.cpu().numpy()
    for b in range(wl.B):
        assert (s[b, int(wl.P[b]):] == 7.25).all()


# --------------------------------------------------------------------------- selection, exact

@pytest.mark.parametrize("kind", ["normal", "ties", "signed_zero", "constant", "wide"])
@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (1000, 1), (1000, 999), (5000, 250), (32768, 2048),
                                 (40000, 4000), (131072, 4096)])
def test_topk_exact(kind, n, k):
    """Same fp32 keys on both sides: the selected index list must be bit-identical."""
    s = make_score_vector(n * 7 + k, n, kind)
    B = 2
    S = np.stack([s, s[::-1].copy()])
    P = np.array([n, max(0, n - 3)], np.int32)
    K = np.array([k, k + 5], np.int32)
    kmax = k + 5
    idx, count = sv.topk_select(torch.from_numpy(S).cuda(), i32(P), i32(K), kmax)
    gi = idx.cpu().numpy()
    for b in range(B):
        want = oracle.topk_select(S[b], int(P[b]), int(K[b]))
        kk = len(want)
        assert int(count[b]) == kk
        np.testing.assert_array_equal(gi[b, :kk], want)
        assert (gi[b, kk:] == -1).all()


def test_topk_degenerate():
    S = np.array([[1.0, 2.0, 3.0, 0.0], [5.0, 5.0, 5.0, 5.0], [0.0, 0.0, 0.0, 0.0]], np.float32)
    P = np.array([4, 0, 3], np.int32)
    K = np.array([0, 2, 10], np.int32)
    idx, count = sv.topk_select(torch.from_numpy(S).cuda(), i32(P), i32(K), 6)
    gi = idx.cpu().numpy()
    assert count.cpu().tolist() == [0, 0, 3]
    assert (gi[0] == -1).all() and (gi[1] == -1).all()
    assert gi[2].tolist() == [0, 1, 2, -1, -1, -1]


# --------------------------------------------------------------------------- sparse draft, direct

@pytest.mark.parametrize("dtype,D,G,ps", [("bf16", 128, 4, 0), ("bf16", 64, 2, 16), ("f32", 128, 4, 16),
                                          ("f32", 64, 1, 0), ("bf16", 128, 4, 24), ("bf16", 128, 2, 1)])
def test_sparse_draft_direct(dtype, D, G, ps):
    Hkv = 4
    wl = make_custom(seed=200 + D + G + ps, B=3, Hq=G * Hkv, Hkv=Hkv, D=D, dtype=dtype, P=[700, 64, 300], N=4,
                     score_rows="all", k_sel=10, decode_steps=2, q_std_mult=6.0,
                     layout="paged" if ps else "contiguous", page_size=ps or 16)
    dw = DevWorkload(wl)
    rng = np.random.default_rng(D + G)
    lists = [rng.choice(704, 257, replace=False),                       # spans prefix and verify tokens
             rng.permutation(68)[:0],                                    # empty -> zeros
             rng.permutation(304)[:65]]
    stride = 300
    arr = np.full((3, stride), -1, np.int32)
    for b, li in enumerate(lists):
        arr[b, : len(li)] = li
    n = np.array([len(x) for x in lists], np.int32)
    out = sv.sparse_draft_attn(dw.dq[1], dw.kv, i32(arr), i32(n), max_idx=260)
    ref = oracle.sparse_draft_attention(wl.dq[1], dtype, OKV.of(wl), lists, wl.scale, wl.Hkv)
    g = as_f64(out)
    check_out(g, ref, dtype, "sparse draft")
    if dtype == "bf16":
        check_out_derived(g, ref, sparse_abs(wl, wl.dq[1], lists), "sparse", "sparse draft")
    assert (g[1] == 0).all()


def _sparse_case(seed, dtype="bf16", paged=False):
    Hkv = 4
    wl = make_custom(seed=seed, B=3, Hq=4 * Hkv, Hkv=Hkv, D=128, dtype=dtype, P=[900, 300, 620], N=4,
                     score_rows="all", k_sel=10, decode_steps=1, q_std_mult=6.0,
                     layout="paged" if paged else "contiguous", page_size=16)
    return wl, DevWorkload(wl)


def _sparse_lists(rng, sizes, spans):
    return [rng.choice(span, size, replace=False).astype(np.int32) for size, span in zip(sizes, spans)]


def _sparse_call_and_check(wl, dw, lists, stride, max_idx, ws, what):
    arr = np.full((len(lists), stride), -1, np.int32)
    for b, li in enumerate(lists):
        arr[b, : len(li)] = li
    n = np.array([len(x) for x in lists], np.int32)
    out = sv.sparse_draft_attn(dw.dq[0], dw.kv, i32(arr), i32(n), max_idx=max_idx, workspace=ws)
    ref = oracle.sparse_draft_attention(wl.dq[0], wl.dtype, OKV.of(wl), lists, wl.scale, wl.Hkv)
    check_out(as_f64(out), ref, wl.dtype, what)


@pytest.mark.parametrize("dtype,D,paged", [("bf16", 128, False), ("bf16", 64, True), ("f32", 128, False)])
def test_sparse_large_grid_chunks(dtype, D, paged):
    """Many lists (B * Hkv * ceil(max_idx / 64) >= 1024 workgroups) switch the
    draft step to 128-position chunks: ragged counts (a partial last chunk, a
    count below one chunk, zero, the full stride) still match the oracle."""
    Hkv, B = 8, 8
    P = [1500, 1300, 900, 700, 1500, 300, 1100, 1250]
    wl = make_custom(seed=230 + D, B=B, Hq=2 * Hkv, Hkv=Hkv, D=D, dtype=dtype, P=P, N=4, score_rows="all",
                     k_sel=10, decode_steps=1, q_std_mult=6.0, layout="paged" if paged else "contiguous",
                     page_size=16)
    dw = DevWorkload(wl)
    stride = 1100
    plan_wgs = B * Hkv * ((stride + 63) // 64)
    assert plan_wgs >= 1024
    rng = np.random.default_rng(7)
    sizes = [1100, 129, 0, 600, 127, 1, 1000, 200]
    lists = [rng.choice(int(P[b]) + 4, sizes[b], replace=False).astype(np.int32) for b in range(B)]
    _sparse_call_and_check(wl, dw, lists, stride, stride, sv.Workspace(), f"large grid {dtype} D={D}")


@pytest.mark.parametrize("paged", [False, True])
def test_sparse_workspace_garbage_and_reuse(paged):
    """The workspace is scratch: a workspace full of garbage, and the same
    workspace reused with other list lengths, give the same results as fresh
    memory would."""
    wl, dw = _sparse_case(410 + int(paged), paged=paged)
    rng = np.random.default_rng(7)
    ws = sv.Workspace()
    nbytes = sv.sparse_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.D, 512)
    ws.get(nbytes, "cuda")
    for fill in ("random", 0xFF, 0x00, "random"):
        if fill == "random":
            ws.buf.copy_(torch.randint(0, 256, ws.buf.shape, dtype=torch.uint8, device="cuda"))
        else:
            ws.buf.fill_(fill)
        for sizes in ([512, 1, 300], [65, 200, 0], [128, 64, 511]):
            lists = _sparse_lists(rng, sizes, [904, 304, 624])
            _sparse_call_and_check(wl, dw, lists, 512, 512, ws, f"sparse fill={fill} sizes={sizes}")


def test_sparse_graph_replay():
    """Captured once in a HIP graph, replayed with other index lists and list
    lengths, with eager calls on the same workspace in between: every replay
    matches the oracle (nothing carries over from one launch to the next)."""
    wl, dw = _sparse_case(420)
    rng = np.random.default_rng(9)
    stride = 512
    ws = sv.Workspace()
    ws.get(sv.sparse_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.D, stride), "cuda")
    idx_t = torch.full((wl.B, stride), -1, dtype=torch.int32, device="cuda")
    n_t = torch.zeros((wl.B,), dtype=torch.int32, device="cuda")
    q = dw.dq[0].contiguous()
    out = torch.empty_like(q)
    sizes0 = [300, 200, 100]
    lists = _sparse_lists(rng, sizes0, [904, 304, 624])

    def load(lists):
        arr = np.full((wl.B, stride), -1, np.int32)
        for b, li in enumerate(lists):
            arr[b, : len(li)] = li
        idx_t.copy_(torch.from_numpy(arr))
        n_t.copy_(torch.from_numpy(np.array([len(x) for x in lists], np.int32)))

    load(lists)
    sv.sparse_draft_attn(q, dw.kv, idx_t, n_t, max_idx=stride, out=out, workspace=ws)  # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.sparse_draft_attn(q, dw.kv, idx_t, n_t, max_idx=stride, out=out, workspace=ws)
    for rep, sizes in enumerate(([300, 200, 100], [512, 7, 0], [64, 300, 450], [1, 1, 1])):
        lists = _sparse_lists(rng, sizes, [904, 304, 624])
        load(lists)
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.sparse_draft_attention(wl.dq[0], wl.dtype, OKV.of(wl), lists, wl.scale, wl.Hkv)
        check_out(as_f64(out), ref, wl.dtype, f"replay {rep} sizes={sizes}")
        # an eager call on the same workspace (a new epoch) between replays
        eager_lists = _sparse_lists(rng, [33, 44, 55], [904, 304, 624])
        _sparse_call_and_check(wl, dw, eager_lists, stride, stride, ws, f"eager after replay {rep}")
        torch.cuda.synchronize()


def test_sparse_full_index_equals_dense_verify_row():
    """k = whole context: the draft output equals dense attention of the same query (N = 1 verify)."""
    wl = make_custom(seed=300, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=4000, N=1, score_rows="all",
                     k_sel=4001, decode_steps=0, q_std_mult=4.0)
    dw = DevWorkload(wl)
    out, scores = dw.verify()
    idx = np.arange(4001, dtype=np.int32)[None]
    d = sv.sparse_draft_attn(dw.q[:, 0].contiguous(), dw.kv, i32(idx), i32([4001]))
    a, b = as_f64(out)[:, 0], as_f64(d)
    assert np.abs(a - b).max() <= 2e-2 * np.abs(a).max()
