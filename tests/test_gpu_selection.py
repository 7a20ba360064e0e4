"""GPU parity of the selection variants against the CPU oracle: per-KV-head
scores (tolerance of the scores), per-head top-k sets (exact outside the tie
band), the per-head sparse draft step (output tolerance), and the sink +
recent-window baseline (exact), on chains and trees with ragged prefixes."""
import numpy as np
import pytest
import torch

import oracle
from oracle import KVCache as OKV
from workloads import make_custom
from tests.gpu_util import DevWorkload, as_f64, check_out, check_scores, check_selection_band, i32, score_floor

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


CASES = {
    "chain8_c2q": lambda: make_custom(seed=501, B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[3001, 1200], N=8,
                                      score_rows="c2q", k_sel=200, heavy_count=30, heavy_c=2.5),
    "tree64_all": lambda: make_custom(seed=502, B=3, Hq=16, Hkv=4, D=128, dtype="bf16", P=[900, 64, 2000], N=64,
                                      tree="best_first", tree_depth=6, score_rows="all", k_sel=100),
    "f32_chain": lambda: make_custom(seed=503, B=1, Hq=8, Hkv=2, D=64, dtype="f32", P=700, N=5, score_rows="all",
                                     k_sel=64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_per_head_scores_selection_and_draft(name):
    wl = CASES[name]()
    dw = DevWorkload(wl)
    rows = [int(r) for r in wl.score_rows]
    hs0 = torch.zeros((wl.B, wl.Hkv, wl.P_max), dtype=torch.float32, device="cuda")  # entries past P_b stay 0
    out, hs = sv.verify_attn_per_head(dw.q, dw.kv, dw.P, P_max=wl.P_max, parent=dw.parent, score_rows=rows,
                                      head_scores=hs0)
    kv = OKV.of(wl)
    ref = oracle.verify_scores_per_head(wl.q, wl.dtype, kv, wl.P, rows, wl.scale, wl.Hkv, wl.P_max)
    g = as_f64(hs)
    B, H = wl.B, wl.Hkv
    P_rows = np.repeat(wl.P, H)
    floor_h = score_floor(wl, rows=rows, per_head=True)
    check_scores(g.reshape(B * H, -1), ref.reshape(B * H, -1), P_rows, floor_h.reshape(B * H, -1))
    # the attention output is that of the ordinary call, and the per-head scores
    # sum to its scores (the merge's fp32 sum over the heads: the same floor)
    out2, tot = dw.verify()
    assert torch.equal(out, out2)
    check_scores(g.sum(axis=1), as_f64(tot).astype(np.float64), wl.P, score_floor(wl, rows=rows))
    # top-k per (sequence, KV head): the B * Hkv rows through the ordinary selection
    k_rows = np.repeat(wl.k_sel, H)
    idx, count = sv.topk_select(hs.view(B * H, wl.P_max), i32(P_rows), i32(k_rows), wl.k_max)
    ref_idx = [oracle.topk_select(ref[b, h], int(wl.P[b]), int(wl.k_sel[b])) for b in range(B) for h in range(H)]
    check_selection_band(idx.cpu().numpy(), ref.reshape(B * H, -1), ref_idx, P_rows, k_rows)
    # the draft step with one list per KV head (the oracle's lists, so the output compares exactly)
    lists = [[ref_idx[b * H + h] for h in range(H)] for b in range(B)]
    arr = np.full((B, H, wl.k_max), -1, np.int32)
    n = np.zeros((B, H), np.int32)
    for b in range(B):
        for h in range(H):
            arr[b, h, : len(lists[b][h])] = lists[b][h]
            n[b, h] = len(lists[b][h])
    if name == "tree64_all":  # ragged and empty lists
        n[0, 1] = 0
        n[2, 3] = 7
        lists[0][1] = lists[0][1][:0]
        lists[2][3] = lists[2][3][:7]
    d = sv.sparse_draft_attn_per_head(dw.dq[0], dw.kv, i32(arr), i32(n), max_idx=wl.k_max)
    dref = oracle.sparse_draft_attention_per_head(wl.dq[0], wl.dtype, kv, lists, wl.scale, H)
    check_out(as_f64(d), dref, wl.dtype, "per-head draft")


def test_sink_window_exact():
    P = np.array([0, 3, 50, 1000, 64], np.int32)
    for sink, window in ((4, 16), (0, 32), (8, 0), (64, 64)):
        k_max = sink + window + 3
        idx, count = sv.select_sink_window(i32(P), 1000, sink, window, k_max)
        idx, count = idx.cpu().numpy(), count.cpu().numpy()
        for b, Pb in enumerate(P):
            ref = oracle.sink_window_select(int(Pb), sink, window)
            assert count[b] == len(ref)
            assert idx[b, : len(ref)].tolist() == ref.tolist() and (idx[b, len(ref):] == -1).all()


def _top_nonnan(row, P, k):
    """The min(k, #finite) largest finite entries of row[:P], lower index first on
    ties, in increasing index order (the selection's contract for NaN entries)."""
    s = np.asarray(row[:P], dtype=np.float64)
    fin = np.nonzero(~np.isnan(s))[0]
    order = fin[np.lexsort((fin, -s[fin]))]
    return np.sort(order[:min(k, len(fin))])


@pytest.mark.parametrize("P,k,nan_frac", [(3000, 100, 0.3), (30000, 2048, 0.1), (30000, 2048, 0.95),
                                          (100000, 4096, 0.5), (5000, 4999, 0.01)])
def test_topk_nan_entries_never_selected(P, k, nan_frac):
    """Rows holding NaN scores (the band path, the radix path, and rows with
    fewer finite entries than k): NaN entries are never selected, `count` is the
    number of indices written, and the rest of the row of indices is -1."""
    r = np.random.default_rng([P, k, int(nan_frac * 100)])
    B = 2
    s = r.standard_normal((B, P)).astype(np.float32)
    s[r.random((B, P)) < nan_frac] = np.nan
    st = torch.from_numpy(s).cuda()
    Pt = torch.full((B,), P, dtype=torch.int32, device="cuda")
    kt = torch.full((B,), k, dtype=torch.int32, device="cuda")
    idx, cnt = sv.topk_select(st, Pt, kt, k)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        ref = _top_nonnan(s[b], P, k)
        assert int(cnt[b]) == len(ref), (b, int(cnt[b]), len(ref))
        assert np.array_equal(idx[b, :len(ref)], ref), f"row {b}"
        assert (idx[b, len(ref):] == -1).all()
