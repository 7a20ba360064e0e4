"""GPU parity at the five measured workloads' full sizes, through the same
entry points and launch configurations the benchmark times.

At these sizes the oracle cannot run every attention row, so:
  * verify outputs are compared on sampled (sequence, node, head) rows, each
    computed by the oracle one by one over all of its visible keys;
  * scores are compared for every prefix entry (the oracle's grouped score sum,
    pinned to its explicit double sum on small inputs);
  * the selected index sets are compared whole against the oracle's selection
    from its own scores (tie-band rule);
  * the sparse draft step runs on the oracle's selected indices (an input from
    the oracle side) and every output is compared; for several draft steps the
    compacted path (rows gathered once, dense decodes) is compared as well.
"""
import functools
import time

import numpy as np
import pytest
import torch

import oracle
from oracle import KVCache as OKV
from workloads import CONFIG_NAMES, make_workload
from tests.gpu_util import (DevWorkload, as_f64, attention_abs, check_out, check_out_derived, check_scores,
                            check_selection_band, i32, score_floor, sparse_abs)

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


@functools.lru_cache(maxsize=1)
def _workload(cfg):
    t0 = time.time()
    wl = make_workload(cfg)
    print(f"[workload {cfg} {CONFIG_NAMES[cfg]}] generated in {time.time() - t0:.1f} s", flush=True)
    return wl


def _sample_rows(wl, n, seed):
    """(b, t, h) rows: the root and last node of a few sequences, plus random ones."""
    r = np.random.default_rng(seed)
    rows = set()
    for b in sorted(set(r.integers(0, wl.B, size=min(wl.B, 3)).tolist())):
        rows.add((b, 0, int(r.integers(0, wl.Hq))))
        rows.add((b, wl.N - 1, int(r.integers(0, wl.Hq))))
    while len(rows) < n:
        rows.add((int(r.integers(0, wl.B)), int(r.integers(0, wl.N)), int(r.integers(0, wl.Hq))))
    return sorted(rows)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_step(cfg):
    print(f"[case] full-size workload {cfg}", flush=True)
    wl = _workload(cfg)
    dw = DevWorkload(wl)
    out, scores = dw.verify()
    idx, count = sv.topk_select(scores, dw.P, dw.k_sel, wl.k_max)
    torch.cuda.synchronize()
    kv = OKV.of(wl)

    # verify outputs on sampled rows
    t0 = time.time()
    rows = _sample_rows(wl, 12, seed=cfg)
    ref = oracle.verify_attention(wl.q, wl.dtype, kv, wl.P, wl.parent, wl.scale, wl.Hkv, rows=rows)
    got = as_f64(out)
    ab = attention_abs(wl, rows=rows) if wl.dtype == "bf16" else None
    for (b, t, h) in rows:
        check_out(got[b, t, h], ref[b, t, h], wl.dtype, f"verify out (b={b}, t={t}, h={h})")
        if ab is not None:
            check_out_derived(got[b, t, h], ref[b, t, h], ab[b, t, h], "verify", f"verify out (b={b}, t={t}, h={h})")
    print(f"  sampled attention rows checked in {time.time() - t0:.1f} s", flush=True)

    # every score, and the whole selection
    t0 = time.time()
    ref_s = oracle.verify_scores_grouped(wl.q, wl.dtype, kv, wl.P, wl.score_rows, wl.scale, wl.Hkv, wl.P_max)
    worst, by_floor = check_scores(as_f64(scores), ref_s, wl.P, score_floor(wl))
    print(f"  scores: worst relative error {worst:.2e}, {by_floor} entries within the fp32 floor only", flush=True)
    ref_idx = [oracle.topk_select(ref_s[b], int(wl.P[b]), int(wl.k_sel[b])) for b in range(wl.B)]
    assert (count.cpu().numpy() == np.minimum(wl.k_sel, wl.P)).all()
    swaps = check_selection_band(idx.cpu().numpy(), ref_s, ref_idx, wl.P, wl.k_sel)
    print(f"  scores + selection checked in {time.time() - t0:.1f} s ({swaps} tie-band swaps)", flush=True)

    # sparse draft steps over the oracle's selection
    steps = sorted({0, wl.dq.shape[0] - 1}) if wl.dq.shape[0] else []
    oi = np.full((wl.B, max(1, wl.k_max)), -1, np.int32)
    for b in range(wl.B):
        oi[b, : len(ref_idx[b])] = ref_idx[b]
    n = np.array([len(x) for x in ref_idx], np.int32)
    compact = wl.dq.shape[0] > 1  # the benchmark's draft path for several draft steps
    if compact:
        cap = max(1, wl.k_max)
        ck, cv = sv.compact_kv(dw.kv, i32(oi), i32(n), cap)
    for s in steps:
        d = sv.sparse_draft_attn(dw.dq[s], dw.kv, i32(oi), i32(n), max_idx=max(1, wl.k_max))
        dref = oracle.sparse_draft_attention(wl.dq[s], wl.dtype, kv, ref_idx, wl.scale, wl.Hkv)
        check_out(as_f64(d), dref, wl.dtype, f"draft step {s}")
        dab = sparse_abs(wl, wl.dq[s], ref_idx) if wl.dtype == "bf16" else None
        if dab is not None:
            check_out_derived(as_f64(d), dref, dab, "sparse", f"draft step {s}")
        if compact:
            dd = sv.dense_draft_attn(dw.dq[s], ck, cv, i32(n))
            check_out(as_f64(dd), dref, wl.dtype, f"compacted draft step {s}")
            if dab is not None:
                check_out_derived(as_f64(dd), dref, dab, "verify", f"compacted draft step {s}")


@pytest.mark.parametrize("cfg", [2, 4])
def test_full_size_selection_is_consistent(cfg):
    """Property at any size: on the GPU's own scores, every selected entry beats
    every unselected one (larger score, or equal score at a lower index)."""
    wl = _workload(cfg)
    dw = DevWorkload(wl)
    _, scores = dw.verify()
    idx, count = sv.topk_select(scores, dw.P, dw.k_sel, wl.k_max)
    s = scores.cpu().numpy()
    gi = idx.cpu().numpy()
    for b in range(wl.B):
        Pb, kb = int(wl.P[b]), int(count[b])
        sel = np.zeros(Pb, bool)
        sel[gi[b, :kb]] = True
        sb = s[b, :Pb].astype(np.float64)
        worst_kept = sb[sel].min()
        best_dropped = sb[~sel].max()
        assert worst_kept >= best_dropped
        if worst_kept == best_dropped:   # ties: kept ones have the lower indices
            tie = np.nonzero(sb == worst_kept)[0]
            assert (np.nonzero(sel[tie])[0] == np.arange(sel[tie].sum())).all()
