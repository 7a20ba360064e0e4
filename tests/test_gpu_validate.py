"""GPU tests of the device-array contract checks (sv_validate_kv,
sv_validate_tree, sv_validate_index): silent on valid inputs of every layout,
and each planted violation is reported with its code, sequence or list,
index and value.  Only the check kernels read the planted arrays (they read
within the arrays' stated sizes); with SV_DEBUG_CHECKS=1 the bindings raise
before any compute kernel is launched."""
import numpy as np
import pytest
import torch

from workloads import make_custom
from tests.gpu_util import DevWorkload, i32

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


def _wl(paged, tree=True, seed=900):
    return make_custom(seed=seed + int(paged), B=3, Hq=8, Hkv=2, D=64, dtype="bf16", P=[300, 17, 1000], N=12,
                       tree="best_first" if tree else None, tree_depth=4, score_rows="all", k_sel=40,
                       decode_steps=1, layout="paged" if paged else "contiguous", page_size=16)


@pytest.mark.parametrize("paged", [False, True])
def test_valid_inputs_pass(paged):
    wl = _wl(paged)
    dw = DevWorkload(wl)
    assert sv.validate_kv(dw.kv, dw.P, P_max=wl.P_max, N=wl.N) == (0, 0, 0, 0)
    assert sv.validate_tree(dw.parent) == (0, 0, 0, 0)
    _, _, idx, count, _ = dw.step()
    assert sv.validate_index(dw.kv, idx, count, max_idx=wl.k_max) == (0, 0, 0, 0)
    # per-KV-head lists: the same list for every head
    idx3 = idx[:, None, :].expand(wl.B, wl.Hkv, idx.shape[1]).contiguous()
    cnt3 = count[:, None].expand(wl.B, wl.Hkv).contiguous()
    assert sv.validate_index(dw.kv, idx3, cnt3, max_idx=wl.k_max) == (0, 0, 0, 0)


def test_prefix_length_out_of_range():
    wl = _wl(False)
    dw = DevWorkload(wl)
    P = wl.P.copy()
    P[1] = wl.P_max + 5
    assert sv.validate_kv(dw.kv, i32(P), P_max=wl.P_max, N=wl.N) == (1, 1, 0, wl.P_max + 5)
    P[1] = -3
    assert sv.validate_kv(dw.kv, i32(P), P_max=wl.P_max, N=wl.N) == (1, 1, 0, -3)


def test_unmapped_page_and_short_storage():
    wl = _wl(True)
    dw = DevWorkload(wl)
    pt = wl.page_table.copy()
    pt[2, 3] = -1  # positions 48..63 of sequence 2 (P_2 = 1000)
    kv = sv.KVCache(dw.kv.k, dw.kv.v, seq_stride=0, page_table=i32(pt), page_size=wl.page_size)
    code, b, i, v = sv.validate_kv(kv, dw.P, P_max=wl.P_max, N=wl.N)
    assert (code, b, i // wl.page_size, v) == (2, 2, 3, -1)
    # the verify tokens' own positions are checked too: a page covering [P_b, P_b + N) unmapped
    pt = wl.page_table.copy()
    last = (int(wl.P[1]) + wl.N - 1) // wl.page_size
    pt[1, last] = -1
    kv = sv.KVCache(dw.kv.k, dw.kv.v, seq_stride=0, page_table=i32(pt), page_size=wl.page_size)
    code, b, i, v = sv.validate_kv(kv, dw.P, P_max=wl.P_max, N=wl.N)
    assert (code, b, i // wl.page_size) == (2, 1, last)
    assert sv.validate_kv(kv, dw.P, P_max=wl.P_max, N=0)[0] in (0, 2)
    # contiguous: a sequence stride too small for the last sequence's range
    wl2 = _wl(False)
    dw2 = DevWorkload(wl2)
    short = sv.KVCache(dw2.kv.k, dw2.kv.v, seq_stride=wl2.seq_stride + 200, page_table=None, page_size=1)
    code, b, i, v = sv.validate_kv(short, dw2.P, P_max=wl2.P_max, N=wl2.N)
    assert code == 2 and b == 2 and 2 * (wl2.seq_stride + 200) + i >= wl2.num_slots


def test_bad_parents():
    wl = _wl(False)
    dw = DevWorkload(wl)
    par = wl.parent.copy()
    par[0, 5] = 7
    assert sv.validate_tree(i32(par)) == (3, 0, 5, 7)
    par = wl.parent.copy()
    par[2, 0] = 0
    assert sv.validate_tree(i32(par)) == (3, 2, 0, 0)
    par = wl.parent.copy()
    par[1, 9] = -1
    assert sv.validate_tree(i32(par)) == (3, 1, 9, -1)


def test_bad_index_lists():
    wl = _wl(True)
    dw = DevWorkload(wl)
    rng = np.random.default_rng(3)
    lists = np.full((wl.B, 64), -1, np.int32)
    n = np.array([50, 10, 64], np.int32)
    for b in range(wl.B):
        lists[b, : n[b]] = np.sort(rng.choice(int(wl.P[b]), n[b], replace=False))
    assert sv.validate_index(dw.kv, i32(lists), i32(n), max_idx=64) == (0, 0, 0, 0)
    bad = lists.copy()
    bad[1, 3] = -2
    assert sv.validate_index(dw.kv, i32(bad), i32(n), max_idx=64) == (5, 1, 3, -2)
    bad = lists.copy()
    far = (wl.max_pages + 2) * wl.page_size  # past every page-table row
    bad[2, 63] = far
    assert sv.validate_index(dw.kv, i32(bad), i32(n), max_idx=64) == (5, 2, 63, far)
    assert sv.validate_index(dw.kv, i32(lists), i32(np.array([50, 65, 64], np.int32)), max_idx=64) == (4, 1, 0, 65)
    # entries past the count are not checked
    bad = lists.copy()
    bad[1, 40] = -9
    assert sv.validate_index(dw.kv, i32(bad), i32(n), max_idx=64) == (0, 0, 0, 0)


def test_record_is_cleared_between_calls_and_debug_env(monkeypatch):
    wl = _wl(False)
    dw = DevWorkload(wl)
    par = wl.parent.copy()
    par[0, 2] = 2
    assert sv.validate_tree(i32(par))[0] == 3
    assert sv.validate_tree(dw.parent) == (0, 0, 0, 0)
    monkeypatch.setenv("SV_DEBUG_CHECKS", "1")
    with pytest.raises(sv.ContractError, match=r"parent\[0\]\[2\] = 2"):
        sv.verify_attn(dw.q, dw.kv, dw.P, P_max=wl.P_max, parent=i32(par), score_rows=[0])
    P = wl.P.copy()
    P[0] = wl.P_max + 1
    with pytest.raises(sv.ContractError, match="prefix_len"):
        sv.verify_attn(dw.q, dw.kv, i32(P), P_max=wl.P_max, parent=dw.parent, score_rows=[0])
    out, _ = sv.verify_attn(dw.q, dw.kv, dw.P, P_max=wl.P_max, parent=dw.parent, score_rows=[0])
    assert torch.isfinite(out.float()).all()


def test_debug_checks_stay_out_of_graph_capture(monkeypatch):
    """With SV_DEBUG_CHECKS=1 an eager call is checked, while a call captured in
    a HIP graph is not (the checks synchronise); the captured call replays."""
    wl = _wl(False, tree=False)
    dw = DevWorkload(wl)
    monkeypatch.setenv("SV_DEBUG_CHECKS", "1")
    _, _, idx, count, _ = dw.step()
    out = torch.empty_like(dw.dq[0])
    ws = sv.Workspace()
    sv.sparse_draft_attn(dw.dq[0], dw.kv, idx, count, max_idx=wl.k_max, out=out, workspace=ws)
    ref = out.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.sparse_draft_attn(dw.dq[0], dw.kv, idx, count, max_idx=wl.k_max, out=out, workspace=ws)
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    bad = count.clone()
    bad[0] = wl.k_max + 1
    with pytest.raises(sv.ContractError, match="n_idx"):
        sv.sparse_draft_attn(dw.dq[0], dw.kv, idx, bad, max_idx=wl.k_max, out=out, workspace=ws)
