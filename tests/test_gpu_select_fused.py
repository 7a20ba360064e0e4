"""sv_verify_select (selection fused into the verification's last kernel)
against the two separate calls it replaces, sv_verify_attn then
sv_topk_select: outputs, scores, indices and counts must be the same bits.
The separate calls are themselves held to the oracle by the parity tests;
here the selections are also checked against the oracle's (tie-band rule)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import KVCache as OKV
from workloads import make_custom, make_workload
from tests.gpu_util import DevWorkload, check_selection_band, i32
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()


def _compare(wl, k_sel=None, check_oracle=True):
    dw = DevWorkload(wl)
    rows = [int(r) for r in wl.score_rows]
    k_sel = wl.k_sel if k_sel is None else np.asarray(k_sel, np.int32)
    kmax = max(int(wl.k_max), int(k_sel.max()))
    k_t = i32(k_sel)
    out1, s1 = dw.verify()
    idx1, cnt1 = sv.topk_select(s1, dw.P, k_t, kmax)
    out2, s2, idx2, cnt2 = sv.verify_select(dw.q, dw.kv, dw.P, k_t, kmax, P_max=wl.P_max, parent=dw.parent,
                                            score_rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "outputs differ"
    for b in range(wl.B):
        Pb = int(wl.P[b])
        assert torch.equal(s1[b, :Pb], s2[b, :Pb]), f"scores differ, seq {b}"
    assert torch.equal(cnt1, cnt2), f"counts differ: {cnt1.tolist()} vs {cnt2.tolist()}"
    assert torch.equal(idx1, idx2), "indices differ"
    if check_oracle:
        ref_s = oracle.verify_scores_grouped(wl.q, wl.dtype, OKV.of(wl), wl.P, wl.score_rows, wl.scale, wl.Hkv,
                                             wl.P_max)
        ref_idx = [oracle.topk_select(ref_s[b], int(wl.P[b]), int(k_sel[b])) for b in range(wl.B)]
        check_selection_band(idx2.cpu().numpy(), ref_s, ref_idx, wl.P, k_sel)
    return idx2, cnt2


@pytest.mark.parametrize("name", [n for n in CASES if n not in ("no_scores",)])
def test_fused_equals_separate_calls(name):
    print(f"[case] {name}", flush=True)
    _compare(CASES[name]())


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fused_full_size(cfg):
    print(f"[case] full-size workload {cfg}", flush=True)
    _compare(make_workload(cfg), check_oracle=cfg in (2, 4))


def test_fused_edge_rows():
    """An empty prefix, k = 0, k = P, k > P and a short row in one batch."""
    wl = make_custom(seed=601, B=6, Hq=8, Hkv=2, D=128, dtype="bf16", P=[0, 5000, 9000, 3000, 20000, 700], N=4,
                     score_rows="all", k_sel=10, decode_steps=0)
    k = np.array([10, 0, 9000, 4000, 1500, 64], np.int32)
    idx, cnt = _compare(wl, k_sel=k)
    assert cnt.tolist() == [0, 0, 9000, 3000, 1500, 64]


def test_fused_ties_take_the_radix_path():
    """All keys equal: every score ties, the band holds the whole row (its
    slots overflow), and the last workgroup runs the exact radix path: the k
    lowest indices."""
    wl = make_custom(seed=602, B=2, Hq=8, Hkv=2, D=128, dtype="bf16", P=[30000, 12000], N=4, score_rows="all",
                     k_sel=1000, decode_steps=0)
    for b in range(wl.B):
        base = b * wl.seq_stride
        wl.k[base: base + int(wl.P[b])] = wl.k[base]
    idx, cnt = _compare(wl)
    gi = idx.cpu().numpy()
    for b in range(wl.B):
        assert gi[b, :1000].tolist() == list(range(1000))


def test_fused_large_k_fraction():
    """k a quarter of the row and more (a fixed budget over short contexts):
    the rows' blocks stay within their slots (1024-entry blocks up to 32768
    entries), and the selection equals the separate calls' and the oracle band."""
    wl = make_custom(seed=603, B=4, Hq=8, Hkv=2, D=128, dtype="bf16", P=[8192, 20000, 32768, 6000], N=4,
                     score_rows="all", k_sel=10, decode_steps=0)
    k = np.array([2048, 6000, 8192, 3000], np.int32)
    idx, cnt = _compare(wl, k_sel=k)
    assert cnt.tolist() == k.tolist()
