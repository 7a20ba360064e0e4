"""The whole step (sv_verify_select, then sv_sparse_draft_attn over its
selection) captured once in a HIP graph and replayed with new queries,
prefix lengths and k, with eager steps on the same workspaces in between:
every replay equals the eager step on the same inputs, bit for bit (the
kernels are deterministic, and nothing may carry over from one launch to the
next)."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DevWorkload
from workloads import make_custom

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


CASES = {
    "chain8_c2q_b2": dict(seed=501, B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[3001, 1700], N=8,
                          score_rows="c2q", k_sel=[200, 90], decode_steps=1),
    "tree64_paged_b2": dict(seed=502, B=2, Hq=32, Hkv=8, D=128, dtype="bf16", P=[2500, 900], N=64,
                            tree="best_first", tree_depth=6, score_rows="all", k_sel="5pct", layout="paged",
                            page_size=16, decode_steps=1),
}


def _buffers(wl, dev="cuda"):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    return {
        "out": torch.empty((wl.B, wl.N, wl.Hq, wl.D), dtype=dt, device=dev),
        "scores": torch.empty((wl.B, wl.P_max), dtype=torch.float32, device=dev),
        "idx": torch.empty((wl.B, wl.k_max), dtype=torch.int32, device=dev),
        "count": torch.empty((wl.B,), dtype=torch.int32, device=dev),
        "draft": torch.empty((wl.B, wl.Hq, wl.D), dtype=dt, device=dev),
    }


def _step(wl, dw, q, P, k, dq, bufs, ws_sel, ws_sp):
    _, _, idx, count = sv.verify_select(q, dw.kv, P, k, wl.k_max, P_max=wl.P_max, parent=dw.parent,
                                        score_rows=[int(r) for r in wl.score_rows], out=bufs["out"],
                                        scores=bufs["scores"], idx=bufs["idx"], count=bufs["count"],
                                        workspace=ws_sel)
    sv.sparse_draft_attn(dq, dw.kv, idx, count, max_idx=wl.k_max, out=bufs["draft"], workspace=ws_sp)


def _same(g, e, P, what):
    assert torch.equal(g["out"], e["out"]), f"{what}: verification outputs differ"
    assert torch.equal(g["count"], e["count"]), f"{what}: counts differ"
    assert torch.equal(g["draft"], e["draft"]), f"{what}: draft outputs differ"
    for b, pb in enumerate(P.tolist()):
        assert torch.equal(g["scores"][b, :pb], e["scores"][b, :pb]), f"{what}: scores of row {b} differ"
        n = int(e["count"][b])
        assert torch.equal(g["idx"][b, :n], e["idx"][b, :n]), f"{what}: indices of row {b} differ"


@pytest.mark.parametrize("name", list(CASES))
def test_step_graph_replay(name):
    print(f"[case] {name}", flush=True)
    wl = make_custom(**CASES[name])
    dw = DevWorkload(wl)
    q, P, k, dq = dw.q.clone(), dw.P.clone(), dw.k_sel.clone(), dw.dq[0].clone()
    gbuf = _buffers(wl)
    ws_sel, ws_sp = sv.Workspace(), sv.Workspace()
    _step(wl, dw, q, P, k, dq, gbuf, ws_sel, ws_sp)  # sizes the workspaces outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(wl, dw, q, P, k, dq, gbuf, ws_sel, ws_sp)
    gen = torch.Generator(device="cuda").manual_seed(7)
    rng = np.random.default_rng(11)
    sigma = 1.0 / np.sqrt(wl.D)
    for rep in range(4):
        # new inputs in the captured buffers: queries, shorter or equal prefixes, k
        q.copy_((torch.randn(q.shape, generator=gen, device="cuda") * (2.0 * sigma)).to(q.dtype))
        dq.copy_((torch.randn(dq.shape, generator=gen, device="cuda") * sigma).to(dq.dtype))
        newP = np.array([int(rng.integers(max(0, p // 2), p + 1)) for p in wl.P], np.int32)
        P.copy_(torch.from_numpy(newP))
        k.copy_(torch.from_numpy(np.array([int(rng.integers(1, wl.k_max + 1)) for _ in range(wl.B)], np.int32)))
        graph.replay()
        torch.cuda.synchronize()
        ebuf = _buffers(wl)
        _step(wl, dw, q, P, k, dq, ebuf, sv.Workspace(), sv.Workspace())
        torch.cuda.synchronize()
        _same(gbuf, ebuf, newP, f"replay {rep}")
        # an eager step on the graph's own workspaces before the next replay
        _step(wl, dw, q, P, k, dq, _buffers(wl), ws_sel, ws_sp)
        torch.cuda.synchronize()
