"""How far a tree-mask mistake moves the outputs of the GPU parity test's
canary cases, measured on the CPU with the mistake planted in the oracle: a
node that also sees one sibling's token, or that no longer sees its parent.
Each must move that node's outputs by at least ten times the bound the GPU
test applies (both the absolute/relative bound and the rounding-derived one),
so the GPU test cannot pass a kernel that makes such a mistake."""
import numpy as np
import pytest

import oracle
import oracle.reference as ref
from oracle import KVCache as OKV
from tests.gpu_util import DERIVED, DERIVED_SLACK, OUT_ABS, OUT_REL_MAX, attention_abs
from tests.test_gpu_parity import CASES

MARGIN = 10.0


def _planted(monkeypatch, b_target, P_target, t_target, mistake, parent):
    orig = ref.visible_positions
    anc = set(ref.ancestors(parent, t_target))
    sibling = next(s for s in range(len(parent)) if s not in anc)  # lowest-index non-ancestor node
    par = int(parent[t_target])

    def vis(P_b, pb, t):
        v = orig(P_b, pb, t)
        if t != t_target or P_b != P_target:
            return v
        if mistake == "sibling":
            return np.concatenate([v, [P_b + sibling]])
        return v[v != P_b + par]
    monkeypatch.setattr(ref, "visible_positions", vis)
    return sibling, par


@pytest.mark.slow
@pytest.mark.parametrize("name,b,nodes", [("tree256_canary", 0, [70, 150, 255]),
                                          ("paged_tree64_canary", 1, [20, 41, 63])])
def test_mask_mistakes_exceed_the_gpu_bound(monkeypatch, name, b, nodes):
    wl = CASES[name]()
    kv = OKV.of(wl)
    full = oracle.verify_attention(wl.q, wl.dtype, kv, wl.P, wl.parent, wl.scale, wl.Hkv)
    # the GPU test's bounds on this case
    bound_abs = min(OUT_ABS["bf16"], OUT_REL_MAX["bf16"] * np.abs(full).max() + 1e-6)
    rows = [(b, t, h) for t in nodes for h in range(wl.Hq)]
    ab = attention_abs(wl, rows=rows)
    a, c = DERIVED["verify"]
    parent = wl.parent[b]
    Pb = int(wl.P[b])
    for t in nodes:
        derived = a * np.abs(full[b, t]) + (c + DERIVED_SLACK) * ab[b, t] + 1e-9
        for mistake in ("sibling", "parent"):
            with monkeypatch.context() as m:
                _planted(m, b, Pb, t, mistake, parent)
                bad = oracle.verify_attention(wl.q, wl.dtype, kv, wl.P, wl.parent, wl.scale, wl.Hkv,
                                              rows=[(b, t, h) for h in range(wl.Hq)])
            diff = np.abs(bad[b, t] - full[b, t])
            assert diff.max() >= MARGIN * bound_abs, (name, t, mistake, diff.max(), bound_abs)
            assert (diff / derived).max() >= MARGIN, (name, t, mistake, (diff / derived).max())
