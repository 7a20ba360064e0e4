"""Helpers for the GPU parity tests: move seeded workloads to the device, run
the HIP path through the C ABI binding, and compare with the oracle under the
stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import tree_verify_sparse_amd as sv

# tolerances (outputs: max-abs; scores: relative to max(|s_i|, rms_b(s)))
OUT_ABS = {"bf16": 2e-2, "f32": 1e-4}
OUT_REL_MAX = {"bf16": 2e-2, "f32": 1e-4}   # relative to max |o_ref| of the compared set
SCORE_REL = 1e-3


def to_torch(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def i32(x, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


class DevWorkload:
    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.q = to_torch(wl.q, wl.dtype, device)
        k = to_torch(wl.k, wl.dtype, device)
        v = to_torch(wl.v, wl.dtype, device)
        pt = i32(wl.page_table, device) if wl.page_table is not None else None
        self.kv = sv.KVCache(k, v, seq_stride=wl.seq_stride, page_table=pt, page_size=wl.page_size)
        self.P = i32(wl.P, device)
        self.parent = i32(wl.parent, device) if wl.parent is not None else None
        self.k_sel = i32(wl.k_sel, device)
        self.dq = [to_torch(wl.dq[s], wl.dtype, device) for s in range(wl.dq.shape[0])]

    def verify(self, **kw):
        return sv.verify_attn(self.q, self.kv, self.P, P_max=self.wl.P_max, parent=self.parent,
                              score_rows=[int(r) for r in self.wl.score_rows], **kw)

    def step(self, decode_step=0):
        """verify -> top-k -> sparse draft, all on the device."""
        out, scores = self.verify()
        idx, count = sv.topk_select(scores, self.P, self.k_sel, self.wl.k_max)
        draft = None
        if self.dq:
            draft = sv.sparse_draft_attn(self.dq[decode_step], self.kv, idx, count, max_idx=self.wl.k_max)
        return out, scores, idx, count, draft


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_out(gpu: np.ndarray, ref: np.ndarray, dtype: str, what="out"):
    mask = ~np.isnan(ref)
    assert mask.any()
    err = np.abs(gpu[mask] - ref[mask])
    scale = np.abs(ref[mask]).max()
    bound = min(OUT_ABS[dtype], OUT_REL_MAX[dtype] * max(scale, 1e-30) + (1e-7 if dtype == "f32" else 1e-6))
    assert np.isfinite(gpu[mask]).all(), f"{what}: non-finite values"
    assert err.max() <= bound, f"{what}: max abs err {err.max():.3e} > {bound:.3e} (max|ref| {scale:.3e})"
    return float(err.max())


def check_scores(gpu: np.ndarray, ref: np.ndarray, P: np.ndarray):
    worst = 0.0
    for b in range(len(P)):
        Pb = int(P[b])
        if Pb == 0:
            continue
        s, g = ref[b, :Pb], gpu[b, :Pb]
        rms = np.sqrt(np.mean(s * s))
        rel = np.abs(g - s) / np.maximum(np.abs(s), rms)
        worst = max(worst, float(rel.max()))
        assert rel.max() <= SCORE_REL, f"seq {b}: score rel err {rel.max():.3e}"
    return worst


def check_selection_band(gpu_idx: np.ndarray, ref_scores: np.ndarray, ref_idx: list, P: np.ndarray, k: np.ndarray):
    """Same set as the oracle except swaps among entries whose oracle score lies
    within 1e-3 (relative, per the score tolerance) of the k-th score."""
    n_swaps = 0
    for b in range(len(P)):
        Pb, kb = int(P[b]), min(int(k[b]), int(P[b]))
        g = gpu_idx[b]
        sel = g[:kb]
        assert (g[kb:] == -1).all(), f"seq {b}: padding not -1"
        assert (np.diff(sel) > 0).all() if kb > 1 else True, f"seq {b}: indices not increasing"
        o = set(ref_idx[b].tolist())
        gs = set(sel.tolist())
        assert len(gs) == kb
        if gs == o:
            continue
        s = ref_scores[b, :Pb]
        kth = np.sort(s)[::-1][kb - 1]
        rms = np.sqrt(np.mean(s * s))
        band = set(np.nonzero(np.abs(s - kth) <= SCORE_REL * max(abs(kth), rms))[0].tolist())
        assert gs - band == o - band, f"seq {b}: selection differs outside the tie band"
        n_swaps += len(gs ^ o) // 2
    return n_swaps
