"""Helpers for the GPU parity tests: move seeded workloads to the device, run
the HIP path through the C ABI binding, and compare with the oracle under the
stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import tree_verify_sparse_amd as sv

# tolerances.  Outputs: max-abs OUT_ABS (and, on sharp and canary cases,
# OUT_REL_MAX of max|o_ref|), plus for bf16 the per-element bound derived from
# the kernels' roundings (check_out_derived).  Scores: |s_gpu - s| <= SCORE_REL
# |s| + a floor from fp32 rounding (score_floor).  Selection: swaps only among
# entries within SCORE_REL |s_k| of the k-th score.
OUT_ABS = {"bf16": 2e-2, "f32": 1e-4}
OUT_REL_MAX = {"bf16": 2e-2, "f32": 1e-4}   # relative to max |o_ref| of the compared set
SCORE_REL = 1e-3
U_F32 = 2.0 ** -24    # unit roundoff of float32 (24-bit significand)
U_BF16 = 2.0 ** -8    # unit roundoff of bfloat16 (8-bit significand)


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


def abs_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """|x| in the same storage format (bf16: the sign bit cleared, which is exact)."""
    if dtype == "bf16":
        return np.asarray(x).view(np.uint16) & np.uint16(0x7FFF)
    return np.abs(np.asarray(x, dtype=np.float32))


def _abs_cache(wl, k_abs: bool, v_abs: bool):
    from oracle import KVCache as OKV
    k = abs_storage(wl.k, wl.dtype) if k_abs else wl.k
    v = abs_storage(wl.v, wl.dtype) if v_abs else wl.v
    return OKV(k, v, wl.dtype, wl.layout, wl.seq_stride, wl.page_size, wl.page_table)


def attention_abs(wl, rows=None) -> np.ndarray:
    """sum_j softmax(l)_j |v_j| per output element: the oracle's attention with |V|.
    Rounding the softmax weights or an unnormalised partial sum to bf16 moves an
    output element by at most u_bf16 times this."""
    import oracle
    return oracle.verify_attention(wl.q, wl.dtype, _abs_cache(wl, False, True), wl.P, wl.parent, wl.scale, wl.Hkv,
                                   rows=rows)


def sparse_abs(wl, q1, idx, per_head=False) -> np.ndarray:
    import oracle
    kv = _abs_cache(wl, False, True)
    if per_head:
        return oracle.sparse_draft_attention_per_head(q1, wl.dtype, kv, idx, wl.scale, wl.Hkv)
    return oracle.sparse_draft_attention(q1, wl.dtype, kv, idx, wl.scale, wl.Hkv)


# Per-element error bounds of the bf16 paths, from their roundings:
#   verify kernels and the dense draft decode: softmax weights rounded to bf16
#     for the P V product (u_bf16 * attention_abs), the unnormalised chunk
#     partials stored in bf16 (another u_bf16 * attention_abs), the output
#     rounded to bf16 (u_bf16 * |o|);
#   sparse draft step: fp32 weights and partials, only the output rounding.
# fp32 accumulation (at most 4096 keys per chunk, gamma_4096 u_f32 < 2^-12) and
# the exp2 and rescale roundings are covered by a 2^-12 * attention_abs slack.
DERIVED = {"verify": (U_BF16, 2 * U_BF16), "sparse": (U_BF16, 0.0)}
DERIVED_SLACK = 2.0 ** -12


def check_out_derived(gpu: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray, path: str, what="out"):
    """bf16 outputs against the rounding-derived bound a |o| + c abs_attention + slack."""
    a, c = DERIVED[path]
    mask = ~np.isnan(ref)
    err = np.abs(gpu[mask] - ref[mask])
    bound = a * np.abs(ref[mask]) + (c + DERIVED_SLACK) * ref_abs[mask] + 1e-9
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{what}: error exceeds the bf16 rounding bound by {worst:.2f}x"
    return worst


def score_floor(wl, rows=None, per_head=False) -> np.ndarray:
    """Absolute floor of the score check: fp32 rounding of the score's sums.
    With a_i = scale sum_{t, h, d} |q_{t,h,d}| |k_{i,g(h),d}| (the oracle's score
    on |q| and |k|) and n the rounding steps behind one score (the query sum of
    the scoring (row, head) pairs, the 3 D products of the split score operand,
    the sum over KV heads), the rounding error stays below 4 sqrt(n) u_f32 a_i
    (a probabilistic bound: independent roundings add like a random walk)."""
    import oracle
    rows = wl.score_rows if rows is None else rows
    G = wl.Hq // wl.Hkv
    qa = abs_storage(wl.q, wl.dtype)
    kv = _abs_cache(wl, True, False)
    if per_head:
        a = oracle.verify_scores_per_head(qa, wl.dtype, kv, wl.P, rows, wl.scale, wl.Hkv, wl.P_max)
    else:
        a = oracle.verify_scores_grouped(qa, wl.dtype, kv, wl.P, rows, wl.scale, wl.Hkv, wl.P_max)
    n = len(rows) * G + 3 * wl.D + wl.Hkv + 4
    return 4.0 * np.sqrt(n) * U_F32 * a


def check_scores(gpu: np.ndarray, ref: np.ndarray, P: np.ndarray, floor: np.ndarray):
    """|s_gpu - s| <= SCORE_REL |s| + floor per entry; returns (worst relative
    error, entries where the floor was needed)."""
    worst, by_floor = 0.0, 0
    for b in range(len(P)):
        Pb = int(P[b])
        if Pb == 0:
            continue
        s, g, f = ref[b, :Pb], gpu[b, :Pb], floor[b, :Pb]
        err = np.abs(g - s)
        assert (err <= SCORE_REL * np.abs(s) + f).all(), \
            f"seq {b}: score error {(err / (SCORE_REL * np.abs(s) + f)).max():.2f}x the bound"
        by_floor += int((err > SCORE_REL * np.abs(s)).sum())
        worst = max(worst, float((err / np.maximum(np.abs(s), 1e-30)).max()))
    return worst, by_floor


def check_selection_band(gpu_idx: np.ndarray, ref_scores: np.ndarray, ref_idx: list, P: np.ndarray, k: np.ndarray):
    """Same set as the oracle except swaps among entries whose oracle score lies
    within 1e-3 of the k-th score, relative to the k-th score."""
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
        band = set(np.nonzero(np.abs(s - kth) <= SCORE_REL * abs(kth))[0].tolist())
        assert gs - band == o - band, f"seq {b}: selection differs outside the tie band"
        n_swaps += len(gs ^ o) // 2
    return n_swaps
