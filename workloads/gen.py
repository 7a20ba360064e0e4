"""Seeded tensors for the five verification workloads and for custom shapes.

Storage conventions (shared by the oracle and the HIP path):

* ``dtype == "f32"``: float32 arrays.
* ``dtype == "bf16"``: uint16 arrays holding bfloat16 bit patterns, obtained by
  drawing float32 values and rounding them once, to nearest-even.
* K and V caches are token-major rows ``[slot][Hkv][D]``.  Contiguous layout:
  logical position i of sequence b lives in slot ``b * seq_stride + i``.  Paged
  layout: slot ``page_table[b][i // page_size] * page_size + i % page_size``.
* The N verify tokens of sequence b (the root/last committed token followed by
  the drafted nodes) have their own K/V at logical positions ``[P_b, P_b + N)``.

Value recipe: Q, K and V entries are N(0, sigma^2) with sigma = 1/sqrt(D);
K and V of sequence b are drawn in blocks of 16384 tokens, block j from its
own stream (seed, tensor, b, j), so generation can fill blocks in parallel.
Planted heavy keys (workloads 1, 2 and 4): a key chosen as heavy gets
``+c * sigma * u_{b,g}`` added in every KV head g, where ``u_{b,g}`` is the unit
vector along the sum of the sequence's scoring-row queries of the heads that
share KV head g.  This makes the planted keys heavy for the scoring queries
(with independent random directions they would not be).  Heavy positions are
drawn without replacement from ``[0, P - 64)``; workloads 2 and 4 also give the
64 most recent prefix keys ``+1 * sigma * u``.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional

import numpy as np

from .tree import best_first_tree, chain_parents, depth_logprobs

# generator stream ids (one stream per tensor)
_S_Q, _S_K, _S_V, _S_HEAVY, _S_TREE, _S_DQ, _S_LEN, _S_PAGES, _S_SCORES, _S_TAIL, _S_ACCEPT = range(11)

CONFIG_NAMES = {
    1: "tiny-fp32-chain-p512",
    2: "llama3-8b-layer-chain-c2q-p32768",
    3: "tree256-p8192",
    4: "long-ctx-b4-p131072-chain16",
    5: "mixed-paged-b16-tree64",
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    N: int                     # verify query nodes per sequence (root included)
    P: np.ndarray              # int32[B] prefix lengths
    P_max: int
    scale: float               # softmax scale 1/sqrt(D)
    layout: str                # "contiguous" or "paged"
    seq_stride: int            # contiguous: slots per sequence
    page_size: int             # paged: tokens per page
    page_table: Optional[np.ndarray]  # paged: int32[B][max_pages], -1 = unused
    num_slots: int
    q: np.ndarray              # [B][N][Hq][D]
    k: np.ndarray              # [num_slots][Hkv][D]
    v: np.ndarray              # [num_slots][Hkv][D]
    parent: Optional[np.ndarray]  # int32[B][N]; None = linear chain
    score_rows: np.ndarray     # int32[n_rows] verify rows whose logits are summed
    k_sel: np.ndarray          # int32[B] requested top-k per sequence
    dq: np.ndarray             # [S][B][Hq][D] draft-step queries (S may be 0)
    heavy: Optional[np.ndarray] = None  # planted heavy positions (shared by all b), for soft checks

    @property
    def max_pages(self) -> int:
        return 0 if self.page_table is None else int(self.page_table.shape[1])

    @property
    def k_max(self) -> int:
        return int(self.k_sel.max()) if self.B else 0

    def slot(self, b: int, i: np.ndarray) -> np.ndarray:
        """Storage slot of logical positions ``i`` of sequence ``b`` (layout bookkeeping only)."""
        i = np.asarray(i, dtype=np.int64)
        if self.layout == "contiguous":
            return b * self.seq_stride + i
        pt = self.page_table[b].astype(np.int64)
        return pt[i // self.page_size] * self.page_size + i % self.page_size


def _draw(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


_CHUNK = 16384  # tokens per independently seeded block of a K or V draw


def _pool():
    import concurrent.futures
    global _POOL
    if _POOL is None:
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


_POOL = None


def _draw_blocks(seed_words, shape, std: float) -> np.ndarray:
    """N(0, std^2) float32 array of `shape`, drawn in blocks of _CHUNK rows along
    axis 0, block j from its own stream SeedSequence(seed_words + [j]); the
    values depend only on the seed, not on how many threads fill them."""
    out = np.empty(shape, dtype=np.float32)
    n = shape[0]

    def fill(j):
        r = np.random.default_rng(np.random.SeedSequence([int(x) for x in seed_words] + [j]))
        blk = out[j * _CHUNK: min(n, (j + 1) * _CHUNK)]
        r.standard_normal(size=blk.shape, dtype=np.float32, out=blk)
        blk *= np.float32(std)

    list(_pool().map(fill, range((n + _CHUNK - 1) // _CHUNK)))
    return out


def _store_blocks(x: np.ndarray, dtype: str) -> np.ndarray:
    """_store applied block-wise in the thread pool (same result)."""
    if dtype == "f32" or x.shape[0] <= _CHUNK:
        return _store(x, dtype)
    out = np.empty(x.shape, dtype=np.uint16)

    def conv(j):
        sl = slice(j * _CHUNK, min(x.shape[0], (j + 1) * _CHUNK))
        out[sl] = bf16_bits_from_f32(x[sl])

    list(_pool().map(conv, range((x.shape[0] + _CHUNK - 1) // _CHUNK)))
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else bf16_bits_from_f32(x)


def _as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else f32_from_bf16_bits(x)


def make_custom(*, seed, B=1, Hq=4, Hkv=1, D=64, dtype="f32", P=512, N=5,
                tree=None, tree_depth=8, score_rows="all", k_sel=64, decode_steps=1,
                layout="contiguous", page_size=16, seq_extra=0,
                heavy_count=0, heavy_c=0.0, window=0, window_c=0.0,
                q_std_mult=1.0, v_canary=0.0, name="custom") -> Workload:
    """Build a workload with explicit parameters.

    ``P`` may be an int (same for all sequences) or a sequence of B ints.
    ``tree``: None for a linear chain, "best_first" for a best-first tree of N
    nodes (per sequence) with max depth ``tree_depth``, or an explicit parent
    array of shape [N] or [B][N].
    ``score_rows``: "all", "c2q" (rows {0, N-1}), or an explicit list.
    ``k_sel``: int, sequence of B ints, or "5pct" (max(1, floor(0.05 P_b))).
    ``q_std_mult``: multiplies the query std (1/sqrt(D) by default) -- values
    above 1 sharpen the attention.  ``v_canary``: if nonzero, the V rows of the
    N verify tokens are set to ``v_canary`` times distinct one-hot-like vectors,
    so that any leak through the tree mask moves outputs by O(v_canary).
    """
    ss = np.random.SeedSequence
    rng = lambda s: np.random.default_rng(ss([int(x) for x in np.atleast_1d(seed)] + [s]))  # noqa: E731
    if np.isscalar(P):
        Pb = np.full(B, int(P), dtype=np.int32)
    else:
        Pb = np.asarray(P, dtype=np.int32)
        assert Pb.shape == (B,)
    P_max = int(Pb.max()) if B else 0
    sigma = 1.0 / np.sqrt(D)
    L = Pb.astype(np.int64) + N  # logical tokens per sequence

    # ---- draft structure
    if tree is None:
        parent = None
    elif isinstance(tree, str) and tree == "best_first":
        parent = np.empty((B, N), dtype=np.int32)
        r = rng(_S_TREE)
        for b in range(B):
            lp = depth_logprobs(r, tree_depth)
            parent[b] = best_first_tree(N, lp, tree_depth)[0]
    else:
        pa = np.asarray(tree, dtype=np.int32)
        parent = np.broadcast_to(pa, (B, N)).copy() if pa.ndim == 1 else pa.copy()

    if isinstance(score_rows, str):
        if score_rows == "all":
            rows = np.arange(N, dtype=np.int32)
        elif score_rows == "c2q":
            rows = np.unique(np.array([0, N - 1], dtype=np.int32))
        else:
            raise ValueError(score_rows)
    else:
        rows = np.asarray(score_rows, dtype=np.int32)

    if isinstance(k_sel, str):
        assert k_sel == "5pct"
        ks = np.maximum(1, (Pb.astype(np.int64) * 5) // 100).astype(np.int32)
    elif np.isscalar(k_sel):
        ks = np.full(B, int(k_sel), dtype=np.int32)
    else:
        ks = np.asarray(k_sel, dtype=np.int32)

    # ---- queries
    qf = _draw(rng(_S_Q), (B, N, Hq, D), sigma * q_std_mult)
    q = _store(qf, dtype)
    qv = _as_f32(q, dtype)

    # ---- layout
    if layout == "contiguous":
        seq_stride = int(P_max + N + seq_extra)
        num_slots = B * seq_stride
        page_table = None
    elif layout == "paged":
        seq_stride = 0
        npages = (L + seq_extra + page_size - 1) // page_size  # seq_extra: mapped room past P_b + N
        total = int(npages.sum())
        perm = rng(_S_PAGES).permutation(total).astype(np.int32)
        max_pages = int(npages.max()) if B else 0
        page_table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            page_table[b, : npages[b]] = perm[off: off + npages[b]]
            off += int(npages[b])
        num_slots = total * page_size
    else:
        raise ValueError(layout)

    # ---- heavy positions (shared by all sequences and heads)
    heavy = None
    if heavy_count > 0:
        hi = max(1, P_max - 64)
        heavy = np.sort(rng(_S_HEAVY).choice(hi, size=min(heavy_count, hi), replace=False)).astype(np.int64)

    G = Hq // Hkv
    kstore = np.zeros((num_slots, Hkv, D), dtype=np.float32 if dtype == "f32" else np.uint16)
    vstore = np.zeros((num_slots, Hkv, D), dtype=kstore.dtype)
    seed_words = [int(x) for x in np.atleast_1d(seed)]
    for b in range(B):
        Lb = int(L[b])
        kb = _draw_blocks(seed_words + [_S_K, b], (Lb, Hkv, D), sigma)
        vb = _draw_blocks(seed_words + [_S_V, b], (Lb, Hkv, D), sigma)
        if heavy is not None or window > 0:
            # direction along the sum of the scoring rows' queries, per KV head
            qsum = qv[b][rows].reshape(len(rows), Hkv, G, D).sum(axis=(0, 2)).astype(np.float64)
            nrm = np.linalg.norm(qsum, axis=-1, keepdims=True)
            u = (qsum / np.where(nrm > 0, nrm, 1.0)).astype(np.float32)  # [Hkv][D]
            if heavy is not None:
                hb = heavy[heavy < Pb[b]]
                kb[hb] += np.float32(heavy_c * sigma) * u[None]
            if window > 0:
                lo = max(0, int(Pb[b]) - window)
                kb[lo: int(Pb[b])] += np.float32(window_c * sigma) * u[None]
        if v_canary:
            for t in range(N):
                vb[int(Pb[b]) + t] = 0.0
                vb[int(Pb[b]) + t, :, t % D] = np.float32(v_canary * (1.0 + t / N))
        slots = (b * seq_stride + np.arange(Lb)) if layout == "contiguous" else (
            page_table[b].astype(np.int64)[np.arange(Lb) // page_size] * page_size + np.arange(Lb) % page_size)
        kstore[slots] = _store_blocks(kb, dtype)
        vstore[slots] = _store_blocks(vb, dtype)

    dq = _store(_draw(rng(_S_DQ), (decode_steps, B, Hq, D), sigma * q_std_mult), dtype)

    return Workload(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, N=N, P=Pb, P_max=P_max,
                    scale=float(1.0 / np.sqrt(D)), layout=layout, seq_stride=seq_stride,
                    page_size=page_size, page_table=page_table, num_slots=num_slots,
                    q=q, k=kstore, v=vstore, parent=parent, score_rows=rows, k_sel=ks, dq=dq,
                    heavy=heavy)


def make_workload(cfg: int, seed: int = 0) -> Workload:
    """The five measured workloads at their full sizes."""
    name = CONFIG_NAMES[cfg]
    s = [cfg, seed]
    if cfg == 1:
        return make_custom(seed=s, B=1, Hq=4, Hkv=1, D=64, dtype="f32", P=512, N=5,
                           score_rows="all", k_sel=64, decode_steps=1,
                           heavy_count=16, heavy_c=3.0, name=name)
    if cfg == 2:
        return make_custom(seed=s, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=32768, N=8,
                           score_rows="c2q", k_sel=2048, decode_steps=1,
                           heavy_count=328, heavy_c=2.5, window=64, window_c=1.0, name=name)
    if cfg == 3:
        return make_custom(seed=s, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=8192, N=256,
                           tree="best_first", tree_depth=8, score_rows="all", k_sel=1024,
                           decode_steps=0, name=name)
    if cfg == 4:
        return make_custom(seed=s, B=4, Hq=32, Hkv=8, D=128, dtype="bf16", P=131072, N=16,
                           score_rows="c2q", k_sel=4096, decode_steps=15,
                           heavy_count=1311, heavy_c=2.5, window=64, window_c=1.0, name=name)
    if cfg == 5:
        lens = np.random.default_rng([cfg, seed, _S_LEN]).integers(4096, 65536, size=16, endpoint=True)
        return make_custom(seed=s, B=16, Hq=32, Hkv=8, D=128, dtype="bf16", P=lens, N=64,
                           tree="best_first", tree_depth=6, score_rows="all", k_sel="5pct",
                           decode_steps=1, layout="paged", page_size=16, name=name)
    raise ValueError(cfg)


def make_tail_rows(seed, steps: int, B: int, Hkv: int, D: int, dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """K and V rows of `steps` drafted tokens per sequence (their tail behind a
    compacted set), storage type, shape [steps][B][Hkv][D], N(0, 1/D) like the cache."""
    r = np.random.default_rng([int(x) for x in np.atleast_1d(seed)] + [_S_TAIL])
    sd = 1.0 / np.sqrt(D)
    k = _draw(r, (steps, B, Hkv, D), sd)
    v = _draw(r, (steps, B, Hkv, D), sd)
    return _store(k, dtype), _store(v, dtype)


def make_accept_tokens(seed, parent: np.ndarray, match_prob: float = 0.75,
                       vocab: int = 32000) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic drafted and target tokens for acceptance on draft trees.

    parent: int32 [B][N].  Drafted token of a node: distinct among siblings (a
    child's rank among its parent's children, offset by a per-parent random
    base, as the per-depth candidate lists of the tree generator give).
    Target token at a node: with probability ``match_prob`` the drafted token of
    one of its children (drawn uniformly), otherwise a token no drafted node
    carries (>= vocab).  Returns (draft, target), int32 [B][N] each."""
    r = np.random.default_rng([int(x) for x in np.atleast_1d(seed)] + [_S_ACCEPT])
    parent = np.asarray(parent, dtype=np.int32)
    B, N = parent.shape
    draft = np.zeros((B, N), dtype=np.int32)
    target = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        base = r.integers(0, vocab // 2, size=N)
        nkids = np.zeros(N, dtype=np.int64)
        kids = [[] for _ in range(N)]
        draft[b, 0] = int(r.integers(0, vocab))
        for t in range(1, N):
            p = int(parent[b, t])
            draft[b, t] = int((base[p] + nkids[p]) % vocab)
            nkids[p] += 1
            kids[p].append(t)
        for t in range(N):
            if kids[t] and r.random() < match_prob:
                target[b, t] = draft[b, kids[t][int(r.integers(0, len(kids[t])))]]
            else:
                target[b, t] = vocab + int(r.integers(0, vocab))
    return draft, target


def make_score_vector(seed: int, n: int, kind: str = "normal") -> np.ndarray:
    """Synthetic fp32 score rows for testing selection on its own.

    kinds: "normal" (N(0,1)), "ties" (small integers, many exact ties),
    "signed_zero" (mix of +0.0, -0.0 and a few nonzeros), "constant" (all equal),
    "wide" (values spread over many binades, both signs).
    """
    r = np.random.default_rng([seed, _S_SCORES])
    if kind == "normal":
        return r.standard_normal(n).astype(np.float32)
    if kind == "ties":
        return r.integers(-4, 5, size=n).astype(np.float32)
    if kind == "signed_zero":
        x = np.where(r.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        m = r.random(n) < 0.05
        x[m] = r.standard_normal(int(m.sum())).astype(np.float32)
        return x
    if kind == "constant":
        return np.full(n, 1.5, dtype=np.float32)
    if kind == "wide":
        return (r.standard_normal(n) * np.exp2(r.integers(-40, 40, size=n))).astype(np.float32)
    raise ValueError(kind)
