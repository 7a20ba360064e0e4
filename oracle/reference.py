"""Plain float64 definitions of verification attention, logit scores, top-k
selection and sparse draft attention (test infrastructure; see package docstring).

Readings taken where the pages are silent (each also listed in the design notes):

* softmax scale is 1/sqrt(D); a "logit" is the softmax argument scale * q . k
  (Vegas §3, the instrumented kernel writes attention logits before the
  softmax normalisation);
* grouped-query attention: query head h reads KV head floor(h / (Hq/Hkv));
* a tree node attends to the whole prefix, to its ancestors and to itself
  (JETFLOW §2, tree causal attention mask); a linear chain is the tree whose
  node i has parent i-1, which makes the mask ordinary causal attention;
* the score of prefix entry i is the sum, over the chosen scoring rows and over
  ALL query heads, of the logits of entry i (Vegas §2.A, selection equation);
  only prefix entries (i < P_b) are scored, since the selected set is a subset
  of the prefix;
* selection keeps min(k, P_b) entries with the largest score, ties going to the
  lower index, returned in increasing index order;
* the draft step attends to exactly the given index list (Vegas §3, sparse
  execution with one-token pages whose page indices are token indices).

Pins (tests/test_oracle_*.py):
  bf16_bits_to_f64     -- values the bfloat16 format fixes (1.0, -2.5, -0.0, the
                          largest finite, the smallest normal and subnormal,
                          infinities); all 65536 patterns == torch's own
                          bfloat16 -> float64 conversion
  ancestors            -- brute-force reachability, hand-made golden trees
  verify_attention     -- torch SDPA (float64, explicit boolean mask); chain ==
                          separately written triangular mask; golden 2-key case;
                          GQA == MHA with repeated K/V; paged == contiguous;
                          star tree == prefix + root + self; N = 1 == decode
  verify_scores        -- closed form scale * sum_g K_g . qbar_g; golden values;
                          linearity; all-rows == union of per-row scores
  verify_scores_grouped -- equal to verify_scores (relative 1e-12) on the pin cases
  topk_select          -- brute-force enumeration of all k-subsets (Vegas §2.A
                          argmax) on tiny inputs with exact ties; golden cases
  sparse_draft_attention -- idx = whole prefix == dense decode; permutation
                          invariance; golden 2-key case
  verify_scores_per_head -- summed over the KV heads == verify_scores; one KV
                          head == verify_scores
  sparse_draft_attention_per_head -- the same list for every head ==
                          sparse_draft_attention
  sink_window_select   -- written out by hand on small cases
  build_best_first_tree -- brute force: node i is the i-th best of every node
                          reachable within the depth limit; golden tie order;
                          equal to the input generator's trees
  greedy_accept        -- chain closed form (leading matches); brute force on
                          trees (the deepest node whose whole branch matches)
  commit_accepted_kv   -- every moved row equals its source row, nothing else
                          changes
  tpt                  -- alpha = 0, alpha = 1 and gamma = 0 closed forms; the
                          expected-token factor == an explicit sum of alpha^i
                          for i = 0..gamma
  compact_kv, dense_draft_attention -- compacted rows == sparse_draft_attention
                          over the same list; a tail == the tail rows placed in
                          a cache past the prefix and listed; one row == its V
                          row exactly; row-permutation invariance
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# storage helpers (the oracle's own; the HIP path has its own conversions)

def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns stored as uint16."""
    w = np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def _f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


class KVCache:
    """Token-major K/V storage [slot][Hkv][D] plus the slot of each logical position.

    Contiguous: slot = b * seq_stride + i.  Paged: slot = page_table[b][i // ps] * ps + i % ps
    (JETFLOW §3 item 3 and Vegas §3 both run on a paged KV cache).
    """

    def __init__(self, k, v, dtype: str, layout: str = "contiguous", seq_stride: int = 0,
                 page_size: int = 1, page_table: Optional[np.ndarray] = None):
        self.k, self.v, self.dtype = k, v, dtype
        self.layout, self.seq_stride = layout, int(seq_stride)
        self.page_size, self.page_table = int(page_size), page_table

    @classmethod
    def of(cls, wl) -> "KVCache":
        return cls(wl.k, wl.v, wl.dtype, wl.layout, wl.seq_stride, wl.page_size, wl.page_table)

    def slots(self, b: int, pos: np.ndarray) -> np.ndarray:
        pos = np.asarray(pos, dtype=np.int64)
        if self.layout == "contiguous":
            return b * self.seq_stride + pos
        pt = np.asarray(self.page_table[b], dtype=np.int64)
        return pt[pos // self.page_size] * self.page_size + pos % self.page_size

    def keys(self, b: int, g: int, pos) -> np.ndarray:
        """float64 [len(pos)][D] keys of KV head g at logical positions pos."""
        return _f64(self.k[self.slots(b, pos), g], self.dtype)

    def values(self, b: int, g: int, pos) -> np.ndarray:
        return _f64(self.v[self.slots(b, pos), g], self.dtype)


# ----------------------------------------------------------------------------
# tree mask (JETFLOW §2, tree causal attention mask)

def ancestors(parent: Optional[np.ndarray], t: int) -> list[int]:
    """Node t and all its ancestors, found by walking parent pointers up to the root.

    ``parent is None`` means a linear chain (parent of i is i - 1).
    """
    out = []
    a = int(t)
    while a != -1:
        out.append(a)
        a = (a - 1) if parent is None else int(parent[a])
    return out


def visible_positions(P_b: int, parent: Optional[np.ndarray], t: int) -> np.ndarray:
    """Logical KV positions verify node t may attend to: the whole prefix
    [0, P_b) and the verify tokens of its ancestors and itself, which sit at
    P_b + node index (JETFLOW §2 tree mask; no siblings, no descendants)."""
    anc = sorted(ancestors(parent, t))
    return np.concatenate([np.arange(P_b, dtype=np.int64), P_b + np.asarray(anc, dtype=np.int64)])


# ----------------------------------------------------------------------------
# verification attention (Vegas §2 "Mecanismo Central" step 1; lossless: §5)

def _softmax_attend(logits: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """o = sum_j softmax(logits)_j v_j, logits [n] or [n][m] (columns independent)."""
    m = logits.max(axis=0)
    p = np.exp(logits - m)
    return (p / p.sum(axis=0)).T @ vals


def verify_attention(q: np.ndarray, dtype: str, kv: KVCache, P: np.ndarray,
                     parent: Optional[np.ndarray], scale: float, Hkv: int,
                     rows: Optional[Sequence[tuple]] = None) -> np.ndarray:
    """Full (dense) masked softmax attention of every verify query.

    q: [B][N][Hq][D] storage.  For sequence b, node t, head h (KV head
    g = h // (Hq/Hkv)): logits l_j = scale * q_{b,t,h} . k_{b,j,g} over the
    visible positions j, o = sum_j softmax(l)_j v_{b,j,g}.

    Returns float64 [B][N][Hq][D]; with ``rows`` = list of (b, t, h), only those
    entries are computed (others are NaN), for sampled checks at large sizes.
    """
    qf = _f64(q, dtype)
    B, N, Hq, D = qf.shape
    G = Hq // Hkv
    out = np.full((B, N, Hq, D), np.nan)
    want = None if rows is None else {}
    if rows is not None:
        for (b, t, h) in rows:
            want.setdefault((int(b), int(h) // G), set()).add((int(t), int(h)))
    for b in range(B):
        Pb = int(P[b])
        for g in range(Hkv):
            if want is not None and (b, g) not in want:
                continue
            allpos = np.arange(Pb + N)
            Kg = kv.keys(b, g, allpos)
            Vg = kv.values(b, g, allpos)
            pb = None if parent is None else parent[b]
            for t in range(N):
                heads = [h for h in range(g * G, (g + 1) * G)
                         if want is None or (t, h) in want[(b, g)]]
                if not heads:
                    continue
                vis = visible_positions(Pb, pb, t)
                lg = scale * (Kg[vis] @ qf[b, t, heads].T)          # [n_vis][len(heads)]
                out[b, t, heads] = _softmax_attend(lg, Vg[vis])
    return out


# ----------------------------------------------------------------------------
# criticality scores (Vegas §2.A selection equation; §2.B Collect-2-Query
# picks which rows are summed; §2.A "Razão": rejected drafts count too)

def verify_scores(q: np.ndarray, dtype: str, kv: KVCache, P: np.ndarray,
                  score_rows: Sequence[int], scale: float, Hkv: int,
                  P_max: Optional[int] = None) -> np.ndarray:
    """s_{b,i} = sum_{t in score_rows} sum_{h < Hq} scale * q_{b,t,h} . k_{b,i,g(h)}, i < P_b.

    Returns float64 [B][P_max]; entries i >= P_b are NaN (not scored).
    """
    qf = _f64(q, dtype)
    B, N, Hq, D = qf.shape
    G = Hq // Hkv
    if P_max is None:
        P_max = int(np.max(P)) if B else 0
    s = np.full((B, P_max), np.nan)
    rows = [int(t) for t in score_rows]
    for b in range(B):
        Pb = int(P[b])
        acc = np.zeros(Pb)
        for g in range(Hkv):
            Kg = kv.keys(b, g, np.arange(Pb))                      # [Pb][D]
            for t in rows:
                for h in range(g * G, (g + 1) * G):
                    acc += scale * (Kg @ qf[b, t, h])              # logits of entry i for (t, h)
        s[b, :Pb] = acc
    return s


def verify_scores_grouped(q: np.ndarray, dtype: str, kv: KVCache, P: np.ndarray,
                          score_rows: Sequence[int], scale: float, Hkv: int,
                          P_max: Optional[int] = None) -> np.ndarray:
    """The same sum as verify_scores, grouped: every logit is linear in q, so
    the sum over rows t and the heads h of KV group g can be taken over the
    queries first, s_{b,i} = scale * sum_g k_{b,i,g} . (sum_{t, h in g} q_{b,t,h}).
    One product per (sequence, KV head) instead of one per (row, head), which
    makes full-size checks affordable; pinned to verify_scores on small inputs."""
    qf = _f64(q, dtype)
    B, N, Hq, D = qf.shape
    G = Hq // Hkv
    if P_max is None:
        P_max = int(np.max(P)) if B else 0
    s = np.full((B, P_max), np.nan)
    rows = [int(t) for t in score_rows]
    for b in range(B):
        Pb = int(P[b])
        acc = np.zeros(Pb)
        for g in range(Hkv):
            qsum = qf[b, rows][:, g * G:(g + 1) * G].sum(axis=(0, 1))   # [D]
            acc += scale * (kv.keys(b, g, np.arange(Pb)) @ qsum)
        s[b, :Pb] = acc
    return s


# ----------------------------------------------------------------------------
# top-k selection (Vegas §2 step 2 and §2.A: T = argmax over |T| = k subsets)

def topk_select(scores_row: np.ndarray, P_b: int, k: int) -> np.ndarray:
    """Indices of the min(k, P_b) largest scores among entries [0, P_b).

    Maximising the sum over a k-subset is the same as keeping the k largest
    entries; equal scores are ordered by lower index first (so -0.0 and +0.0
    compare equal).  Full stable sort, then the chosen indices in increasing order.
    """
    kk = max(0, min(int(k), int(P_b)))
    s = np.asarray(scores_row[:P_b], dtype=np.float64)
    idx = np.arange(P_b)
    order = np.lexsort((idx, -s))
    return np.sort(order[:kk]).astype(np.int64)


# ----------------------------------------------------------------------------
# sparse draft attention (Vegas §2 step 3; §3 sparse execution, page size 1)

def sparse_draft_attention(q1: np.ndarray, dtype: str, kv: KVCache,
                           idx: Sequence[np.ndarray], scale: float, Hkv: int) -> np.ndarray:
    """One draft query per sequence attending to exactly the keys idx[b].

    q1: [B][Hq][D] storage.  Returns float64 [B][Hq][D]; an empty index list gives 0.
    """
    qf = _f64(q1, dtype)
    B, Hq, D = qf.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        ib = np.asarray(idx[b], dtype=np.int64)
        if ib.size == 0:
            continue
        for g in range(Hkv):
            Kg = kv.keys(b, g, ib)
            Vg = kv.values(b, g, ib)
            hs = list(range(g * G, (g + 1) * G))
            lg = scale * (Kg @ qf[b, hs].T)                        # [n][G]
            out[b, hs] = _softmax_attend(lg, Vg)
    return out


# ----------------------------------------------------------------------------
# selection variants: one key set per KV head (the score of Vegas §2.A summed
# over the query heads of one group only), and a query-agnostic sink + recent
# window (the selector the Vegas results section compares against)

def verify_scores_per_head(q: np.ndarray, dtype: str, kv: KVCache, P: np.ndarray,
                           score_rows: Sequence[int], scale: float, Hkv: int,
                           P_max: Optional[int] = None) -> np.ndarray:
    """s_{b,g,i} = sum_{t in score_rows} sum_{h in group g} scale * q_{b,t,h} . k_{b,i,g}, i < P_b.

    Returns float64 [B][Hkv][P_max]; entries i >= P_b are NaN."""
    qf = _f64(q, dtype)
    B, N, Hq, D = qf.shape
    G = Hq // Hkv
    if P_max is None:
        P_max = int(np.max(P)) if B else 0
    s = np.full((B, Hkv, P_max), np.nan)
    rows = [int(t) for t in score_rows]
    for b in range(B):
        Pb = int(P[b])
        for g in range(Hkv):
            Kg = kv.keys(b, g, np.arange(Pb))
            acc = np.zeros(Pb)
            for t in rows:
                for h in range(g * G, (g + 1) * G):
                    acc += scale * (Kg @ qf[b, t, h])
            s[b, g, :Pb] = acc
    return s


def sparse_draft_attention_per_head(q1: np.ndarray, dtype: str, kv: KVCache,
                                    idx: Sequence[Sequence[np.ndarray]], scale: float, Hkv: int) -> np.ndarray:
    """One draft query per sequence; the query heads of KV group g attend to
    exactly the keys idx[b][g].  Returns float64 [B][Hq][D]; an empty list gives 0."""
    qf = _f64(q1, dtype)
    B, Hq, D = qf.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for g in range(Hkv):
            ib = np.asarray(idx[b][g], dtype=np.int64)
            if ib.size == 0:
                continue
            hs = list(range(g * G, (g + 1) * G))
            lg = scale * (kv.keys(b, g, ib) @ qf[b, hs].T)
            out[b, hs] = _softmax_attend(lg, kv.values(b, g, ib))
    return out


def sink_window_select(P_b: int, sink: int, window: int) -> np.ndarray:
    """The first `sink` and the last `window` prefix positions, increasing."""
    keep = set(range(min(sink, P_b))) | set(range(max(0, P_b - window), P_b))
    return np.asarray(sorted(keep), dtype=np.int64)


# ----------------------------------------------------------------------------
# draft loop over a compacted KV: the draft model's attention runs once per
# draft token over the same selected set (Vegas §2 step 3; §3, where the sparse
# kernel is called several times per step), so the selected rows are gathered
# once into a dense buffer, and each draft token's own K/V row is appended
# behind them (its tail) before its decode attends to all rows so far

def compact_kv(kv: KVCache, idx: Sequence[np.ndarray], cap: int) -> tuple[np.ndarray, np.ndarray]:
    """Dense K and V buffers [B][cap][Hkv][D] in the cache's storage type: row j
    of sequence b is the row of logical position idx[b][j] (all KV heads);
    rows from len(idx[b]) on are zero."""
    B = len(idx)
    Hkv, D = kv.k.shape[1], kv.k.shape[2]
    ck = np.zeros((B, cap, Hkv, D), dtype=kv.k.dtype)
    cv = np.zeros((B, cap, Hkv, D), dtype=kv.v.dtype)
    for b in range(B):
        ib = np.asarray(idx[b], dtype=np.int64)[:cap]
        if ib.size:
            sl = kv.slots(b, ib)
            ck[b, : ib.size] = kv.k[sl]
            cv[b, : ib.size] = kv.v[sl]
    return ck, cv


def dense_draft_attention(q1: np.ndarray, dtype: str, ck: np.ndarray, cv: np.ndarray,
                          n_rows: Sequence[int], scale: float, Hkv: int) -> np.ndarray:
    """One query per sequence attending to rows [0, n_rows[b]) of dense K/V
    buffers [B][cap][Hkv][D] (the compacted set and the draft tail).

    q1: [B][Hq][D] storage.  Returns float64 [B][Hq][D]; n_rows[b] = 0 gives 0.
    """
    qf = _f64(q1, dtype)
    B, Hq, D = qf.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(n_rows[b])
        if n <= 0:
            continue
        for g in range(Hkv):
            Kg = _f64(ck[b, :n, g], dtype)
            Vg = _f64(cv[b, :n, g], dtype)
            hs = list(range(g * G, (g + 1) * G))
            out[b, hs] = _softmax_attend(scale * (Kg @ qf[b, hs].T), Vg)
    return out


# ----------------------------------------------------------------------------
# draft tree construction (JETFLOW §2, tree construction: the draft head gives
# log-probabilities for every depth at once, a branch is scored by its
# cumulative draft log-probability, and best-first expansion grows the tree up
# to a node budget)

def build_best_first_tree(lp: np.ndarray, n_nodes: int, max_depth: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """lp: float64 [max_depth + 1][n_cand], row d the candidate log-probs at
    depth d in decreasing order (row 0 unused).  Node 0 is the root.  A
    candidate is (parent node, rank) at depth(parent) + 1 with score
    cum(parent) + lp[depth][rank]; the best candidate (highest score, then
    lower parent id, then lower rank) becomes the next node.  A new node offers
    its rank-0 child; a taken candidate offers its parent's next rank (the
    lists are sorted, so the untaken ranks of a parent are never better than
    the next one).  Returns (parent, depth, rank), int32 [n_nodes] each."""
    n_cand = lp.shape[1]
    parent, depth, rank, cum = [-1], [0], [0], [0.0]
    cands = []  # (score, parent, rank, depth)
    if n_nodes > 1 and max_depth >= 1:
        cands.append((0.0 + float(lp[1][0]), 0, 0, 1))
    while len(parent) < n_nodes:
        best = min(range(len(cands)), key=lambda j: (-cands[j][0], cands[j][1], cands[j][2]))
        sc, p, r, d = cands.pop(best)
        i = len(parent)
        parent.append(p)
        depth.append(d)
        rank.append(r)
        cum.append(sc)
        if d < max_depth:
            cands.append((sc + float(lp[d + 1][0]), i, 0, d + 1))
        if r + 1 < n_cand:
            cands.append((cum[p] + float(lp[d][r + 1]), p, r + 1, d))
    return (np.asarray(parent, dtype=np.int32), np.asarray(depth, dtype=np.int32), np.asarray(rank, dtype=np.int32))


# ----------------------------------------------------------------------------
# acceptance after verification and the accepted path's KV (Vegas §2: draft,
# verify, accept; JETFLOW §2: a tree node's token is conditioned on its own
# branch, so an accepted path is one root-to-node branch of the tree)

def greedy_accept(parent: Optional[np.ndarray], draft: np.ndarray, target: np.ndarray) -> list[int]:
    """Accepted path of one sequence, root first.  target[t] is the target
    model's token after node t (its greedy choice); from the root, the path
    moves to a child whose drafted token equals the target token at the
    current node, the lowest-index one if several do, and stops when none does.
    ``parent is None``: a linear chain."""
    N = len(draft)
    path = [0]
    cur = 0
    while True:
        nxt = None
        for c in range(cur + 1, N):
            pc = (c - 1) if parent is None else int(parent[c])
            if pc == cur and int(draft[c]) == int(target[cur]):
                nxt = c
                break
        if nxt is None:
            return path
        path.append(nxt)
        cur = nxt


def commit_accepted_kv(kv: KVCache, b: int, P_b: int, path: Sequence[int]) -> None:
    """Moves the accepted path's K/V rows to consecutive positions, in place on
    kv.k / kv.v: after the call, logical position P_b + d holds the row that
    position P_b + path[d] held before (d = 1 .. len(path) - 1; the root stays
    at P_b).  The committed prefix then ends at P_b + len(path)."""
    src = kv.slots(b, P_b + np.asarray(path[1:], dtype=np.int64))
    dst = kv.slots(b, P_b + np.arange(1, len(path), dtype=np.int64))
    krows, vrows = kv.k[src].copy(), kv.v[src].copy()
    kv.k[dst] = krows
    kv.v[dst] = vrows


# ----------------------------------------------------------------------------

def run_step(wl, rows=None, decode_step: int = 0, with_attention: bool = True) -> dict:
    """One pass of the hot path on a workload object (duck-typed: the attributes
    produced by the seeded generators).  Verify -> scores -> top-k -> sparse draft."""
    kv = KVCache.of(wl)
    res = {}
    if with_attention:
        res["out"] = verify_attention(wl.q, wl.dtype, kv, wl.P, wl.parent, wl.scale, wl.Hkv, rows=rows)
    res["scores"] = verify_scores(wl.q, wl.dtype, kv, wl.P, wl.score_rows, wl.scale, wl.Hkv, wl.P_max)
    res["idx"] = [topk_select(res["scores"][b], int(wl.P[b]), int(wl.k_sel[b])) for b in range(wl.B)]
    if wl.dq.shape[0] > decode_step:
        res["draft"] = sparse_draft_attention(wl.dq[decode_step], wl.dtype, kv, res["idx"], wl.scale, wl.Hkv)
    return res


# ----------------------------------------------------------------------------
# Tokens per time (KnapSpec §2, the TPT metric): with acceptance rate alpha and
# draft length gamma, a draft-verify round yields (1 - alpha^(gamma+1)) /
# (1 - alpha) tokens in expectation and costs gamma draft steps plus one
# target (verification) pass.  At alpha = 1 the factor is its limit gamma + 1.

def tpt(alpha: float, gamma: int, t_draft: float, t_target: float) -> float:
    """Tokens per unit of time (the unit of t_draft and t_target)."""
    alpha = float(alpha)
    if alpha == 1.0:
        tokens = float(gamma + 1)
    else:
        tokens = (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)
    return tokens / (gamma * float(t_draft) + float(t_target))
