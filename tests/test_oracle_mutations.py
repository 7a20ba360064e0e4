"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatching) and
check that at least one pin catches each of them."""
import numpy as np

import oracle
import oracle.reference as ref
from tests import test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(ref, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(check, *args):
    try:
        check(*args)
    except AssertionError:
        return True
    return False


def test_ancestors_without_self_is_caught(monkeypatch):
    orig = ref.ancestors
    _patch(monkeypatch, "ancestors", lambda parent, t: orig(parent, t)[1:])
    assert _fails(pins.test_golden_tree_uniform)


def test_ancestors_with_siblings_is_caught(monkeypatch):
    def leaky(parent, t):
        out, x = [], int(t)
        while x != -1:
            out.append(x)
            x = (x - 1) if parent is None else int(parent[x])
        if parent is not None and t > 0:      # also sees the previous node (a sibling or cousin)
            out.append(t - 1)
        return sorted(set(out))
    _patch(monkeypatch, "ancestors", leaky)
    assert _fails(pins.test_golden_tree_uniform)


def test_prefix_off_by_one_is_caught(monkeypatch):
    def vis(P_b, parent, t):
        anc = sorted(ref.ancestors(parent, t))
        return np.concatenate([np.arange(max(P_b - 1, 0)), P_b + np.asarray(anc, dtype=np.int64)])
    _patch(monkeypatch, "visible_positions", vis)
    assert _fails(pins.test_golden_attention_three_keys)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    orig_keys = ref.KVCache.keys

    def keys_interleaved(self, b, g, pos):
        # a mistaken layout reading heads as if h % Hkv mapped to g: swap KV heads 0 and 1
        Hkv = self.k.shape[1]
        return orig_keys(self, b, (g + 1) % Hkv if Hkv > 1 else g, pos)
    monkeypatch.setattr(ref.KVCache, "keys", keys_interleaved)
    case = dict(dtype="bf16", B=2, Hq=8, Hkv=2, D=128, P=[200, 333], N=7, tree="best_first", tree_depth=4)
    assert _fails(pins.test_verify_matches_torch_sdpa, case)


def test_scores_missing_scale_is_caught(monkeypatch):
    orig = ref.verify_scores

    def unscaled(q, dtype, kv, P, rows, scale, Hkv, P_max=None):
        return orig(q, dtype, kv, P, rows, 1.0, Hkv, P_max)
    _patch(monkeypatch, "verify_scores", unscaled)
    assert _fails(pins.test_golden_scores_small)
    assert _fails(pins.test_scores_closed_form, dict(dtype="f32", B=1, Hq=4, Hkv=1, D=64, P=77, N=5,
                                                     score_rows="all"))


def test_scores_one_head_per_group_is_caught(monkeypatch):
    def first_head_only(q, dtype, kv, P, rows, scale, Hkv, P_max=None):
        qf = ref._f64(q, dtype)
        B, N, Hq, D = qf.shape
        G = Hq // Hkv
        s = np.full((B, P_max or int(np.max(P))), np.nan)
        for b in range(B):
            Pb = int(P[b])
            acc = np.zeros(Pb)
            for g in range(Hkv):
                Kg = kv.keys(b, g, np.arange(Pb))
                for t in rows:
                    acc += scale * (Kg @ qf[b, t, g * G])
            s[b, :Pb] = acc
        return s
    _patch(monkeypatch, "verify_scores", first_head_only)
    assert _fails(pins.test_golden_scores_small)


def test_topk_ties_to_higher_index_is_caught(monkeypatch):
    def hi_ties(scores_row, P_b, k):
        kk = max(0, min(int(k), int(P_b)))
        s = np.asarray(scores_row[:P_b], dtype=np.float64)
        order = np.lexsort((-np.arange(P_b), -s))
        return np.sort(order[:kk])
    _patch(monkeypatch, "topk_select", hi_ties)
    assert _fails(pins.test_golden_topk_ties)
    assert any(_fails(pins.test_topk_brute_force, seed) for seed in range(30))


def test_sparse_drops_last_index_is_caught(monkeypatch):
    orig = ref.sparse_draft_attention

    def drop_last(q1, dtype, kv, idx, scale, Hkv):
        return orig(q1, dtype, kv, [np.asarray(i)[:-1] for i in idx], scale, Hkv)
    _patch(monkeypatch, "sparse_draft_attention", drop_last)
    assert _fails(pins.test_golden_sparse_two_keys)


def test_dense_draft_drops_last_row_is_caught(monkeypatch):
    orig = ref.dense_draft_attention

    def drop_last(q1, dtype, ck, cv, n_rows, scale, Hkv):
        return orig(q1, dtype, ck, cv, [max(0, int(n) - 1) for n in n_rows], scale, Hkv)
    _patch(monkeypatch, "dense_draft_attention", drop_last)
    assert _fails(pins.test_compacted_draft_equals_sparse_list, "bf16", "contiguous")


def test_compact_shifted_rows_is_caught(monkeypatch):
    orig = ref.compact_kv

    def shifted(kv, idx, cap):  # gathers the position after each listed one
        return orig(kv, [np.asarray(i) + 1 for i in idx], cap)
    _patch(monkeypatch, "compact_kv", shifted)
    assert _fails(pins.test_compacted_draft_equals_sparse_list, "bf16", "contiguous")


def test_accept_compares_child_target_is_caught(monkeypatch):
    def wrong(parent, draft, target):  # compares the child's drafted token with the child's own target
        N = len(draft)
        path, cur = [0], 0
        while True:
            nxt = None
            for c in range(cur + 1, N):
                pc = (c - 1) if parent is None else int(parent[c])
                if pc == cur and int(draft[c]) == int(target[c]):
                    nxt = c
                    break
            if nxt is None:
                return path
            path.append(nxt)
            cur = nxt
    _patch(monkeypatch, "greedy_accept", wrong)
    assert _fails(pins.test_greedy_accept_golden)


def test_commit_off_by_one_is_caught(monkeypatch):
    orig = ref.commit_accepted_kv

    def shifted(kv, b, P_b, path):
        return orig(kv, b, P_b - 1, path)
    _patch(monkeypatch, "commit_accepted_kv", shifted)
    assert _fails(pins.test_commit_accepted_kv_moves_only_the_path)


def test_tree_builder_ties_to_higher_parent_is_caught(monkeypatch):
    def wrong(lp, n_nodes, max_depth):  # same expansion, ties broken toward the higher parent id
        n_cand = lp.shape[1]
        parent, depth, rank, cum = [-1], [0], [0], [0.0]
        cands = [(float(lp[1][0]), 0, 0, 1)] if n_nodes > 1 and max_depth >= 1 else []
        while len(parent) < n_nodes:
            best = min(range(len(cands)), key=lambda j: (-cands[j][0], -cands[j][1], cands[j][2]))
            sc, p, r, d = cands.pop(best)
            i = len(parent)
            parent.append(p), depth.append(d), rank.append(r), cum.append(sc)
            if d < max_depth:
                cands.append((sc + float(lp[d + 1][0]), i, 0, d + 1))
            if r + 1 < n_cand:
                cands.append((cum[p] + float(lp[d][r + 1]), p, r + 1, d))
        return tuple(np.asarray(x, dtype=np.int32) for x in (parent, depth, rank))
    _patch(monkeypatch, "build_best_first_tree", wrong)
    assert _fails(pins.test_best_first_tree_golden_ties_and_generator)


def test_tree_builder_without_sibling_offers_is_caught(monkeypatch):
    def wrong(lp, n_nodes, max_depth):  # a taken candidate does not offer the next rank
        parent, depth, rank, cum = [-1], [0], [0], [0.0]
        cands = [(float(lp[1][0]), 0, 0, 1)] if n_nodes > 1 and max_depth >= 1 else []
        while len(parent) < n_nodes and cands:
            best = min(range(len(cands)), key=lambda j: (-cands[j][0], cands[j][1], cands[j][2]))
            sc, p, r, d = cands.pop(best)
            i = len(parent)
            parent.append(p), depth.append(d), rank.append(r), cum.append(sc)
            if d < max_depth:
                cands.append((sc + float(lp[d + 1][0]), i, 0, d + 1))
        while len(parent) < n_nodes:
            parent.append(0), depth.append(1), rank.append(0)
        return tuple(np.asarray(x, dtype=np.int32) for x in (parent, depth, rank))
    _patch(monkeypatch, "build_best_first_tree", wrong)
    assert any(_fails(pins.test_best_first_tree_brute_force, seed) for seed in range(10))


def test_bf16_misdecode_is_caught(monkeypatch):
    # a shift by 15 instead of 16 (an off-by-one in the bit layout), then a
    # decode that drops the sign bit
    for bad in (lambda u: (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(15))
                .view(np.float32).astype(np.float64),
                lambda u: ((np.asarray(u, dtype=np.uint16).astype(np.uint32) & np.uint32(0x7FFF)) << np.uint32(16))
                .view(np.float32).astype(np.float64)):
        _patch(monkeypatch, "bf16_bits_to_f64", bad)
        assert _fails(pins.test_bf16_decoder_format_values)
        case = dict(dtype="bf16", B=2, Hq=8, Hkv=2, D=128, P=[200, 333], N=7, tree="best_first", tree_depth=4)
        assert _fails(pins.test_verify_matches_torch_sdpa, case)


def test_unmutated_oracle_passes_the_same_checks():
    # the same check functions pass on the real oracle (guards against vacuous mutation tests)
    pins.test_bf16_decoder_format_values()
    pins.test_verify_matches_torch_sdpa(dict(dtype="bf16", B=2, Hq=8, Hkv=2, D=128, P=[200, 333], N=7,
                                             tree="best_first", tree_depth=4))
    pins.test_golden_attention_three_keys()
    pins.test_golden_tree_uniform()
    pins.test_golden_scores_small()
    pins.test_golden_topk_ties()
    pins.test_golden_sparse_two_keys()
    pins.test_compacted_draft_equals_sparse_list("bf16", "contiguous")
    pins.test_greedy_accept_golden()
    pins.test_best_first_tree_golden_ties_and_generator()
    pins.test_commit_accepted_kv_moves_only_the_path()
