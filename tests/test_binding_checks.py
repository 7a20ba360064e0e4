"""The Python binding checks that the tensors of a call agree with each other
before it takes any pointer or launches anything.  CPU tensors are used on
purpose: a call that got past the checks would stop at the first pointer with
"must live on the GPU", so each test's specific message shows that the
mismatch was caught first."""
import pytest
import torch

import tree_verify_sparse_amd as sv

B, N, Hq, Hkv, D, P = 2, 4, 8, 2, 64, 100
bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def kv(dtype=bf, D_=D, Hkv_=Hkv, pt=None):
    k = torch.zeros((B * (P + N), Hkv_, D_), dtype=dtype)
    return sv.KVCache(k, k.clone(), seq_stride=P + N, page_table=pt, page_size=16)


def q4(dtype=bf, D_=D, Hq_=Hq):
    return torch.zeros((B, N, Hq_, D_), dtype=dtype)


def pl(n=B, dtype=i32):
    return torch.full((n,), P, dtype=dtype)


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_gpu_pointer_guard_is_what_a_consistent_call_reaches():
    with pytest.raises(ValueError, match="must live on the GPU"):
        sv.verify_attn(q4(), kv(), pl(), P_max=P, score_rows=[0])


@pytest.mark.parametrize("case", [
    ("dtype", lambda: sv.verify_attn(q4(f32), kv(bf), pl(), P_max=P), "differs from the KV cache"),
    ("head dim", lambda: sv.verify_attn(q4(D_=128), kv(), pl(), P_max=P), "head dim 128 differs"),
    ("heads", lambda: sv.verify_attn(q4(Hq_=6), kv(Hkv_=4), pl(), P_max=P), "not a multiple"),
    ("k/v dtype", lambda: sv.verify_attn(q4(), sv.KVCache(torch.zeros((10, Hkv, D), dtype=bf),
                                                          torch.zeros((10, Hkv, D), dtype=f32)), pl(), P_max=P),
     "share a dtype"),
    ("prefix_len dtype", lambda: sv.verify_attn(q4(), kv(), pl(dtype=torch.int64), P_max=P), "prefix_len must be int32"),
    ("prefix_len shape", lambda: sv.verify_attn(q4(), kv(), pl(n=3), P_max=P), "prefix_len must have shape"),
    ("parent shape", lambda: sv.verify_attn(q4(), kv(), pl(), P_max=P, parent=torch.zeros((B, N + 1), dtype=i32)),
     "parent must have shape"),
    ("out shape", lambda: sv.verify_attn(q4(), kv(), pl(), P_max=P, out=torch.zeros((B, N, Hq, D - 1), dtype=bf)),
     "out must have shape"),
    ("out dtype", lambda: sv.verify_attn(q4(), kv(), pl(), P_max=P, out=torch.zeros((B, N, Hq, D), dtype=f32)),
     "out must be"),
    ("scores narrow", lambda: sv.verify_attn(q4(), kv(), pl(), P_max=P, score_rows=[0],
                                             scores=torch.zeros((B, P - 1), dtype=f32)), "scores must have shape"),
    ("page table", lambda: sv.verify_attn(q4(), kv(pt=torch.zeros((B, 8), dtype=torch.int64)), pl(), P_max=P),
     "page_table must be int32"),
])
def test_verify_mismatches(case):
    _, fn, match = case
    raises(match, fn)


def test_per_head_and_noalloc_mismatches():
    raises("head_scores must have shape", sv.verify_attn_per_head, q4(), kv(), pl(), P_max=P, score_rows=[0],
           head_scores=torch.zeros((B, Hkv, P - 1), dtype=f32))
    raises("differs from the KV cache", sv.verify_attn_per_head, q4(f32), kv(), pl(), P_max=P)
    raises("head dim", sv.verify_attn_noalloc, q4(D_=128), kv(), pl(), P_max=P)


def test_topk_mismatches():
    s = torch.zeros((B, P), dtype=f32)
    k = torch.full((B,), 5, dtype=i32)
    raises("scores must be float32", sv.topk_select, s.double(), pl(), k, 8)
    raises("prefix_len must have shape", sv.topk_select, s, pl(n=1), k, 8)
    raises("k must be int32", sv.topk_select, s, pl(), k.long(), 8)
    raises("idx must have shape", sv.topk_select, s, pl(), k, 8, idx=torch.zeros((B, 7), dtype=i32))
    raises("count must have shape", sv.topk_select, s, pl(), k, 8, count=torch.zeros((B + 1,), dtype=i32))


def test_sparse_mismatches():
    q = torch.zeros((B, Hq, D), dtype=bf)
    idx = torch.zeros((B, 16), dtype=i32)
    n = torch.full((B,), 16, dtype=i32)
    raises("differs from the KV cache", sv.sparse_draft_attn, q.float(), kv(), idx, n)
    raises("head dim", sv.sparse_draft_attn, torch.zeros((B, Hq, 128), dtype=bf), kv(), idx, n)
    raises("idx must be int32", sv.sparse_draft_attn, q, kv(), idx.long(), n)
    raises("n_idx must have shape", sv.sparse_draft_attn, q, kv(), idx, torch.full((B - 1,), 3, dtype=i32))
    raises("max_idx", sv.sparse_draft_attn, q, kv(), idx, n, max_idx=17)
    raises("out must have shape", sv.sparse_draft_attn, q, kv(), idx, n, out=torch.zeros((B, Hq, D + 1), dtype=bf))
    hidx = torch.zeros((B, Hkv, 16), dtype=i32)
    raises("n_idx must have shape", sv.sparse_draft_attn_per_head, q, kv(), hidx, n)
    raises("idx must be int32 \\[B\\]\\[Hkv\\]", sv.sparse_draft_attn_per_head, q, kv(), idx, n)


def test_compact_and_dense_mismatches():
    idx = torch.zeros((B, 16), dtype=i32)
    n = torch.full((B,), 16, dtype=i32)
    ck = torch.zeros((B, 16, Hkv, D), dtype=f32)
    raises("ck must be", sv.compact_kv, kv(), idx, n, 16, ck=ck, cv=ck)
    raises("ck must have shape", sv.compact_kv, kv(), idx, n, 16, ck=torch.zeros((B, 15, Hkv, D), dtype=bf),
           cv=torch.zeros((B, 16, Hkv, D), dtype=bf))
    q = torch.zeros((B, Hq, D), dtype=bf)
    raises("must have q's dtype", sv.dense_draft_attn, q, ck, ck, n)
    ckb = ck.to(bf)
    raises("n_rows must have shape", sv.dense_draft_attn, q, ckb, ckb, torch.zeros((B + 1,), dtype=i32))


def test_accept_mismatches():
    d = torch.zeros((B, N), dtype=i32)
    raises("target_tokens must have shape", sv.accept_commit, d, torch.zeros((B, N + 1), dtype=i32))
    raises("parent must be int32", sv.accept_commit, d, d.clone(), parent=d.long())
    raises("prefix_len must have shape", sv.accept_commit, d, d.clone(), prefix_len=pl(n=3))
