"""GPU parity of greedy acceptance and the accepted branch's K/V move
(sv_accept_commit) against the CPU oracle: integer outputs and moved bytes
compared exactly, on chains and best-first trees of up to 256 nodes, contiguous
and paged caches, with the edge cases (a single node, nothing accepted, a fully
accepted chain)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import KVCache as OKV
from workloads import best_first_tree, depth_logprobs, make_accept_tokens, make_custom
from tests.gpu_util import DevWorkload, i32

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


def _trees(seed, B, N, depth):
    r = np.random.default_rng(seed)
    return np.stack([best_first_tree(N, depth_logprobs(r, depth), depth)[0] for _ in range(B)]).astype(np.int32)


def _bits(t: torch.Tensor) -> np.ndarray:
    x = t.detach().cpu()
    return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()


@pytest.mark.parametrize("B,N,depth,chain,p", [(1, 256, 8, False, 0.9), (16, 64, 6, False, 0.75),
                                                (3, 37, 5, False, 0.5), (4, 16, 0, True, 0.8),
                                                (2, 256, 0, True, 1.0), (5, 1, 0, True, 0.5)])
def test_accept_paths_exact(B, N, depth, chain, p):
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1)) if chain else _trees(50 + N, B, N, depth)
    draft, target = make_accept_tokens(60 + N + B, parent, match_prob=p)
    path, n_acc, bonus, newp = sv.accept_commit(i32(draft), i32(target), parent=None if chain else i32(parent),
                                                prefix_len=i32(np.arange(B) * 10), P_max=10 * B)
    path, n_acc, bonus, newp = (x.cpu().numpy() for x in (path, n_acc, bonus, newp))
    for b in range(B):
        ref = oracle.greedy_accept(None if chain else parent[b], draft[b], target[b])
        assert path[b, : len(ref)].tolist() == ref and (path[b, len(ref):] == -1).all(), f"sequence {b}"
        assert n_acc[b] == len(ref) - 1
        assert bonus[b] == target[b, ref[-1]]
        assert newp[b] == 10 * b + len(ref)
    if chain and p == 1.0:
        assert (n_acc == N - 1).all()


@pytest.mark.parametrize("dtype,layout", [("bf16", "contiguous"), ("f32", "paged"), ("bf16", "paged")])
def test_accept_commit_moves_kv(dtype, layout):
    """After the call the cache equals the oracle's: each depth's row holds the
    accepted node's row, every other row is unchanged."""
    B, N = 6, 64
    wl = make_custom(seed=70, B=B, Hq=8, Hkv=2, D=128, dtype=dtype, P=[300, 17, 0, 555, 128, 40], N=N,
                     tree="best_first", tree_depth=6, layout=layout, page_size=16)
    dw = DevWorkload(wl)
    draft, target = make_accept_tokens(71, wl.parent, match_prob=0.85)
    path, n_acc, _, newp = sv.accept_commit(i32(draft), i32(target), parent=dw.parent, kv=dw.kv, prefix_len=dw.P,
                                            P_max=wl.P_max)
    k_ref, v_ref = wl.k.copy(), wl.v.copy()
    okv = OKV(k_ref, v_ref, dtype, wl.layout, wl.seq_stride, wl.page_size, wl.page_table)
    moved = 0
    for b in range(B):
        ref = oracle.greedy_accept(wl.parent[b], draft[b], target[b])
        oracle.commit_accepted_kv(okv, b, int(wl.P[b]), ref)
        moved += sum(1 for d, v in enumerate(ref) if v != d)
        assert int(newp[b]) == int(wl.P[b]) + len(ref)
    assert moved > 0  # the case does exercise moves
    assert np.array_equal(_bits(dw.kv.k), k_ref) and np.array_equal(_bits(dw.kv.v), v_ref)


def test_accept_without_kv_leaves_cache_alone():
    wl = make_custom(seed=72, B=2, Hq=8, Hkv=2, D=64, dtype="bf16", P=[50, 60], N=32, tree="best_first", tree_depth=5)
    dw = DevWorkload(wl)
    draft, target = make_accept_tokens(73, wl.parent, match_prob=1.0)
    k0 = dw.kv.k.clone()
    path, n_acc, bonus, newp = sv.accept_commit(i32(draft), i32(target), parent=dw.parent)
    torch.cuda.synchronize()
    assert torch.equal(dw.kv.k, k0) and newp is None
    for b in range(2):
        assert path[b, : int(n_acc[b]) + 1].tolist() == oracle.greedy_accept(wl.parent[b], draft[b], target[b])
