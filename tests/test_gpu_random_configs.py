"""GPU parity on seeded random configurations: batch, heads, head dim, node
count, chain or best-first tree, cache layout and page size, prefix lengths,
scoring rows and k drawn from one fixed generator, each case checked against
the oracle like the named cases (outputs, scores, the selection band and the
draft steps)."""
import numpy as np
import pytest
import torch

from tests.test_gpu_parity import check_workload
from workloads import make_custom

pytestmark = pytest.mark.gpu

import tree_verify_sparse_amd as sv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sv.lib()  # the HIP library must be there: no fallback


def _config(i):
    r = np.random.default_rng([20261202, i])
    dtype = "f32" if r.random() < 0.2 else "bf16"
    D = int(r.choice([64, 128]))
    Hq, Hkv = [(8, 2), (16, 4), (32, 8), (4, 4), (12, 4), (8, 1)][int(r.integers(6))]
    N = int(r.choice([1, 3, 8, 17, 40, 64, 100]))
    B = int(r.integers(1, 4))
    P = [int(x) for x in r.integers(0, 3000, size=B)]
    if r.random() < 0.3:
        P[int(r.integers(B))] = int(r.integers(0, 40))  # a short or empty prefix
    tree = "best_first" if (N > 2 and r.random() < 0.6) else None
    paged = r.random() < 0.4
    page_size = int(r.choice([1, 8, 16, 24])) if paged else 16
    kind = r.random()
    if kind < 0.4:
        rows = "all"
    elif kind < 0.7:
        rows = "c2q"
    elif kind < 0.9:
        rows = sorted(int(x) for x in r.choice(N, size=min(N, int(r.integers(1, 6))), replace=False))
    else:
        rows = []
    k_sel = "5pct" if r.random() < 0.3 else int(r.integers(1, 300))
    return dict(seed=3000 + i, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, P=P, N=N, tree=tree,
                tree_depth=int(r.integers(2, 9)), score_rows=rows, k_sel=k_sel,
                layout="paged" if paged else "contiguous", page_size=page_size,
                q_std_mult=float(r.choice([1.0, 3.0])), decode_steps=1 if rows != [] else 0)


CONFIGS = [_config(i) for i in range(24)]


@pytest.mark.parametrize("i", range(len(CONFIGS)))
def test_random_config_parity(i):
    cfg = CONFIGS[i]
    print(f"[random config {i}] {cfg}", flush=True)
    check_workload(make_custom(**cfg))
