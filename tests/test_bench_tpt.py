"""bench.py's tokens-per-time projection (KnapSpec §2, the TPT metric) against
the oracle's definition, on a grid that includes alpha = 0 and alpha = 1."""
import pytest

import bench
import oracle


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.6, 0.8, 0.9, 0.99, 1.0])
@pytest.mark.parametrize("gamma", [0, 1, 7, 15])
def test_bench_tpt_matches_oracle(alpha, gamma):
    for t_draft, t_target in ((3.0, 60.0), (12.5, 430.0)):
        assert bench.tpt(alpha, gamma, t_draft, t_target) == pytest.approx(
            oracle.tpt(alpha, gamma, t_draft, t_target), rel=1e-12)
