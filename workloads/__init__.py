"""Seeded synthetic inputs for the verification-attention hot path.

This module only draws random numbers and lays them out in memory.  It holds
none of the method's arithmetic (no attention, no logit sums, no selection):
both the CPU oracle and the HIP path consume what it produces, and neither
imports the other.

Workloads (shapes follow the five configurations the hot path is measured on):

  1  tiny fp32 chain        B=1, Hq/Hkv=4/1, D=64,  P=512,   chain gamma=4, all rows, k=64
  2  32k chain (C2Q)        B=1, Hq/Hkv=32/8, D=128, P=32768, chain gamma=7, rows {0,7}, k=2048
  3  tree verify            B=1, 32/8, D=128, P=8192, 256-node best-first tree, all rows, k=1024
  4  long context           B=4, 32/8, D=128, P=131072, chain gamma=15, rows {0,15}, k=4096, 15 decodes
  5  mixed paged batch      B=16, 32/8, D=128, P~U[4096,65536], 16-token shuffled pages,
                            64-node trees (depth<=6), all rows, k=floor(0.05 P)

Every tensor comes from its own generator stream ``np.random.default_rng([seed, stream])``
so that the same (config, seed) always yields bit-identical inputs.
"""
from .gen import (  # noqa: F401
    Workload,
    make_workload,
    make_custom,
    make_score_vector,
    make_tail_rows,
    make_accept_tokens,
    CONFIG_NAMES,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
)
from .tree import best_first_tree, chain_parents, depth_logprobs  # noqa: F401
