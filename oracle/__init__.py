"""CPU oracle for the verification-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers or pre/post-processing); both sides only
consume the same seeded inputs from ``workloads``.

It is a plain, slow, obviously-correct numpy implementation in float64 of what
the path computes, each function citing the passage it follows.  Sources cited
(titles of the technical-summary pages, gist.science/pt/paper/...):

* "Vegas" (2602.07223) -- Resumo Técnico: Vegas, Decodificação Auto-Especulativa
  com Atenção Esparsa Guiada por Verificação.
* "JETFLOW" (2606.18394) -- Resumo Técnico: JETFLOW.
* "KnapSpec" (2602.20217) -- Resumo Técnico: KnapSpec (§2, the tokens-per-time metric).

Every function here is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force, library routines and invariants; see ``oracle/reference.py``'s
header for which pin covers which function.
"""
from .reference import (  # noqa: F401
    KVCache,
    ancestors,
    visible_positions,
    verify_attention,
    verify_scores,
    verify_scores_grouped,
    topk_select,
    sparse_draft_attention,
    verify_scores_per_head,
    sparse_draft_attention_per_head,
    sink_window_select,
    compact_kv,
    dense_draft_attention,
    build_best_first_tree,
    greedy_accept,
    commit_accepted_kv,
    run_step,
    bf16_bits_to_f64,
    tpt,
)
