"""CPU oracle for one Medusa draft-and-verify step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the step computes, in numpy float64, used to check the HIP
library.  Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never imports, calls or falls back to it, and
it shares no code, tables or helpers with that path.

Sources (web pages on Medusa heads; cited by page title and section):
  * aicassindra.com, "Medusa deep dive" (tm_medusa_deep): head formula
    (section "The heads are residual blocks, not linear layers"), sparse tree
    ("From top-k heads to a sparse candidate tree"), typical acceptance
    ("Typical acceptance, not exact rejection sampling").
  * inferensys.com, "Medusa Heads" glossary: verification pass, early stop and
    rollback, speculative KV cache, tree attention over a shared prefix.
  * aiunderstanding.org, "Medusa Decoding Heads" ("Deep Dive"): accept the
    longest prefix matching what the model would have produced.
  * zackli.ai, "Speculative Decoding Deep Dive II: Medusa, MTP" (section
    "Medusa"): Anc(i), full-path and tree-node counts; head indexing.
  * aicassindra.com "Medusa deep dive", "What it costs on a CPU-bound SLM":
    expected acceptance length as the throughput multiplier, the tree size as
    a tuned budget (module ``budget``).
  * zackli.ai, "Speculative Decoding Deep Dive II" ("Medusa"): Hydra-style
    heads that see the token just drafted (module ``hydra``); ("MTP"):
    heads that are transformer layers sharing one unembedding (module
    ``mtp``).

Every function states the passage it follows and, where the pages leave a step
open, the reading taken.  Pins: ``tests/test_oracle_*.py``.
"""

from .bf16 import round_bf16
from .heads import heads, lm_project
from .topk import topk_stable, argmax_lowest
from .rng import splitmix64, counter_uniform, sample_tempered
from .tree import tree_plan, tree_gather, full_tree_node_count, full_path_count, TreePlan
from .attention import tree_attention, path_attention
from .accept import (accept_greedy_walk, accept_greedy_parallel, accept_typical, typical_local,
                     accept_reject)
from .compact import kv_compact
from .step import oracle_step
from .budget import tree_plan_rates, expected_tokens, plan_from_tables, accept_tally
from .hydra import hydra_draft
from .mtp import mtp_draft, mtp_head, rmsnorm

__all__ = [
    "round_bf16", "heads", "lm_project", "topk_stable", "argmax_lowest",
    "splitmix64", "counter_uniform", "sample_tempered", "tree_plan", "tree_gather",
    "full_tree_node_count", "full_path_count", "TreePlan", "tree_attention",
    "path_attention", "accept_greedy_walk", "accept_greedy_parallel",
    "accept_typical", "typical_local", "accept_reject", "kv_compact", "oracle_step",
    "tree_plan_rates", "expected_tokens", "plan_from_tables", "accept_tally", "hydra_draft",
    "mtp_draft", "mtp_head", "rmsnorm",
]
