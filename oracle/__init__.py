"""CPU oracle for SpecOPD branch-parallel target scoring — TEST INFRASTRUCTURE.

This package is the slow, plain, fp64 statement of what the GPU library must
compute.  It exists to check the library, never to stand in for it: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it.  It shares no code with the HIP path (no kernels, headers, helpers or
tables) and imports nothing from it.

Sources cited (the web pages describing arXiv 2611.02846, "SpecOPD:
Branch-Parallel On-Policy Distillation for Speculative Decoding"):
  [R] the jaehun.me review of the paper (its sections mirror the paper's)
  [A] the readsearch.ai listing with the authors' abstract
  [N] the richland.au news post on SpecOPD
  [S] the rustineverything.app summary (Chinese), which cites paper sections

Readings taken where the pages are silent are stated in each function.

Pinning: every function here is checked by tests against facts fixed
independently of its own code (worked examples printed on the pages, closed
forms, library routines, brute force, Monte Carlo).  No function is "parity
unpinned".
"""

from .rope import rope, rope_angles
from .tree_attention import (walk_ancestors, tree_depths, check_positions,
                             branch_mask, packed_tree_mask, tree_attention_branch,
                             tree_attention, tree_attention_packed)
from .e2etv import (logsumexp, log_softmax, overlap, prefix_products, suffix_sums,
                    e2etv, e2etv_branch)
from .rows import score_row_source, new_score_rows, shared_row_count
from .prefill import trunk_prefill, trunk_prefill_cache
from .gdn import (gated_delta_update, gdn_read, run_tokens, trunk_checkpoints, replay_span,
                  anchor_state, gdn_branch, gdn_replay, update_counts, conv_history, branch_conv,
                  gdn_branch_conv)
from .qsa import (rms_norm, compress_group, sequence_group_keys, select_topk, plain_row_select,
                  branch_group_keys, qsa_branch_select, qsa_select, causal_tail, round_bf16)
from .lmhead import lmhead_logits, lmhead_e2etv

__all__ = [
    "rope", "rope_angles", "walk_ancestors", "tree_depths", "check_positions",
    "branch_mask", "packed_tree_mask", "tree_attention_branch", "tree_attention",
    "tree_attention_packed", "logsumexp", "log_softmax", "overlap", "prefix_products",
    "suffix_sums", "e2etv", "e2etv_branch", "score_row_source", "new_score_rows",
    "shared_row_count", "trunk_prefill", "trunk_prefill_cache", "gated_delta_update",
    "gdn_read", "run_tokens", "trunk_checkpoints", "replay_span", "anchor_state", "gdn_branch",
    "gdn_replay", "update_counts", "conv_history", "branch_conv", "gdn_branch_conv",
    "rms_norm", "compress_group", "sequence_group_keys", "select_topk", "plain_row_select",
    "branch_group_keys", "qsa_branch_select", "qsa_select", "causal_tail", "round_bf16",
    "lmhead_logits", "lmhead_e2etv",
]
