"""CPU oracle for the Medusa verify tree-step (test infrastructure only).

Only the test-suite, the smoke check and the bench's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .medusa import (  # noqa: F401
    TreeError, bf16_round, medusa_heads, verification_logits, medusa_topk, dense_paths,
    greedy_paths, validate_paths, build_tree, ancestors, tree_positions,
    tree_tokens, tree_attention, row_distribution, typical_accept,
    rs_accept_prob, rs_residual, sample_inverse_cdf, rejection_accept,
    topk_per_head, kv_commit, step,
)
