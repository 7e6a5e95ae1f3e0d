"""Plain fp64 CPU oracle for draft-block verification.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the library never does, and the
oracle never imports the library.  It shares no code with the GPU path.
"""
from .verify import (  # noqa: F401
    Weights, bf16_rne, from_bf16_bits, from_e4m3_bits, silu, target_hidden, lm_logits, softmax_t, row_stats,
    inverse_cdf, accept_sample, accept_greedy, propose, survival_schedule,
    verify_greedy, verify_sample, verify_scheduled,
)
from .commit import commit  # noqa: F401
from .tree import (  # noqa: F401
    children as tree_children, next_residual, accept_tree_greedy, accept_tree_sample, verify_tree_greedy,
    verify_tree_sample,
)
from .theory import (  # noqa: F401
    expected_tokens, speedup, best_draft_length, tau_from_position_acceptance,
    conditional_acceptance, acceptance_rate, tau_closed_form, tokens_per_step,
)
