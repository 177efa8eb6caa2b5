"""fp64 CPU oracle of the pooled-wave capacity-dispatch MoE forward and of
the backward of its routed path, and of the router's next-step bias update
(`oracle.router_bias`).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Every function is
pinned by CPU tests against closed forms, brute force, special cases that
reduce to textbook or library routines, and the constants the pages print.
"""
from .moe_oracle import (  # noqa: F401
    assign_slots, bank_expert_rows, capacity_plan, combine, drop_fractions,
    expert_out_pool_layout, expert_outputs, forward, forward_dropless, gates,
    latent, pool_of, ragged_order, route_topk, router_logits, selection_scores,
    shared_experts, silu, swiglu, up_project, wave_ranges,
)
from .moe_backward import (  # noqa: F401
    combine_backward, dispatch_backward, experts_backward, gates_backward,
    routed_backward, scatter_logit_grad, swiglu_backward,
)
