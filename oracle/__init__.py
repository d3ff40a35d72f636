"""CPU oracle (test infrastructure only; see ``moe_oracle``)."""
from .moe_oracle import (  # noqa: F401
    GATE_MODES,
    capacity,
    expert_choice,
    expert_choice_forward,
    gates,
    load_balance,
    moe_forward,
    near_tie,
    route_maps,
    route_maps_score_drop,
    router_probs,
    router_logits,
    selection_keys,
    silu,
    swiglu_ffn,
    topk,
)
