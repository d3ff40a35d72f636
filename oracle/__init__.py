"""CPU oracle (test infrastructure only; see ``moe_oracle``)."""
from .moe_oracle import (  # noqa: F401
    GATE_MODES,
    capacity,
    gates,
    load_balance,
    moe_forward,
    near_tie,
    route_maps,
    router_probs,
    router_logits,
    selection_keys,
    silu,
    swiglu_ffn,
    topk,
)
