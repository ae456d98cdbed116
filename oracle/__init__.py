"""CPU oracle of the MoE-layer forward (test infrastructure; never used by the product path)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (Dispatch, Forward, Routing, aux_loss, capacity_from_factor, combine,  # noqa: F401
                         dispatch, expert_ffn, forward, forward_rows, gate_weights, round_bf16,
                         round_storage, route, router_logits, router_probs, selection_keys, silu,
                         top_k, topk_gap)
