"""Convenience wrappers: a workload's MoEConfig, and a forward call that allocates its outputs."""
from __future__ import annotations

from typing import Optional

import torch

from . import binding
from .binding import MoEConfig
from .inputs import Workload


def config_for(w: Workload, T: Optional[int] = None) -> MoEConfig:
    """The MoEConfig of a workload; the capacity factor is turned into an absolute capacity by
    the library's moe_capacity_from_factor."""
    T = w.T if T is None else T
    cap = binding.MOE_NO_CAPACITY
    if w.capacity_factor is not None:
        cap = binding.capacity_from_factor(T, w.top_k, w.num_experts, *w.capacity_factor)
    return MoEConfig(T=T, d_model=w.d_model, d_ffn=w.d_ffn, num_experts=w.num_experts, top_k=w.top_k,
                     capacity=cap, temperature=w.temperature, renormalize=w.renormalize,
                     aux_coef=w.aux_coef, dtype=w.dtype, noise_in_logits=w.router_noise > 0.0,
                     d_ffn_shared=w.d_ffn_shared, weight_dtype=w.weight_dtype,
                     straight_through=w.straight_through)


def forward(cfg: MoEConfig, x, w_router, w1, w2, *, bias=None, gumbel=None, token_mask=None, w1_shared=None,
            w2_shared=None, ws=None, debug=None):
    """Run moe_forward on the current stream; returns (out [T, d], aux [3]) GPU tensors."""
    if ws is None:
        ws = binding.new_workspace(cfg, x.device)
    out = torch.empty(cfg.T, cfg.d_model, dtype=cfg.torch_dtype, device=x.device)
    aux = torch.empty(3, dtype=torch.float32, device=x.device)
    binding.moe_forward(cfg, x, w_router, w1, w2, out, aux, ws, bias=bias, gumbel=gumbel, token_mask=token_mask,
                        w1_shared=w1_shared, w2_shared=w2_shared, debug=debug)
    return out, aux
