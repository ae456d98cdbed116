"""MI355X (gfx950) forward pass of a top-k routed MoE FFN layer: HIP kernels behind a C ABI.

The compute path is libmoe.so (csrc/, built by `python -m sparse_mixture_experts_02_amd.build`);
`binding` marshals torch GPU tensors into its calls. PyTorch supplies device memory and the
stream only.
"""
from .binding import (FORWARD_KERNEL_NAMES, backward_workspace_bytes, moe_backward, moe_combine_backward,  # noqa: F401
                      moe_dispatch_backward, moe_expert_ffn_backward, moe_route_backward, new_backward_workspace, MOE_NO_CAPACITY, HipEvents, MoEConfig, MoEError,  # noqa: F401
                      capacity_from_factor, int4_bytes, moe_aux_loss, moe_combine, moe_dispatch, moe_expert_ffn,
                      moe_forward, moe_forward_noalloc, forward_noalloc_max_bytes, moe_route, new_workspace, quantize_int4, status_string, validate_config,
                      workspace_bytes)
from .layer import config_for, forward  # noqa: F401
