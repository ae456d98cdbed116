"""moe_forward_noalloc (the entry point for callers that cannot allocate) against moe_forward on
the GPU: bitwise equal out and aux on two calls in a row, the second with a smaller input, so
that the static workspace holds the first call's values when the second one runs."""
import pytest
import torch

import sparse_mixture_experts_02_amd as moe
from sparse_mixture_experts_02_amd.inputs import WORKLOADS, derived, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # the weight-streaming layer at full size (capacity drops), then a smaller one with Gumbel keys,
    # a router bias and capacity
    (WORKLOADS["small_t_streaming"],
     derived(WORKLOADS["skewed_gumbel_capacity"], name="noalloc_small", T=100, d_model=512, d_ffn=1024,
             num_experts=8)),
    # the 128 x 128 grouped GEMM with a shared expert and padding, then fp32 with additive noise
    (derived(WORKLOADS["main_bf16"], name="noalloc_mid", T=200, d_model=256, d_ffn=512, num_experts=4,
             d_ffn_shared=256, padding=0.2),
     derived(WORKLOADS["tiny_f32"], name="noalloc_f32", T=50, router_noise=0.3, capacity_factor=(9, 10))),
]


def _run(w, noalloc: bool):
    inp = make_inputs(w)
    cfg = moe.config_for(w)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    out = torch.full((w.T, w.d_model), float("nan"), dtype=cfg.torch_dtype, device="cuda")
    aux = torch.full((3,), float("nan"), dtype=torch.float32, device="cuda")
    kw = dict(bias=dev["bias"], gumbel=dev["gumbel"], token_mask=dev["token_mask"], w1_shared=dev["w1_shared"],
              w2_shared=dev["w2_shared"])
    if noalloc:
        moe.moe_forward_noalloc(cfg, dev["x"], dev["w_router"], dev["w1"], dev["w2"], out, aux, **kw)
    else:
        moe.moe_forward(cfg, dev["x"], dev["w_router"], dev["w1"], dev["w2"], out, aux, moe.new_workspace(cfg), **kw)
    torch.cuda.synchronize()
    return out.cpu(), aux.cpu()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forward_noalloc_matches_forward(case):
    for w in CASES[case]:       # the second call has a smaller input than the first
        print(f"[gpu] moe_forward_noalloc vs moe_forward: {w}", flush=True)
        ref_out, ref_aux = _run(w, noalloc=False)
        out, aux = _run(w, noalloc=True)
        assert torch.equal(out.view(torch.uint8), ref_out.view(torch.uint8)), w.name
        assert torch.equal(aux.view(torch.uint8), ref_aux.view(torch.uint8)), w.name
        assert not torch.isnan(out.float()).any()
