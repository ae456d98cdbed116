"""Seeded synthetic inputs for the MoE-layer forward, shared by the HIP path and the oracle.

This module only draws random numbers and casts them to storage dtypes; it holds none of
the layer's arithmetic. Both sides of every parity check receive the same tensors from here.

Workloads follow the pages' own model shapes (pages cited by title):
  [P2] "Twinkle首发适配Deepseek-V4系列模型高效训练" (www.wmrh.cn/news/44033)
  [P3] "DeepSpeed ZeRO-3与MoE显存精算实战指南" (m.nlpx.cn/news/237350)
  [P4] "手搓一个LLaMA4-MoE" (www.nxmr.cn/news/140631)

* main_bf16: P4 §2.1 model config (hidden 2048, intermediate 4096, 8 experts, 2 per token,
  aux coefficient 0.01, init std 0.02) at batch 8 x seq 2048.
* small_bf16: P4 §3.1 single-GPU bring-up size (4 experts, hidden 1024, sequence 512), batch 8.
* skewed_gumbel_capacity / small_t_streaming: P2's 16-expert top-2 model with router
  temperature 0.7 (P2 §3.1) and P3's capacity factor 1.2 (P3 §3.4).

Value distributions: x ~ N(0, 1); router weight ~ N(0, 1/d) (1/d read as a variance, so
logits have unit variance); expert weights ~ N(0, 0.02^2) (0.02 is P4's init std);
per-expert router bias ~ N(0, 1.5^2). bf16 tensors are fp32 draws rounded to nearest-even.
Gumbel noise is G = -log(-log U), U uniform on (0, 1) in fp64, stored as fp32 [T, E].
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                      # tokens (batch x sequence)
    d_model: int
    d_ffn: int
    num_experts: int
    top_k: int
    dtype: str                  # "f32" or "bf16": storage type of x, W1, W2, H, Y, out
    capacity_factor: Optional[Tuple[int, int]] = None   # (num, den) of a decimal factor; None = no limit
    temperature: float = 1.0
    gumbel: bool = False
    router_bias: bool = False
    aux_coef: float = 0.01
    renormalize: bool = True
    router_noise: float = 0.0   # std of additive router-logit noise (0: none); excludes gumbel
    padding: float = 0.0        # fraction of padding tokens (drawn per token; 0: no mask)
    d_ffn_shared: int = 0       # width of the shared expert (0: none)
    weight_dtype: Optional[str] = None   # "int4": the library gets 4-bit copies of W1/W2
    straight_through: bool = False       # gate weights 1, gradient through the full softmax
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.T


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=64, d_model=32, d_ffn=64, num_experts=4, top_k=2, dtype="f32"),
    "small_bf16": Workload("small_bf16", T=4096, d_model=1024, d_ffn=2048, num_experts=4, top_k=2,
                           dtype="bf16"),
    "main_bf16": Workload("main_bf16", T=16384, d_model=2048, d_ffn=4096, num_experts=8, top_k=2,
                          dtype="bf16"),
    "skewed_gumbel_capacity": Workload("skewed_gumbel_capacity", T=32768, d_model=2048, d_ffn=4096,
                                       num_experts=16, top_k=2, dtype="bf16", capacity_factor=(12, 10),
                                       temperature=0.7, gumbel=True, router_bias=True),
    "small_t_streaming": Workload("small_t_streaming", T=256, d_model=2048, d_ffn=4096, num_experts=16,
                                  top_k=2, dtype="bf16", capacity_factor=(12, 10)),
    # the main layer with P4's router variants: additive logit noise of scale 0.1 (P4 §3.2, its
    # value at the start of training) and 10% padding tokens (P4 §4.1)
    "main_noise_padding": Workload("main_noise_padding", T=16384, d_model=2048, d_ffn=4096, num_experts=8,
                                   top_k=2, dtype="bf16", router_noise=0.1, padding=0.1),
    # the weight-streaming layer with 4-bit expert weights (P4 §5.2)
    "small_t_int4": Workload("small_t_int4", T=256, d_model=2048, d_ffn=4096, num_experts=16, top_k=2,
                             dtype="bf16", capacity_factor=(12, 10), weight_dtype="int4"),
    # the main layer with one shared expert of the routed experts' width (P4 §5.2)
    "main_shared": Workload("main_shared", T=16384, d_model=2048, d_ffn=4096, num_experts=8, top_k=2,
                            dtype="bf16", d_ffn_shared=4096),
}

# The workload the headline throughput is quoted on.
MAIN = "main_bf16"


def derived(base: Workload, **changes) -> Workload:
    """A copy of `base` with some fields replaced (used for reduced-size parity cases)."""
    return dataclasses.replace(base, **changes)


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(w: Workload) -> dict:
    """Draw the inputs of workload `w` on the CPU, in a fixed order from one seeded generator.

    Order: x [T,d], router weight [E,d], W1 [E,f,d], W2 [E,d,f], then (if enabled) router
    bias [E], Gumbel noise [T,E], additive router noise [T,E] (standard normal times
    router_noise), and the padding mask [T] (token t is padding when a uniform draw is below
    `padding`), then the shared expert W1s [fs,d] and W2s [d,fs] (0.02 std, as the routed
    experts). Returns CPU tensors: x/w1/w2 in the storage dtype, w_router/bias and the noise in
    fp32, the mask in uint8 (1 = real token). The noise (Gumbel or additive: a workload has at
    most one) is returned under "gumbel", the library's single noise input; bias, noise and mask
    are None when disabled.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    T, d, f, E = w.T, w.d_model, w.d_ffn, w.num_experts
    x = torch.randn(T, d, generator=g, dtype=torch.float32)
    w_router = torch.randn(E, d, generator=g, dtype=torch.float32) * (1.0 / d ** 0.5)
    w1 = torch.randn(E, f, d, generator=g, dtype=torch.float32) * 0.02
    w2 = torch.randn(E, d, f, generator=g, dtype=torch.float32) * 0.02
    bias = None
    gumbel = None
    if w.router_bias:
        bias = torch.randn(E, generator=g, dtype=torch.float32) * 1.5
    if w.gumbel:
        u = torch.rand(T, E, generator=g, dtype=torch.float64)
        tiny = 2.0 ** -53
        u = u.clamp_(tiny, 1.0 - tiny)
        gumbel = (-torch.log(-torch.log(u))).to(torch.float32)
    if w.router_noise > 0.0:
        if w.gumbel:
            raise ValueError("a workload has either Gumbel or additive router noise")
        gumbel = torch.randn(T, E, generator=g, dtype=torch.float32) * w.router_noise
    token_mask = None
    if w.padding > 0.0:
        token_mask = (torch.rand(T, generator=g, dtype=torch.float64) >= w.padding).to(torch.uint8)
    w1s = w2s = None
    if w.d_ffn_shared > 0:
        w1s = torch.randn(w.d_ffn_shared, d, generator=g, dtype=torch.float32) * 0.02
        w2s = torch.randn(d, w.d_ffn_shared, generator=g, dtype=torch.float32) * 0.02
    st = _torch_dtype(w.dtype)
    return {
        "x": x.to(st).contiguous(),
        "w_router": w_router.contiguous(),
        "w1": w1.to(st).contiguous(),
        "w2": w2.to(st).contiguous(),
        "bias": bias,
        "gumbel": gumbel,
        "token_mask": token_mask,
        "w1_shared": None if w1s is None else w1s.to(st).contiguous(),
        "w2_shared": None if w2s is None else w2s.to(st).contiguous(),
    }


def inputs_digest(inp: dict) -> str:
    """SHA-256 over the raw bytes of all input tensors (logged so runs can be compared)."""
    h = hashlib.sha256()
    for key in ("x", "w_router", "w1", "w2", "bias", "gumbel", "token_mask", "w1_shared", "w2_shared"):
        t = inp.get(key)
        if t is None:
            h.update(b"none")
            continue
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
