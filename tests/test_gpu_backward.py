"""GPU parity of the backward-pass calls against the CPU oracle, step by step (needs an MI355X).

Each step gets the GPU's own inputs (the forward's intermediates, the previous step's output),
as the forward parity does: moe_combine_backward against the combine's backward,
moe_expert_ffn_backward against the expert FFNs' backward, moe_dispatch_backward against the
gather's backward. Tolerances as the forward's (normwise 2e-2 bf16, 1e-5 fp32); the gate-weight
gradients (fp32 dot products) normwise 1e-5. moe_route_backward against the oracle's router
backward on the GPU's logits, ids, weights and counts with seeded gate-weight gradients: the
logit, router-weight and bias gradients normwise 1e-5 (fp32 against float64), dx as stored.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_02_amd as moe
from sparse_mixture_experts_02_amd.inputs import WORKLOADS, derived, make_inputs

from parity import NORM_TOL, normwise, run_gpu, to_device

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["main_bf16"]

CASES = {
    "bwd_f32": derived(WORKLOADS["tiny_f32"], name="bwd_f32", T=200, d_model=48, d_ffn=40, num_experts=5, top_k=3),
    # fp32 weight gradients over several 128 x 128 tiles (ragged in both M and N) and many
    # 16-row stages with a ragged last one
    "bwd_f32_tiles": derived(WORKLOADS["tiny_f32"], name="bwd_f32_tiles", T=900, d_model=136, d_ffn=264,
                             num_experts=3, top_k=2),
    "bwd_bf16_ragged": derived(BASE, name="bwd_bf16_ragged", T=600, d_model=256, d_ffn=384, num_experts=6),
    "bwd_capacity_padding": derived(WORKLOADS["skewed_gumbel_capacity"], name="bwd_capacity_padding", T=500,
                                    d_model=128, d_ffn=192, num_experts=8, padding=0.2, capacity_factor=(9, 10)),
    # 256 x 256 grouped GEMMs for the backward products (K = 256 and 512)
    "bwd_big": derived(BASE, name="bwd_big", T=2048, d_model=256, d_ffn=512, num_experts=2),
    # d a multiple of 512 with top-2: the combine backward that loads a token's rows up front
    "bwd_k2_prefetch": derived(BASE, name="bwd_k2_prefetch", T=700, d_model=1024, d_ffn=256, num_experts=4),
    # weight-streaming GEMMs (at most 64 rows per expert)
    "bwd_stream": derived(WORKLOADS["small_t_streaming"], name="bwd_stream", T=96, d_model=256, d_ffn=512),
    # half-width narrow slices of the emptiest last m-tiles on the recompute and dH GEMMs
    "bwd_half_slices": derived(BASE, name="bwd_half_slices", T=4104, d_model=256, d_ffn=4096),
    # one round of 32 tiles with 16 stages per tile for the dH GEMM (K = d = 1024)
    "bwd_split_single": derived(BASE, name="bwd_split_single", T=2048, d_model=1024, d_ffn=512, num_experts=2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_steps(name):
    w = CASES[name]
    print(f"[gpu] backward steps {name}: {w}", flush=True)
    cfg = moe.config_for(w)
    inp = make_inputs(w)
    dinp = to_device(inp)
    g = run_gpu(cfg, dinp)
    T, d, E, k = cfg.T, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, st = cfg.torch_dtype, cfg.dtype
    tol = NORM_TOL[st]
    gen = torch.Generator().manual_seed(77)
    d_out = torch.randn(T, d, generator=gen).to(dt)
    dev = "cuda"
    y, row_of, wts = g["y"].to(dev), g["row_of"].to(dev), g["weights"].to(dev)
    xp, off, h = g["xp"].to(dev), g["offsets"].to(dev), g["h"]
    N = int(g["offsets"][-1])
    dy = torch.zeros(T * k, d, dtype=dt, device=dev)
    dwt = torch.empty(T, k, dtype=torch.float32, device=dev)
    moe.moe_combine_backward(cfg, d_out.to(dev), y, row_of, wts, dy, dwt)
    ws = moe.new_backward_workspace(cfg)
    dxp = torch.zeros(T * k, d, dtype=dt, device=dev)
    f = cfg.d_ffn
    dw1 = torch.full((E, f, d), float("nan"), dtype=torch.float32, device=dev)
    dw2 = torch.full((E, d, f), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_expert_ffn_backward(cfg, xp, off, dinp["w1"], dinp["w2"], dy, dxp, ws, h=h.to(dev), dw1=dw1, dw2=dw2)
    dx = torch.empty(T, d, dtype=dt, device=dev)
    moe.moe_dispatch_backward(cfg, dxp, row_of, dx)
    torch.cuda.synchronize()
    # combine backward
    dy_ref, dw_ref = oracle.combine_backward(d_out, g["y"], g["row_of"].numpy(), g["weights"].numpy(), st)
    gdy = dy.cpu().float().numpy()[:N]
    assert normwise(gdy, dy_ref[:N]) <= tol, f"dY normwise error {normwise(gdy, dy_ref[:N])}"
    dw_err = normwise(dwt.cpu().numpy(), dw_ref)
    assert dw_err <= 1e-5, f"gate-weight gradient normwise error {dw_err}"
    # expert FFN backward on the GPU's dY
    dxp_ref, dw1_ref, dw2_ref = oracle.expert_ffn_backward(g["xp"][:N], g["offsets"].numpy(), inp["w1"],
                                                           inp["w2"], h[:N], dy.cpu()[:N], st)
    dxp_err = normwise(dxp.cpu().float().numpy()[:N], dxp_ref)
    assert dxp_err <= tol, f"dXp normwise error {dxp_err}"
    # weight gradients: dW2 from the GPU's dY and H exactly as the oracle has them; dW1 from the
    # GPU's dA (bf16-rounded there), so its tolerance is the storage one
    dw2_err = normwise(dw2.cpu().numpy(), dw2_ref)
    dw1_err = normwise(dw1.cpu().numpy(), dw1_ref)
    assert dw2_err <= (1e-5 if st == "f32" else 1e-5), f"dW2 normwise error {dw2_err}"
    assert dw1_err <= tol, f"dW1 normwise error {dw1_err}"
    # gather backward on the GPU's dXp
    dx_ref = oracle.dispatch_backward(dxp.cpu()[:max(N, 1)], g["row_of"].numpy(), T, st)
    dx_err = normwise(dx.cpu().float().numpy(), dx_ref)
    assert dx_err <= tol, f"dx normwise error {dx_err}"
    print(f"[gpu] {name}: dY {normwise(gdy, dy_ref[:N]):.2e} dw {dw_err:.2e} dXp {dxp_err:.2e} dx {dx_err:.2e} "
          f"dW2 {dw2_err:.2e} dW1 {dw1_err:.2e}", flush=True)


ROUTER_CASES = {
    # renormalised weights, aux term, bf16 x (dW_r with 16 experts per thread)
    "rbwd_bf16": (derived(BASE, name="rbwd_bf16", T=700, d_model=264, num_experts=8), 0.7),
    # full-softmax weights, fp32, 5 experts, ragged tokens and columns
    "rbwd_f32_full_softmax": (derived(WORKLOADS["tiny_f32"], name="rbwd_f32_full_softmax", T=333, d_model=40,
                                      num_experts=5, top_k=3, renormalize=False, temperature=0.7), 1.3),
    # padding, Gumbel selection, capacity, 32 experts
    "rbwd_padding_gumbel": (derived(WORKLOADS["skewed_gumbel_capacity"], name="rbwd_padding_gumbel", T=900,
                                    d_model=512, d_ffn=64, num_experts=24, padding=0.25), 1.0),
    # additive noise in the logits, 64 experts, no aux gradient
    "rbwd_noise_e64": (derived(WORKLOADS["main_noise_padding"], name="rbwd_noise_e64", T=520, d_model=128,
                               d_ffn=64, num_experts=64, top_k=4), 0.0),
    # the straight-through estimator with Gumbel selection and capacity (P2 §3.1)
    "rbwd_straight_through": (derived(WORKLOADS["skewed_gumbel_capacity"], name="rbwd_straight_through", T=800,
                                      d_model=256, d_ffn=64, straight_through=True), 1.0),
    # the layer's full size (16384 tokens, d 2048, 8 experts)
    "rbwd_main": (BASE, 1.0),
}


@pytest.mark.parametrize("name", list(ROUTER_CASES))
def test_router_backward(name):
    w, d_aux = ROUTER_CASES[name]
    print(f"[gpu] router backward {name}: {w} d_aux={d_aux}", flush=True)
    cfg = moe.config_for(w)
    inp = make_inputs(w)
    dinp = to_device(inp)
    g = run_gpu(cfg, dinp)
    T, d, E, k = cfg.T, cfg.d_model, cfg.num_experts, cfg.top_k
    dt = cfg.torch_dtype
    gen = torch.Generator().manual_seed(91)
    dwts = torch.randn(T, k, generator=gen)
    dx0 = torch.randn(T, d, generator=gen).to(dt)
    dev = "cuda"
    mask = inp.get("token_mask")
    dlog = torch.full((T, E), float("nan"), device=dev)
    dx = dx0.to(dev)
    dwr = torch.full((E, d), float("nan"), device=dev)
    db = torch.full((E,), float("nan"), device=dev)
    ws = moe.new_backward_workspace(cfg)
    moe.moe_route_backward(cfg, g["logits"].to(dev), g["ids"].to(dev), g["weights"].to(dev), dwts.to(dev), dlog,
                           x=dinp["x"], w_router=dinp["w_router"], counts_pre=g["counts_pre"].to(dev),
                           token_mask=dinp.get("token_mask"), d_aux=d_aux, dx=dx, dw_router=dwr, dbias=db, ws=ws)
    torch.cuda.synchronize()
    real = np.ones(T, dtype=bool) if mask is None else mask.numpy() != 0
    probs = np.zeros((T, E))
    probs[real] = oracle.router_probs(g["logits"].numpy()[real], cfg.temperature)
    dl_ref = oracle.router_backward(probs, g["ids"].numpy(), g["weights"].numpy(), real, dwts.numpy(),
                                    g["counts_pre"].numpy(), tau=cfg.temperature,
                                    renormalize=cfg.renormalize and not cfg.straight_through,
                                    aux_coef=cfg.aux_coef, d_aux=d_aux)
    dwr_ref, db_ref, dxr_ref = oracle.router_input_grads(dl_ref, inp["x"], inp["w_router"])
    errs = {"dL": normwise(dlog.cpu().numpy(), dl_ref), "dW_r": normwise(dwr.cpu().numpy(), dwr_ref),
            "db": normwise(db.cpu().numpy(), db_ref)}
    dx_ref = dx0.double().numpy() + dxr_ref
    errs["dx"] = normwise(dx.cpu().double().numpy(), dx_ref)
    print(f"[gpu] {name}: " + " ".join(f"{a} {b:.2e}" for a, b in errs.items()), flush=True)
    assert not real.all() or np.all(np.isfinite(dlog.cpu().numpy()))
    assert np.all(dlog.cpu().numpy()[~real] == 0.0), "padding tokens must get a zero logit gradient"
    # fp32 arithmetic against float64: 1e-5 normwise; dx is stored in act (one more rounding)
    assert errs["dL"] <= 1e-5 and errs["dW_r"] <= 1e-5 and errs["db"] <= 1e-5, errs
    assert errs["dx"] <= (1e-5 if cfg.dtype == "f32" else 4e-3), errs


FULL_CASES = {
    "bwd_all_bf16": (derived(BASE, name="bwd_all_bf16", T=600, d_model=256, d_ffn=384, num_experts=6), 0.7),
    # fp32, full-softmax weights, capacity drops, Gumbel selection, bias
    "bwd_all_f32_capacity": (derived(WORKLOADS["skewed_gumbel_capacity"], name="bwd_all_f32_capacity", T=300,
                                     d_model=64, d_ffn=96, num_experts=5, top_k=3, dtype="f32", renormalize=False,
                                     capacity_factor=(4, 5)), 1.0),
    # shared expert, additive noise, padding tokens
    "bwd_all_shared_noise_padding": (derived(WORKLOADS["main_noise_padding"], name="bwd_all_shared_noise_padding",
                                             T=520, d_model=128, d_ffn=192, num_experts=8, d_ffn_shared=160),
                                     1.0),
    # the straight-through estimator: unit gate weights, Gumbel selection, capacity drops
    "bwd_all_straight_through": (derived(WORKLOADS["skewed_gumbel_capacity"], name="bwd_all_straight_through",
                                         T=600, d_model=128, d_ffn=192, num_experts=8, straight_through=True), 1.0),
    # 256 x 256 grouped GEMMs on both the routed and the shared products
    "bwd_all_big_shared": (derived(BASE, name="bwd_all_big_shared", T=2048, d_model=128, d_ffn=256, num_experts=2,
                                   d_ffn_shared=256), 0.5),
    # dx formed in one pass from the gather and the router term: top-1 with 16 experts (a token's
    # second row absent), and 12 experts over d = 2056 (a second 2048-column block with 8 columns)
    "bwd_all_e16_top1": (derived(BASE, name="bwd_all_e16_top1", T=500, d_model=200, d_ffn=128, num_experts=16,
                                 top_k=1), 1.0),
    "bwd_all_e12_d2056": (derived(BASE, name="bwd_all_e12_d2056", T=333, d_model=2056, d_ffn=64, num_experts=12),
                          1.0),
    # degenerate cases: every slot dropped (C = 0: only the aux term reaches the router), one token,
    # the most experts and slots (64, top-8: most experts get no rows), every token padding
    "bwd_all_zero_capacity": (derived(BASE, name="bwd_all_zero_capacity", T=200, d_model=64, d_ffn=64,
                                      num_experts=4), 1.0, {"capacity": 0}),
    "bwd_all_one_token": (derived(BASE, name="bwd_all_one_token", T=1, d_model=64, d_ffn=64, num_experts=4), 1.0),
    "bwd_all_e64_k8": (derived(BASE, name="bwd_all_e64_k8", T=300, d_model=64, d_ffn=64, num_experts=64, top_k=8),
                       1.0),
    "bwd_all_all_padding": (derived(WORKLOADS["main_noise_padding"], name="bwd_all_all_padding", T=100, d_model=64,
                                    d_ffn=64, padding=1.0), 1.0),
}


def _oracle_forward_from_gpu(g, inp, cfg):
    """The oracle's Forward record holding the GPU forward's own routing, dispatch, H and Y."""
    T, E = cfg.T, cfg.num_experts
    mask = inp.get("token_mask")
    real = np.ones(T, dtype=bool) if mask is None else mask.numpy() != 0
    logits = g["logits"].numpy()
    probs = np.zeros((T, E))
    probs[real] = oracle.router_probs(logits[real], cfg.temperature)
    N = int(g["offsets"][-1])
    r = oracle.Routing(logits, None, g["ids"].numpy(), g["weights"].numpy(), probs, real, None)
    dp = oracle.Dispatch(g["counts_pre"].numpy(), g["counts"].numpy(), g["offsets"].numpy(),
                         g["perm_token"].numpy()[:N], g["row_of"].numpy(), g["dropped"].numpy(),
                         int(g["n_dropped"][0]), None)
    return oracle.Forward(r, dp, cfg.capacity, g["h"][:N], g["y"][:N], g["out"], tuple(g["aux"].tolist()))


@pytest.mark.parametrize("name", list(FULL_CASES))
def test_moe_backward_whole_layer(name):
    """moe_backward from the forward's workspace against the oracle's backward of the same forward."""
    w, d_aux, *changes = FULL_CASES[name]
    print(f"[gpu] moe_backward {name}: {w} d_aux={d_aux} {changes}", flush=True)
    cfg = moe.config_for(w)
    if changes:
        cfg = dataclasses.replace(cfg, **changes[0])
    inp = make_inputs(w)
    dinp = to_device(inp)
    g = run_gpu(cfg, dinp)          # the intermediates, from a forward with debug buffers
    T, d, f, E = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts
    fs = cfg.d_ffn_shared
    dt, st = cfg.torch_dtype, cfg.dtype
    dev = "cuda"
    fwd_ws = moe.new_workspace(cfg, dev)
    out, aux = moe.forward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], bias=dinp["bias"],
                           gumbel=dinp["gumbel"], token_mask=dinp.get("token_mask"), w1_shared=dinp.get("w1_shared"),
                           w2_shared=dinp.get("w2_shared"), ws=fwd_ws)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), g["out"]), "the forward is deterministic"
    gen = torch.Generator().manual_seed(5)
    d_out = torch.randn(T, d, generator=gen).to(dt)
    nan = float("nan")
    grads = {"dx": torch.full((T, d), nan, dtype=dt, device=dev),
             "dw_router": torch.full((E, d), nan, device=dev), "dbias": torch.full((E,), nan, device=dev),
             "dw1": torch.full((E, f, d), nan, device=dev), "dw2": torch.full((E, d, f), nan, device=dev)}
    if fs:
        grads["dw1_shared"] = torch.full((fs, d), nan, device=dev)
        grads["dw2_shared"] = torch.full((d, fs), nan, device=dev)
    ws = moe.new_backward_workspace(cfg)
    moe.moe_backward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], d_out.to(dev), fwd_ws, grads["dx"], ws,
                     token_mask=dinp.get("token_mask"), w1_shared=dinp.get("w1_shared"),
                     w2_shared=dinp.get("w2_shared"), d_aux=d_aux,
                     **{k: v for k, v in grads.items() if k != "dx"})
    torch.cuda.synchronize()
    fw = _oracle_forward_from_gpu(g, inp, cfg)
    ref = oracle.backward(fw, inp["x"], inp["w_router"], inp["w1"], inp["w2"], d_out, storage=st,
                          tau=cfg.temperature, renormalize=cfg.renormalize, aux_coef=cfg.aux_coef, d_aux=d_aux,
                          straight_through=cfg.straight_through,
                          w1_shared=inp.get("w1_shared"), w2_shared=inp.get("w2_shared"))
    pairs = {"dx": ref.dx, "dw_router": ref.dw_router, "dbias": ref.dbias, "dw1": ref.dw1, "dw2": ref.dw2}
    if fs:
        pairs["dw1_shared"] = ref.dw1_shared
        pairs["dw2_shared"] = ref.dw2_shared
    errs = {n: normwise(grads[n].cpu().double().numpy(), r) for n, r in pairs.items()}
    print(f"[gpu] {name}: " + " ".join(f"{a} {b:.2e}" for a, b in errs.items()), flush=True)
    # bf16: the products stored in bf16 (dY, dA, dXp, dx) give the storage tolerance; the router's
    # gradients come from fp32 gate-weight gradients (1e-5 for fp32 arithmetic, 1e-4 once dx's
    # bf16 values are not involved)
    tol = NORM_TOL[st]
    for n, e in errs.items():
        lim = 1e-4 if (n in ("dw_router", "dbias")) else tol
        assert e <= lim, (n, errs)


SAMPLED_CASES = {
    "main": BASE,
    # d 4096: the dH GEMM (K = d, 64 stages) and the recomputed pre-activation have ~320 tiles, so
    # their last partial round is split in two K halves; the tail kernel sums the parts (and, for
    # the pre-activation, stores the sum and applies SiLU to it)
    "split_dh_d4096": derived(BASE, name="split_dh_d4096", T=4200, d_model=4096, d_ffn=2048),
}


@pytest.mark.parametrize("case", list(SAMPLED_CASES))
def test_moe_backward_full_size_sampled(case):
    """moe_backward at full size (the main layer: 16384 tokens, d 2048, f 4096, 8 experts, top-2,
    the launch configuration the bench's backward leg times; and a d 4096 layer whose dH GEMM
    splits its last round) on outputs the oracle can form exactly one by one: the hidden units are
    independent in dW1 / dW2 (the oracle's expert backward on 16 sampled units gives those rows of
    dW1 and columns of dW2 exactly), dXp is per row (the oracle's expert backward on 48 sampled
    tokens' rows gives their dx), and the router gradients are cheap in full."""
    w, d_aux = SAMPLED_CASES[case], 1.0
    print(f"[gpu] moe_backward full size sampled: {w}", flush=True)
    cfg = moe.config_for(w)
    inp = make_inputs(w)
    dinp = to_device(inp)
    g = run_gpu(cfg, dinp)
    T, d, f, E, k = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts, cfg.top_k
    dt = cfg.torch_dtype
    dev = "cuda"
    fwd_ws = moe.new_workspace(cfg, dev)
    moe.forward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], bias=dinp["bias"], gumbel=dinp["gumbel"],
                ws=fwd_ws)
    gen = torch.Generator().manual_seed(6)
    d_out = torch.randn(T, d, generator=gen).to(dt)
    dx = torch.empty(T, d, dtype=dt, device=dev)
    dwr = torch.empty(E, d, device=dev)
    db = torch.empty(E, device=dev)
    dw1 = torch.empty(E, f, d, device=dev)
    dw2 = torch.empty(E, d, f, device=dev)
    moe.moe_backward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], d_out.to(dev), fwd_ws, dx,
                     moe.new_backward_workspace(cfg), d_aux=d_aux, dw_router=dwr, dbias=db, dw1=dw1, dw2=dw2)
    torch.cuda.synchronize()
    row_of = g["row_of"].numpy()
    offsets = g["offsets"].numpy()
    N = int(offsets[-1])
    dy, dwts = oracle.combine_backward(d_out, g["y"], row_of, g["weights"].numpy(), "f64")
    rng = np.random.default_rng(8)
    # 16 hidden units: dW1[:, u, :] and dW2[:, :, u]
    u = np.sort(rng.choice(f, 16, replace=False))
    w1_64 = inp["w1"].double().numpy()
    w2_64 = inp["w2"].double().numpy()
    h = g["h"][:N]
    _, dw1_u, dw2_u = oracle.expert_ffn_backward(g["xp"][:N], offsets, w1_64[:, u, :], w2_64[:, :, u],
                                                 h[:, u], dy[:N], "f64")
    e1 = normwise(dw1.cpu().numpy()[:, u, :], dw1_u)
    e2 = normwise(dw2.cpu().numpy()[:, :, u], dw2_u)
    # 48 tokens: their kept rows, ascending (grouped by expert), through the full expert weights
    toks = np.sort(rng.choice(T, 48, replace=False))
    rows = np.sort(row_of[toks][row_of[toks] >= 0])
    off_s = np.searchsorted(rows, offsets).astype(np.int32)
    dxp_s, _, _ = oracle.expert_ffn_backward(g["xp"][rows], off_s, w1_64, w2_64, g["h"][rows], dy[rows], "f64")
    where = {int(r): i for i, r in enumerate(rows)}
    probs = oracle.router_probs(g["logits"].numpy(), cfg.temperature)
    real = np.ones(T, dtype=bool)
    dl = oracle.router_backward(probs, g["ids"].numpy(), g["weights"].numpy(), real, dwts, g["counts_pre"].numpy(),
                                tau=cfg.temperature, renormalize=cfg.renormalize, aux_coef=cfg.aux_coef, d_aux=d_aux)
    dwr_ref, db_ref, _ = oracle.router_input_grads(dl, inp["x"], inp["w_router"])
    wr64 = inp["w_router"].double().numpy()
    dx_ref = np.zeros((len(toks), d))
    for i, t in enumerate(toks):
        for j in range(k):
            if row_of[t, j] >= 0:
                dx_ref[i] += dxp_s[where[int(row_of[t, j])]]
        dx_ref[i] += dl[t] @ wr64
    ex = normwise(dx.cpu().double().numpy()[toks], dx_ref)
    er = normwise(dwr.cpu().numpy(), dwr_ref)
    eb = normwise(db.cpu().numpy(), db_ref)
    print(f"[gpu] full size: dW1[units] {e1:.2e} dW2[units] {e2:.2e} dx[tokens] {ex:.2e} dW_r {er:.2e} db {eb:.2e}",
          flush=True)
    tol = NORM_TOL[cfg.dtype]
    assert e1 <= tol and e2 <= tol and ex <= tol, (e1, e2, ex)
    assert er <= 1e-4 and eb <= 1e-4, (er, eb)


def test_moe_backward_is_deterministic():
    """Two moe_backward calls on the same forward give bit-identical gradients, including the
    weight gradients whose reduction is split in two halves added into a zeroed output (a
    shared expert's, and the routed experts' when there are fewer tiles than CUs)."""
    w = derived(BASE, name="bwd_repeat", T=1500, d_model=256, d_ffn=512, num_experts=4, d_ffn_shared=512)
    print(f"[gpu] moe_backward repeat: {w}", flush=True)
    cfg = moe.config_for(w)
    dinp = to_device(make_inputs(w))
    T, d, f, E, fs = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts, cfg.d_ffn_shared
    fwd_ws = moe.new_workspace(cfg, "cuda")
    moe.forward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], w1_shared=dinp["w1_shared"],
                w2_shared=dinp["w2_shared"], ws=fwd_ws)
    d_out = torch.randn(T, d, generator=torch.Generator().manual_seed(3)).to(cfg.torch_dtype).cuda()
    runs = []
    for _ in range(2):
        g = {"dw_router": torch.empty(E, d, device="cuda"), "dbias": torch.empty(E, device="cuda"),
             "dw1": torch.empty(E, f, d, device="cuda"), "dw2": torch.empty(E, d, f, device="cuda"),
             "dw1_shared": torch.empty(fs, d, device="cuda"), "dw2_shared": torch.empty(d, fs, device="cuda")}
        dx = torch.empty(T, d, dtype=cfg.torch_dtype, device="cuda")
        moe.moe_backward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], d_out, fwd_ws, dx,
                         moe.new_backward_workspace(cfg), w1_shared=dinp["w1_shared"], w2_shared=dinp["w2_shared"],
                         d_aux=1.0, **g)
        g["dx"] = dx
        runs.append({k: v.cpu() for k, v in g.items()})
    torch.cuda.synchronize()
    for k in runs[0]:
        assert torch.equal(runs[0][k], runs[1][k]), k


KEEP_CASES = {
    "keep_big": derived(BASE, name="keep_big", T=2048, d_model=256, d_ffn=512, num_experts=2),
    "keep_main": BASE,                                                    # 256 x 256 tiles + split tail
    # GEMM1 with K = d = 4096: its last partial round is split, and the tail kernel stores the
    # pre-activation and its SiLU
    "keep_split_k4096": derived(BASE, name="keep_split_k4096", T=4200, d_model=4096, d_ffn=2048),
    # one round of 32 tiles with 16 stages per tile, pre-activation kept
    "keep_split_single": derived(BASE, name="keep_split_single", T=2048, d_model=1024, d_ffn=512, num_experts=2),
    "keep_stream": derived(WORKLOADS["small_t_streaming"], name="keep_stream", T=96, d_model=256, d_ffn=512),
    # half-width narrow slices storing the pre-activation too
    "keep_half_slices": derived(BASE, name="keep_half_slices", T=4104, d_model=256, d_ffn=4096),
    "keep_f32": derived(WORKLOADS["tiny_f32"], name="keep_f32", T=150, d_model=48, d_ffn=40, num_experts=5, top_k=3),
    "keep_shared_padding": derived(WORKLOADS["main_noise_padding"], name="keep_shared_padding", T=520, d_model=128,
                                   d_ffn=192, d_ffn_shared=160),
}


@pytest.mark.parametrize("name", list(KEEP_CASES))
def test_keep_preact_is_bitwise_the_recompute(name):
    """keep_preact = 1: the forward's SiLU GEMM also stores its pre-activation and moe_backward
    reads it instead of recomputing it. Same kernels, tiles and reduction order, so the output
    and every gradient must be bit-identical to the recomputing path."""
    w = KEEP_CASES[name]
    print(f"[gpu] keep_preact {name}: {w}", flush=True)
    cfg0 = moe.config_for(w)
    cfg1 = dataclasses.replace(cfg0, keep_preact=True)
    dinp = to_device(make_inputs(w))
    T, d, f, E, fs = cfg0.T, cfg0.d_model, cfg0.d_ffn, cfg0.num_experts, cfg0.d_ffn_shared
    d_out = torch.randn(T, d, generator=torch.Generator().manual_seed(4)).to(cfg0.torch_dtype).cuda()
    res = []
    for cfg in (cfg0, cfg1):
        ws = moe.new_workspace(cfg, "cuda")
        out, aux = moe.forward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], bias=dinp["bias"],
                               gumbel=dinp["gumbel"], token_mask=dinp.get("token_mask"),
                               w1_shared=dinp.get("w1_shared"), w2_shared=dinp.get("w2_shared"), ws=ws)
        g = {"dw_router": torch.empty(E, d, device="cuda"), "dbias": torch.empty(E, device="cuda"),
             "dw1": torch.empty(E, f, d, device="cuda"), "dw2": torch.empty(E, d, f, device="cuda")}
        if fs:
            g.update(dw1_shared=torch.empty(fs, d, device="cuda"), dw2_shared=torch.empty(d, fs, device="cuda"))
        dx = torch.empty(T, d, dtype=cfg.torch_dtype, device="cuda")
        moe.moe_backward(cfg, dinp["x"], dinp["w_router"], dinp["w1"], dinp["w2"], d_out, ws, dx,
                         moe.new_backward_workspace(cfg), token_mask=dinp.get("token_mask"),
                         w1_shared=dinp.get("w1_shared"), w2_shared=dinp.get("w2_shared"), d_aux=1.0, **g)
        g.update(out=out, aux=aux, dx=dx)
        torch.cuda.synchronize()
        res.append({k: v.cpu() for k, v in g.items()})
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k
