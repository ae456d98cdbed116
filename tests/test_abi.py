"""The C ABI without a GPU: the library loads, exports every declared symbol, and every host-side
validation path returns its status code before anything is launched."""
import ctypes
import os
import re

import pytest

import oracle
import sparse_mixture_experts_02_amd as moe
from sparse_mixture_experts_02_amd import binding
from sparse_mixture_experts_02_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    declared = _declared_functions()
    assert declared == sorted(binding.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    assert moe.status_string(0) == "ok"
    assert moe.status_string(3) == "workspace too small"
    assert moe.status_string(99) == "unknown status"


def _cfg(**kw):
    base = dict(T=64, d_model=32, d_ffn=64, num_experts=4, top_k=2, dtype="f32")
    base.update(kw)
    return moe.MoEConfig(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"T": 0}, 1), ({"T": -3}, 1), ({"T": (1 << 24) + 1}, 1),
    ({"d_model": 12}, 1), ({"d_model": 0}, 1), ({"d_ffn": 20}, 1), ({"d_ffn": 32776}, 1),
    ({"num_experts": 0}, 1), ({"num_experts": 65}, 1),
    ({"top_k": 0}, 1), ({"top_k": 5}, 1), ({"num_experts": 16, "top_k": 9}, 1),
    ({"num_experts": 64, "top_k": 8}, 0),
    ({"capacity": -2}, 1), ({"capacity": 0}, 0), ({"capacity": -1}, 0),
    ({"temperature": 0.0}, 1), ({"temperature": -1.0}, 1), ({"temperature": float("inf")}, 1),
    ({"temperature": float("nan")}, 1), ({"aux_coef": float("nan")}, 1),
    ({"dtype": "bf16", "weight_dtype": "f32"}, 2), ({"dtype": "f16"}, 1),
    ({"d_ffn_shared": 64}, 0), ({"d_ffn_shared": 12}, 1), ({"d_ffn_shared": -8}, 1), ({"d_ffn_shared": 32776}, 1),
    # 4-bit weights: bf16 activations, d and f multiples of 512, the weight-streaming regime, no shared expert
    ({"dtype": "bf16", "weight_dtype": "int4", "d_model": 512, "d_ffn": 1024, "T": 128}, 0),
    ({"dtype": "f32", "weight_dtype": "int4", "d_model": 512, "d_ffn": 512}, 2),
    ({"dtype": "bf16", "weight_dtype": "int4", "d_model": 256, "d_ffn": 512}, 2),
    ({"dtype": "bf16", "weight_dtype": "int4", "d_model": 512, "d_ffn": 512, "T": 129}, 2),
    ({"dtype": "bf16", "weight_dtype": "int4", "d_model": 512, "d_ffn": 512, "d_ffn_shared": 64}, 2),
])
def test_validate_config(kw, status):
    assert moe.validate_config(_cfg(**kw)) == status


def test_validate_rejects_bad_renormalize_flag():
    c = _cfg().to_c()
    c.renormalize = 2
    assert binding.lib().moe_validate_config(ctypes.byref(c)) == 1
    c = _cfg().to_c()
    c.noise_in_logits = 2
    assert binding.lib().moe_validate_config(ctypes.byref(c)) == 1
    c.noise_in_logits = 1
    assert binding.lib().moe_validate_config(ctypes.byref(c)) == 0
    c.straight_through = 2
    assert binding.lib().moe_validate_config(ctypes.byref(c)) == 1
    c.straight_through = 1
    assert binding.lib().moe_validate_config(ctypes.byref(c)) == 0
    c.keep_preact = 2
    assert binding.lib().moe_validate_config(ctypes.byref(c)) == 1
    c.keep_preact = 1
    assert binding.lib().moe_validate_config(ctypes.byref(c)) == 0
    q4 = _cfg(dtype="bf16", weight_dtype="int4", d_model=512, d_ffn=1024, T=128)
    assert moe.validate_config(q4) == 0
    assert moe.validate_config(__import__("dataclasses").replace(q4, keep_preact=True)) == 2
    # the kept pre-activation [T*k, f] act is part of the forward workspace
    base = _cfg()
    kept = __import__("dataclasses").replace(base, keep_preact=True)
    assert moe.workspace_bytes(kept) >= moe.workspace_bytes(base) + base.T * base.top_k * base.d_ffn * 4
    assert binding.lib().moe_validate_config(None) == 1


def test_capacity_from_factor_matches_oracle():
    for w in WORKLOADS.values():
        if w.capacity_factor is None:
            continue
        assert moe.capacity_from_factor(w.T, w.top_k, w.num_experts, *w.capacity_factor) == \
            oracle.capacity_from_factor(w.T, w.top_k, w.num_experts, w.capacity_factor)
    for T, k, E, n, d in [(4, 2, 4, 1, 1), (1000, 3, 7, 12, 10), (1, 1, 64, 1, 1), (16777216, 8, 1, 3, 2)]:
        assert moe.capacity_from_factor(T, k, E, n, d) == min(oracle.capacity_from_factor(T, k, E, (n, d)),
                                                              2 ** 31 - 1)
    assert moe.capacity_from_factor(0, 2, 4, 1, 1) == -1
    assert moe.capacity_from_factor(4, 2, 4, 0, 1) == -1


def test_int4_sizes_and_quantize_validation():
    assert moe.int4_bytes(16 * 4096, 2048) == 16 * 4096 * 1024 + 16 * 4096 * 32 * 2
    assert moe.int4_bytes(16, 128) == 1024 + 16 * 2 * 2
    assert moe.int4_bytes(0, 128) == 0 and moe.int4_bytes(24, 128) == 0 and moe.int4_bytes(16, 192) == 0
    L = binding.lib()
    fake, odd = ctypes.c_void_p(256), ctypes.c_void_p(264)
    assert L.moe_quantize_int4(16, 192, fake, fake, None) == 1
    assert L.moe_quantize_int4(20, 128, fake, fake, None) == 1
    assert L.moe_quantize_int4(16, 128, None, fake, None) == 1
    assert L.moe_quantize_int4(16, 128, fake, odd, None) == 1


def test_workspace_bytes():
    assert moe.workspace_bytes(_cfg(T=0)) == 0
    small = moe.workspace_bytes(_cfg())
    big = moe.workspace_bytes(_cfg(T=128))
    assert 0 < small < big
    c = moe.config_for(WORKLOADS["main_bf16"])
    # Xp, H and Y dominate: (2 d + f) * T * k * 2 bytes
    assert moe.workspace_bytes(c) >= (2 * 2048 + 4096) * 16384 * 2 * 2


def test_calls_validate_before_any_launch():
    """Invalid arguments come back as status codes from host code (no GPU is touched)."""
    L = binding.lib()
    good = _cfg().to_c()
    bad = _cfg(T=0).to_c()
    fake = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    B = ctypes.byref
    # moe_route(cfg, x, w_router, bias, noise, token_mask, logits_in, logits_out, probs_out, ids, weights, ws,
    #           ws_bytes, stream)
    def route(x=fake, wr=fake, ids=fake, wts=fake, ws=fake, nbytes=1 << 30, cfg=good):
        return L.moe_route(B(cfg), x, wr, None, None, None, None, None, None, ids, wts, ws, nbytes, None)

    # moe_forward(cfg, x, w_router, bias, noise, token_mask, w1, w2, w1_shared, w2_shared, out, aux, dbg, ws,
    #             ws_bytes, stream)
    def forward(x=fake, wr=fake, w1=fake, w2=fake, w1s=None, w2s=None, out=fake, aux=fake, dbg=None, ws=fake,
                nbytes=1 << 30, cfg=good):
        return L.moe_forward(B(cfg), x, wr, None, None, None, w1, w2, w1s, w2s, out, aux, dbg, ws, nbytes, None)

    # moe_combine(cfg, y, row_of, weights, y_shared, out, stream)
    def combine(y=fake, row_of=fake, wts=fake, ys=None, out=fake, cfg=good):
        return L.moe_combine(B(cfg), y, row_of, wts, ys, out, None)

    # moe_aux_loss(cfg, probs, logits, token_mask, counts_pre, aux, ws, ws_bytes, stream)
    def aux_loss(probs=fake, logits=None, counts=fake, aux=fake, ws=fake, nbytes=1 << 30, cfg=good):
        return L.moe_aux_loss(B(cfg), probs, logits, None, counts, aux, ws, nbytes, None)

    # invalid configuration
    assert route(cfg=bad) == 1
    assert L.moe_dispatch(B(bad), *([fake] * 10), fake, 1 << 30, None) == 1
    assert L.moe_expert_ffn(B(bad), *([fake] * 6), fake, 1 << 30, None) == 1
    assert combine(cfg=bad) == 1
    assert aux_loss(cfg=bad) == 1
    assert forward(cfg=bad) == 1
    # null required pointers
    assert route(ids=None) == 1
    assert route(x=None, wr=None) == 1
    assert L.moe_dispatch(B(good), *([fake] * 9), None, fake, 1 << 30, None) == 1
    assert L.moe_expert_ffn(B(good), fake, fake, fake, None, fake, fake, fake, 1 << 30, None) == 1
    assert combine(row_of=None) == 1
    assert aux_loss(probs=None, logits=None) == 1
    assert forward(out=None) == 1
    assert forward(aux=None) == 1
    # misaligned activation pointers
    odd = ctypes.c_void_p(256 + 8)
    assert combine(y=odd) == 1
    assert combine(ys=odd) == 1
    assert forward(x=odd) == 1
    # shared expert: its weights are required (and aligned) when d_ffn_shared > 0
    shared = _cfg(d_ffn_shared=16).to_c()
    need_s = moe.workspace_bytes(_cfg(d_ffn_shared=16))
    assert forward(cfg=shared, nbytes=need_s) == 1
    assert forward(cfg=shared, w1s=fake, nbytes=need_s) == 1
    assert forward(cfg=shared, w1s=fake, w2s=odd, nbytes=need_s) == 1
    assert need_s > moe.workspace_bytes(_cfg())
    # misaligned router weight (read with 16-byte loads)
    assert forward(wr=odd) == 1
    assert route(wr=odd) == 1
    # workspace: missing, misaligned, too small
    need = moe.workspace_bytes(_cfg())
    assert route(ws=None, nbytes=need) == 1
    assert route(ws=odd, nbytes=need) == 1
    assert route(nbytes=need - 1) == 3
    assert L.moe_dispatch(B(good), *([fake] * 10), fake, need - 1, None) == 3
    assert L.moe_expert_ffn(B(good), *([fake] * 6), fake, 16, None) == 3
    assert aux_loss(nbytes=0) == 3
    assert forward(nbytes=need - 1) == 3
    # too few timing events
    dbg = binding._Debug()
    dbg.events = fake
    dbg.n_events = binding.MOE_FORWARD_NUM_KERNELS
    assert forward(dbg=B(dbg), nbytes=need) == 1


def test_route_backward_validation():
    L = binding.lib()
    good = _cfg().to_c()
    fake, odd = ctypes.c_void_p(256), ctypes.c_void_p(264)
    B = ctypes.byref
    need = moe.backward_workspace_bytes(_cfg())

    # moe_route_backward(cfg, x, w_router, logits, ids, weights, dweights, counts_pre, token_mask, d_aux,
    #                    dlogits, dx, dw_router, dbias, ws, ws_bytes, stream)
    def rb(x=fake, wr=fake, logits=fake, dl=fake, counts=fake, d_aux=1.0, dx=fake, dwr=fake, ws=fake, nbytes=need,
           cfg=good):
        return L.moe_route_backward(B(cfg), x, wr, logits, fake, fake, fake, counts, None, d_aux, dl, dx, dwr, None,
                                    ws, nbytes, None)

    assert rb(cfg=_cfg(T=0).to_c()) == 1
    assert rb(logits=None) == 1 and rb(dl=None) == 1
    assert rb(counts=None) == 1                       # the aux term needs the counts
    assert rb(d_aux=float("nan")) == 1
    assert rb(dx=fake, wr=None) == 1 and rb(dx=odd) == 1
    assert rb(dwr=fake, x=None) == 1 and rb(x=odd) == 1 and rb(ws=None) == 1
    assert rb(nbytes=need - 1) == 3
    assert need > moe.backward_workspace_bytes(_cfg(T=32)) > 0


def test_whole_backward_validation():
    L = binding.lib()
    fake, odd = ctypes.c_void_p(256), ctypes.c_void_p(264)
    B = ctypes.byref
    need_f, need_b = moe.workspace_bytes(_cfg()), moe.backward_workspace_bytes(_cfg())

    # moe_backward(cfg, x, w_router, token_mask, w1, w2, w1s, w2s, d_out, d_aux, fwd_ws, fwd_bytes, dx,
    #              dw_router, dbias, dw1, dw2, dw1s, dw2s, ws, ws_bytes, stream)
    def bw(cfg=None, x=fake, d_out=fake, fwd=fake, fb=need_f, dx=fake, ws=fake, wb=need_b, w1s=None, w2s=None,
           d_aux=0.0):
        c = cfg or _cfg().to_c()
        return L.moe_backward(B(c), x, fake, None, fake, fake, w1s, w2s, d_out, d_aux, fwd, fb, dx, None, None,
                              None, None, None, None, ws, wb, None)

    assert bw(cfg=_cfg(T=0).to_c()) == 1
    assert bw(x=None) == 1 and bw(d_out=None) == 1 and bw(fwd=None) == 1 and bw(dx=None) == 1 and bw(ws=None) == 1
    assert bw(x=odd) == 1 and bw(fwd=odd) == 1 and bw(dx=odd) == 1
    assert bw(d_aux=float("inf")) == 1
    assert bw(fb=need_f - 1) == 3 and bw(wb=need_b - 1) == 3
    shared = _cfg(d_ffn_shared=16)
    assert bw(cfg=shared.to_c(), fb=moe.workspace_bytes(shared), wb=moe.backward_workspace_bytes(shared)) == 1
    q4 = _cfg(dtype="bf16", weight_dtype="int4", d_model=512, d_ffn=1024, T=128)
    assert bw(cfg=q4.to_c(), fb=1 << 40, wb=1 << 40) == 2


def test_forward_noalloc_validates_before_touching_the_gpu():
    """moe_forward_noalloc (the variant for callers that cannot allocate): its limit, and every
    argument error, come back from host code before its static workspace is looked up."""
    L = binding.lib()
    B = ctypes.byref
    fake = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(256 + 8)
    assert moe.forward_noalloc_max_bytes() == 64 << 20

    def fwd(cfg, x=fake, wr=fake, w1=fake, w2=fake, w1s=None, w2s=None, out=fake, aux=fake):
        return L.moe_forward_noalloc(B(cfg.to_c()), x, wr, None, None, None, w1, w2, w1s, w2s, out, aux, None)

    assert fwd(_cfg(T=0)) == 1
    assert fwd(_cfg(), out=None) == 1
    assert fwd(_cfg(), aux=None) == 1
    assert fwd(_cfg(), x=odd) == 1
    assert fwd(_cfg(d_ffn_shared=16), w1s=fake) == 1
    # the main layer's workspace (~513 MiB) is beyond the array: rejected with a clear status
    main = moe.config_for(WORKLOADS["main_bf16"])
    assert moe.workspace_bytes(main) > moe.forward_noalloc_max_bytes()
    assert fwd(main) == 3
    # the weight-streaming layer fits
    small = moe.config_for(WORKLOADS["small_t_streaming"])
    assert moe.workspace_bytes(small) <= moe.forward_noalloc_max_bytes()
