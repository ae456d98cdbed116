"""ctypes binding of libmoe.so (include/moe.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks shapes, dtypes and
contiguity, and passes raw pointers plus torch's current HIP stream to the C ABI. All compute
runs in the library's HIP kernels; there is no fallback path. If libmoe.so has not been built,
the first call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_F32 = 0
MOE_BF16 = 1
MOE_INT4 = 2
MOE_NO_CAPACITY = -1
MOE_FORWARD_NUM_KERNELS = 8
FORWARD_KERNEL_NAMES = ("route", "dispatch_hist", "dispatch_scan_aux", "dispatch_gather", "gemm1_silu", "gemm2",
                        "shared_ffn", "combine")

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

# Every symbol include/moe.h declares.
EXPORTED_SYMBOLS = ("moe_status_string", "moe_validate_config", "moe_capacity_from_factor",
                    "moe_int4_bytes", "moe_quantize_int4", "moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                    "moe_aux_loss", "moe_forward", "moe_backward_workspace_bytes", "moe_combine_backward",
                    "moe_expert_ffn_backward", "moe_dispatch_backward", "moe_route_backward",
                    "moe_backward", "moe_forward_noalloc_max_bytes", "moe_forward_noalloc")


class MoEError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class _Config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("temperature", ctypes.c_float), ("renormalize", ctypes.c_int32),
                ("aux_coef", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("noise_in_logits", ctypes.c_int32),
                ("d_ffn_shared", ctypes.c_int32), ("straight_through", ctypes.c_int32),
                ("keep_preact", ctypes.c_int32)]


class _Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("logits", "probs", "ids", "weights", "counts_pre", "counts",
                                                "offsets", "perm_token", "row_of", "dropped", "n_dropped",
                                                "xp", "h", "y", "y_shared", "events")] + [("n_events", ctypes.c_int32)]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """Mirror of moe_config_t."""
    T: int
    d_model: int
    d_ffn: int
    num_experts: int
    top_k: int
    capacity: int = MOE_NO_CAPACITY
    temperature: float = 1.0
    renormalize: bool = True
    aux_coef: float = 0.01
    dtype: str = "bf16"          # "bf16" or "f32" (activations and expert weights)
    weight_dtype: Optional[str] = None   # defaults to dtype; "int4" = packed 4-bit expert weights
    noise_in_logits: bool = False        # the noise input: Gumbel key noise (False) or additive logit noise
    d_ffn_shared: int = 0                # width of the shared expert (0: none)
    straight_through: bool = False       # gate weights 1, gradient through the full softmax
    keep_preact: bool = False            # training: the forward keeps Xp W1^T for the backward

    def to_c(self) -> _Config:
        dt = {"f32": MOE_F32, "bf16": MOE_BF16, "int4": MOE_INT4}
        wd = self.weight_dtype or self.dtype
        return _Config(self.T, self.d_model, self.d_ffn, self.num_experts, self.top_k, self.capacity,
                       self.temperature, int(self.renormalize), self.aux_coef, dt.get(self.dtype, 99),
                       dt.get(wd, 99), int(self.noise_in_logits), self.d_ffn_shared, int(self.straight_through),
                       int(self.keep_preact))

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def int4(self) -> bool:
        return self.weight_dtype == "int4"


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_02_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(_Config)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_validate_config.restype = ctypes.c_int
        L.moe_validate_config.argtypes = [cfgp]
        L.moe_capacity_from_factor.restype = i32
        L.moe_capacity_from_factor.argtypes = [i32] * 5
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [cfgp]
        L.moe_int4_bytes.restype = sz
        L.moe_int4_bytes.argtypes = [ctypes.c_int64, i32]
        L.moe_quantize_int4.restype = ctypes.c_int
        L.moe_quantize_int4.argtypes = [ctypes.c_int64, i32, vp, vp, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [cfgp] + [vp] * 10 + [vp, sz, vp]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [cfgp] + [vp] * 10 + [vp, sz, vp]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [cfgp] + [vp] * 6 + [vp, sz, vp]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [cfgp] + [vp] * 5 + [vp]
        L.moe_aux_loss.restype = ctypes.c_int
        L.moe_aux_loss.argtypes = [cfgp] + [vp] * 5 + [vp, sz, vp]
        L.moe_backward_workspace_bytes.restype = sz
        L.moe_backward_workspace_bytes.argtypes = [cfgp]
        L.moe_combine_backward.restype = ctypes.c_int
        L.moe_combine_backward.argtypes = [cfgp] + [vp] * 6 + [vp]
        L.moe_expert_ffn_backward.restype = ctypes.c_int
        L.moe_expert_ffn_backward.argtypes = [cfgp] + [vp] * 9 + [vp, sz, vp]
        L.moe_dispatch_backward.restype = ctypes.c_int
        L.moe_dispatch_backward.argtypes = [cfgp] + [vp] * 3 + [vp]
        L.moe_route_backward.restype = ctypes.c_int
        L.moe_route_backward.argtypes = [cfgp] + [vp] * 8 + [ctypes.c_float] + [vp] * 5 + [sz, vp]
        L.moe_backward.restype = ctypes.c_int
        L.moe_backward.argtypes = [cfgp] + [vp] * 8 + [ctypes.c_float, vp, sz] + [vp] * 8 + [sz, vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward.argtypes = [cfgp] + [vp] * 11 + [ctypes.POINTER(_Debug), vp, sz, vp]
        L.moe_forward_noalloc_max_bytes.restype = sz
        L.moe_forward_noalloc_max_bytes.argtypes = []
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = [cfgp] + [vp] * 11 + [vp]
        _lib = L
    return _lib


# ------------------------------------------------------------------------------ host helpers

def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def validate_config(cfg: MoEConfig) -> int:
    c = cfg.to_c()
    return lib().moe_validate_config(ctypes.byref(c))


def capacity_from_factor(T: int, k: int, E: int, num: int, den: int) -> int:
    return lib().moe_capacity_from_factor(T, k, E, num, den)


def workspace_bytes(cfg: MoEConfig) -> int:
    c = cfg.to_c()
    return lib().moe_workspace_bytes(ctypes.byref(c))


def int4_bytes(rows: int, K: int) -> int:
    return lib().moe_int4_bytes(rows, K)


def quantize_int4(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed 4-bit copy (uint8 GPU tensor) of a bf16 GPU weight [..., K] through moe_quantize_int4."""
    K = w.shape[-1]
    rows = w.numel() // K
    n = int4_bytes(rows, K)
    if n == 0:
        raise ValueError(f"cannot quantise a [{rows}, {K}] weight (rows a multiple of 16, K of 128)")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check("moe_quantize_int4", lib().moe_quantize_int4(rows, K, _ptr(w, "w", dtype=torch.bfloat16),
                                                        _ptr(out, "packed", (n,), torch.uint8), _stream()))
    return out


def _wptr(cfg: MoEConfig, t, name: str, rows: int, K: int, shape):
    """Pointer of an expert weight: the bf16/fp32 tensor, or its packed 4-bit buffer."""
    if cfg.int4:
        return _ptr(t, name, (int4_bytes(rows, K),), torch.uint8)
    return _ptr(t, name, shape, cfg.torch_dtype)


def new_workspace(cfg: MoEConfig, device="cuda") -> torch.Tensor:
    n = workspace_bytes(cfg)
    if n == 0:
        raise MoEError("moe_workspace_bytes", validate_config(cfg))
    return torch.empty(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------ marshalling

def _ptr(t: Optional[torch.Tensor], name: str, shape=None, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(func: str, status: int):
    if status != MOE_OK:
        raise MoEError(func, status)


def moe_route(cfg: MoEConfig, x, w_router, ids, weights, ws, *, bias=None, gumbel=None, token_mask=None,
              logits_in=None, logits_out=None, probs_out=None):
    """`gumbel` is the noise input (Gumbel key noise, or additive logit noise with
    cfg.noise_in_logits); `token_mask` a [T] uint8 tensor, 0 marking padding tokens."""
    T, d, E, k = cfg.T, cfg.d_model, cfg.num_experts, cfg.top_k
    c = cfg.to_c()
    st = lib().moe_route(
        ctypes.byref(c),
        _ptr(x, "x", (T, d), cfg.torch_dtype) if logits_in is None else _ptr(x, "x"),
        _ptr(w_router, "w_router", (E, d), torch.float32) if logits_in is None else _ptr(w_router, "w_router"),
        _ptr(bias, "bias", (E,), torch.float32), _ptr(gumbel, "gumbel", (T, E), torch.float32),
        _ptr(token_mask, "token_mask", (T,), torch.uint8),
        _ptr(logits_in, "logits_in", (T, E), torch.float32), _ptr(logits_out, "logits_out", (T, E), torch.float32),
        _ptr(probs_out, "probs_out", (T, E), torch.float32), _ptr(ids, "ids", (T, k), torch.int32),
        _ptr(weights, "weights", (T, k), torch.float32), _ptr(ws, "ws"), ws.numel(), _stream())
    _check("moe_route", st)


def moe_dispatch(cfg: MoEConfig, ids, x, counts_pre, counts, offsets, perm_token, row_of, dropped, n_dropped,
                 xp, ws):
    T, d, E, k = cfg.T, cfg.d_model, cfg.num_experts, cfg.top_k
    c = cfg.to_c()
    st = lib().moe_dispatch(
        ctypes.byref(c), _ptr(ids, "ids", (T, k), torch.int32), _ptr(x, "x", (T, d), cfg.torch_dtype),
        _ptr(counts_pre, "counts_pre", (E,), torch.int32), _ptr(counts, "counts", (E,), torch.int32),
        _ptr(offsets, "offsets", (E + 1,), torch.int32), _ptr(perm_token, "perm_token", (T * k,), torch.int32),
        _ptr(row_of, "row_of", (T, k), torch.int32), _ptr(dropped, "dropped", (T, k), torch.uint8),
        _ptr(n_dropped, "n_dropped", (1,), torch.int32), _ptr(xp, "xp", (T * k, d), cfg.torch_dtype),
        _ptr(ws, "ws"), ws.numel(), _stream())
    _check("moe_dispatch", st)


def moe_expert_ffn(cfg: MoEConfig, xp, offsets, w1, w2, h, y, ws):
    T, d, f, E, k = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts, cfg.top_k
    c = cfg.to_c()
    dt = cfg.torch_dtype
    st = lib().moe_expert_ffn(
        ctypes.byref(c), _ptr(xp, "xp", (T * k, d), dt), _ptr(offsets, "offsets", (E + 1,), torch.int32),
        _wptr(cfg, w1, "w1", E * f, d, (E, f, d)), _wptr(cfg, w2, "w2", E * d, f, (E, d, f)),
        _ptr(h, "h", (T * k, f), dt),
        _ptr(y, "y", (T * k, d), dt), _ptr(ws, "ws"), ws.numel(), _stream())
    _check("moe_expert_ffn", st)


def moe_combine(cfg: MoEConfig, y, row_of, weights, out, *, y_shared=None):
    T, d, k = cfg.T, cfg.d_model, cfg.top_k
    c = cfg.to_c()
    dt = cfg.torch_dtype
    st = lib().moe_combine(ctypes.byref(c), _ptr(y, "y", (T * k, d), dt), _ptr(row_of, "row_of", (T, k), torch.int32),
                           _ptr(weights, "weights", (T, k), torch.float32), _ptr(y_shared, "y_shared", (T, d), dt),
                           _ptr(out, "out", (T, d), dt), _stream())
    _check("moe_combine", st)


def moe_aux_loss(cfg: MoEConfig, counts_pre, aux, ws, *, probs=None, logits=None, token_mask=None):
    T, E = cfg.T, cfg.num_experts
    c = cfg.to_c()
    st = lib().moe_aux_loss(ctypes.byref(c), _ptr(probs, "probs", (T, E), torch.float32),
                            _ptr(logits, "logits", (T, E), torch.float32),
                            _ptr(token_mask, "token_mask", (T,), torch.uint8),
                            _ptr(counts_pre, "counts_pre", (E,), torch.int32), _ptr(aux, "aux", (3,), torch.float32),
                            _ptr(ws, "ws"), ws.numel(), _stream())
    _check("moe_aux_loss", st)


def moe_forward(cfg: MoEConfig, x, w_router, w1, w2, out, aux, ws, *, bias=None, gumbel=None, token_mask=None,
                w1_shared=None, w2_shared=None, debug: Optional[dict] = None, events=None):
    """The whole layer. `debug` maps moe_debug_outputs field names to GPU tensors that receive
    those intermediates; `events` is a HipEvents object whose events are recorded between the
    kernels."""
    T, d, f, E, k = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts, cfg.top_k
    dt = cfg.torch_dtype
    c = cfg.to_c()
    dbg = None
    if debug or events is not None:
        dbg = _Debug()
        for name, t in (debug or {}).items():
            if name not in dict(_Debug._fields_) or name in ("events", "n_events"):
                raise ValueError(f"unknown debug output {name!r}")
            setattr(dbg, name, _ptr(t, name))
        if events is not None:
            dbg.events = ctypes.cast(events.array, ctypes.c_void_p)
            dbg.n_events = len(events)
    st = lib().moe_forward(
        ctypes.byref(c), _ptr(x, "x", (T, d), dt), _ptr(w_router, "w_router", (E, d), torch.float32),
        _ptr(bias, "bias", (E,), torch.float32), _ptr(gumbel, "gumbel", (T, E), torch.float32),
        _ptr(token_mask, "token_mask", (T,), torch.uint8),
        _wptr(cfg, w1, "w1", E * f, d, (E, f, d)), _wptr(cfg, w2, "w2", E * d, f, (E, d, f)),
        _ptr(w1_shared, "w1_shared", (cfg.d_ffn_shared, d), dt) if cfg.d_ffn_shared else None,
        _ptr(w2_shared, "w2_shared", (d, cfg.d_ffn_shared), dt) if cfg.d_ffn_shared else None,
        _ptr(out, "out", (T, d), dt),
        _ptr(aux, "aux", (3,), torch.float32), ctypes.byref(dbg) if dbg is not None else None,
        _ptr(ws, "ws"), ws.numel(), _stream())
    _check("moe_forward", st)


def forward_noalloc_max_bytes() -> int:
    return lib().moe_forward_noalloc_max_bytes()


def moe_forward_noalloc(cfg: MoEConfig, x, w_router, w1, w2, out, aux, *, bias=None, gumbel=None, token_mask=None,
                        w1_shared=None, w2_shared=None):
    """The whole layer with the library's own static workspace (moe_forward_noalloc): no
    workspace argument, nothing allocated by the call."""
    T, d, f, E = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts
    dt = cfg.torch_dtype
    c = cfg.to_c()
    st = lib().moe_forward_noalloc(
        ctypes.byref(c), _ptr(x, "x", (T, d), dt), _ptr(w_router, "w_router", (E, d), torch.float32),
        _ptr(bias, "bias", (E,), torch.float32), _ptr(gumbel, "gumbel", (T, E), torch.float32),
        _ptr(token_mask, "token_mask", (T,), torch.uint8),
        _wptr(cfg, w1, "w1", E * f, d, (E, f, d)), _wptr(cfg, w2, "w2", E * d, f, (E, d, f)),
        _ptr(w1_shared, "w1_shared", (cfg.d_ffn_shared, d), dt) if cfg.d_ffn_shared else None,
        _ptr(w2_shared, "w2_shared", (d, cfg.d_ffn_shared), dt) if cfg.d_ffn_shared else None,
        _ptr(out, "out", (T, d), dt), _ptr(aux, "aux", (3,), torch.float32), _stream())
    _check("moe_forward_noalloc", st)


# ------------------------------------------------------------------------------ backward pass

def backward_workspace_bytes(cfg: MoEConfig) -> int:
    c = cfg.to_c()
    return lib().moe_backward_workspace_bytes(ctypes.byref(c))


def new_backward_workspace(cfg: MoEConfig, device="cuda") -> torch.Tensor:
    n = backward_workspace_bytes(cfg)
    if n == 0:
        raise MoEError("moe_backward_workspace_bytes", validate_config(cfg))
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_combine_backward(cfg: MoEConfig, d_out, y, row_of, weights, dy, dweights):
    T, d, k = cfg.T, cfg.d_model, cfg.top_k
    c = cfg.to_c()
    dt = cfg.torch_dtype
    st = lib().moe_combine_backward(
        ctypes.byref(c), _ptr(d_out, "d_out", (T, d), dt), _ptr(y, "y", (T * k, d), dt),
        _ptr(row_of, "row_of", (T, k), torch.int32), _ptr(weights, "weights", (T, k), torch.float32),
        _ptr(dy, "dy", (T * k, d), dt), _ptr(dweights, "dweights", (T, k), torch.float32), _stream())
    _check("moe_combine_backward", st)


def moe_expert_ffn_backward(cfg: MoEConfig, xp, offsets, w1, w2, dy, dxp, ws, *, h=None, dw1=None, dw2=None):
    T, d, f, E, k = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts, cfg.top_k
    c = cfg.to_c()
    dt = cfg.torch_dtype
    st = lib().moe_expert_ffn_backward(
        ctypes.byref(c), _ptr(xp, "xp", (T * k, d), dt), _ptr(offsets, "offsets", (E + 1,), torch.int32),
        _ptr(w1, "w1", (E, f, d), dt), _ptr(w2, "w2", (E, d, f), dt), _ptr(h, "h", (T * k, f), dt),
        _ptr(dy, "dy", (T * k, d), dt), _ptr(dxp, "dxp", (T * k, d), dt),
        _ptr(dw1, "dw1", (E, f, d), torch.float32), _ptr(dw2, "dw2", (E, d, f), torch.float32),
        _ptr(ws, "ws"), ws.numel(), _stream())
    _check("moe_expert_ffn_backward", st)


def moe_dispatch_backward(cfg: MoEConfig, dxp, row_of, dx):
    T, d, k = cfg.T, cfg.d_model, cfg.top_k
    c = cfg.to_c()
    dt = cfg.torch_dtype
    st = lib().moe_dispatch_backward(ctypes.byref(c), _ptr(dxp, "dxp", (T * k, d), dt),
                                     _ptr(row_of, "row_of", (T, k), torch.int32), _ptr(dx, "dx", (T, d), dt),
                                     _stream())
    _check("moe_dispatch_backward", st)


def moe_route_backward(cfg: MoEConfig, logits, ids, weights, dweights, dlogits, *, x=None, w_router=None,
                       counts_pre=None, token_mask=None, d_aux: float = 0.0, dx=None, dw_router=None, dbias=None,
                       ws=None):
    T, d, E, k = cfg.T, cfg.d_model, cfg.num_experts, cfg.top_k
    c = cfg.to_c()
    dt = cfg.torch_dtype
    f32 = torch.float32
    st = lib().moe_route_backward(
        ctypes.byref(c), _ptr(x, "x", (T, d), dt), _ptr(w_router, "w_router", (E, d), f32),
        _ptr(logits, "logits", (T, E), f32), _ptr(ids, "ids", (T, k), torch.int32),
        _ptr(weights, "weights", (T, k), f32), _ptr(dweights, "dweights", (T, k), f32),
        _ptr(counts_pre, "counts_pre", (E,), torch.int32), _ptr(token_mask, "token_mask", (T,), torch.uint8),
        float(d_aux), _ptr(dlogits, "dlogits", (T, E), f32), _ptr(dx, "dx", (T, d), dt),
        _ptr(dw_router, "dw_router", (E, d), f32), _ptr(dbias, "dbias", (E,), f32), _ptr(ws, "ws"),
        0 if ws is None else ws.numel(), _stream())
    _check("moe_route_backward", st)


def moe_backward(cfg: MoEConfig, x, w_router, w1, w2, d_out, fwd_ws, dx, ws, *, token_mask=None, w1_shared=None,
                 w2_shared=None, d_aux: float = 0.0, dw_router=None, dbias=None, dw1=None, dw2=None,
                 dw1_shared=None, dw2_shared=None):
    """The layer's backward from the intermediates moe_forward left in `fwd_ws`."""
    T, d, f, E = cfg.T, cfg.d_model, cfg.d_ffn, cfg.num_experts
    fs = cfg.d_ffn_shared
    dt = cfg.torch_dtype
    f32 = torch.float32
    c = cfg.to_c()
    st = lib().moe_backward(
        ctypes.byref(c), _ptr(x, "x", (T, d), dt), _ptr(w_router, "w_router", (E, d), f32),
        _ptr(token_mask, "token_mask", (T,), torch.uint8), _ptr(w1, "w1", (E, f, d), dt),
        _ptr(w2, "w2", (E, d, f), dt), _ptr(w1_shared, "w1_shared", (fs, d), dt) if fs else None,
        _ptr(w2_shared, "w2_shared", (d, fs), dt) if fs else None, _ptr(d_out, "d_out", (T, d), dt),
        float(d_aux), _ptr(fwd_ws, "fwd_ws"), fwd_ws.numel(), _ptr(dx, "dx", (T, d), dt),
        _ptr(dw_router, "dw_router", (E, d), f32), _ptr(dbias, "dbias", (E,), f32),
        _ptr(dw1, "dw1", (E, f, d), f32), _ptr(dw2, "dw2", (E, d, f), f32),
        _ptr(dw1_shared, "dw1_shared", (fs, d), f32) if fs else None,
        _ptr(dw2_shared, "dw2_shared", (d, fs), f32) if fs else None,
        _ptr(ws, "ws"), ws.numel(), _stream())
    _check("moe_backward", st)


# ------------------------------------------------------------------------------ HIP events

class HipEvents:
    """A fixed array of hipEvent_t created through the HIP runtime (for per-kernel timing on
    the stream the library launches on)."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.array = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.array[i] = ev
        self.n = n

    def __len__(self):
        return self.n

    def record(self, i: int):
        if self._hip.hipEventRecord(self.array[i], ctypes.c_void_p(_stream())) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        self._hip.hipEventSynchronize(self.array[j])
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.array[i], self.array[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(self.n):
            if self.array[i]:
                self._hip.hipEventDestroy(self.array[i])
                self.array[i] = None
