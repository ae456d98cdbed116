"""Plain CPU oracle for the forward pass of a top-k routed MoE FFN layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this module: only
the tests, the smoke check and the CPU-baseline leg of the benchmark use it. It shares no
code with the HIP library; both receive the same seeded inputs and nothing else.

Pages cited (by title):
  [P2] "Twinkle首发适配Deepseek-V4系列模型高效训练" (www.wmrh.cn/news/44033)
  [P3] "DeepSpeed ZeRO-3与MoE显存精算实战指南" (m.nlpx.cn/news/237350)
  [P4] "手搓一个LLaMA4-MoE" (www.nxmr.cn/news/140631)

Arithmetic: every dot product and sum is done in float64 (numpy; matrix products use the BLAS
dgemm as a primitive) and rounded once at the storage points the layer defines: router
logits to fp32; H, Y and the output to the storage dtype (bf16 round-to-nearest-even or fp32);
gate weights to fp32. The selection key is formed in fp32 exactly as the layer does (an fp32
add, then an fp32 divide), because it decides an integer (the chosen experts).

Readings where the pages are silent or disagree (each is listed with its reason in the design
notes): select on the key, lowest expert index wins ties, -0.0 ties +0.0; weights are the
softmax restricted to the selected logits; Gumbel noise changes selection only, additive router
noise (the other noise mode) changes the logits themselves; padding tokens are not routed and
are left out of the statistics; capacity keeps the
first C assignments of an expert in (token, slot) order; a dropped slot contributes zero;
aux losses use pre-drop counts.

Every function is pinned by the CPU tests in tests/test_oracle_pins.py (brute force, closed
forms, invariants, a hand-worked example, and finite differences for the backward pass).
forward_rows, the token-by-token output used to check sampled tokens, is pinned to forward()'s
output bit for bit on layers with capacity drops, fully dropped tokens, padding, both noise
modes, a shared expert and the straight-through estimator, and planted mistakes in a copy of it
(a skipped drop check, an unrounded term, a lost gate weight, a wrong expert) fail that pin.
There is no "parity unpinned" function.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


# ---------------------------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------------------------

def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and the fp32 exponent range; the quantum of a value with
    binary exponent e (a = m * 2**e, 0.5 <= |m| < 1) is 2**(e - 8), floored at the subnormal
    quantum 2**-133; np.rint rounds half to even.
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    q_exp = np.maximum(e, -125) - 8
    return np.ldexp(np.rint(np.ldexp(a, -q_exp)), q_exp)


def round_storage(a, storage: str) -> np.ndarray:
    """Round float64 values to the storage dtype ("bf16" or "f32"); float64 result. "f64" keeps
    them (the exact layer, used to check the backward pass by finite differences)."""
    if storage == "f64":
        return np.asarray(a, dtype=np.float64)
    if storage == "bf16":
        return round_bf16(a)
    if storage == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {storage!r}")


def _f64(a) -> np.ndarray:
    """Exact widening of fp32 / bf16 (given as float32) data to float64."""
    if hasattr(a, "detach"):          # a torch tensor: bf16 -> fp32 is exact
        a = a.detach().float().cpu().numpy()
    return np.asarray(a, dtype=np.float64)


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().float().cpu().numpy()
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------------------------
# routing  ([P2 §3.1], [P4 §1.3, §2.4])
# ---------------------------------------------------------------------------------------------

def router_logits(x, w_router, bias=None, exact: bool = False) -> np.ndarray:
    """logits[t, e] = sum_c x[t, c] * W_r[e, c] + b[e], exact in float64, rounded once to fp32
    (kept in float64 with exact=True).

    P4 §2.4: the router is a linear layer producing one score per expert; P2 §3.1 writes
    scores = W_router x. The per-expert bias is the workload's load-skew term.
    """
    l = _f64(x) @ _f64(w_router).T
    if bias is not None:
        l = l + _f64(bias)[None, :]
    return l if exact else l.astype(np.float32)


def selection_keys(logits, gumbel=None, tau: float = 1.0) -> np.ndarray:
    """fp32 key that top-k ranks: the logits, or (logits + g) / tau with Gumbel noise g.

    P2 §3.1 forms the noisy logits as (logits + gumbel) / temperature and ranks them with top-k.
    Computed in fp32: one rounded add, then one rounded divide by tau (tau itself held in fp32).
    """
    l = _f32(logits)
    if gumbel is None:
        return l.copy()
    s = np.add(l, _f32(gumbel), dtype=np.float32)
    return np.divide(s, np.float32(tau), dtype=np.float32)


def top_k(keys, k: int) -> np.ndarray:
    """ids[t, :] = the k largest keys of row t, in descending order, lowest index on ties.

    P2 §3.1 and P4 §1.3: each token goes to the k experts with the highest scores. Done as k
    rounds of "take the largest key not taken yet"; np.argmax returns the first maximum, so the
    lowest expert index wins a tie, and -0.0 compares equal to +0.0.
    """
    kf = _f64(keys)
    if not np.all(np.isfinite(kf)):
        raise ValueError("oracle top_k: keys must be finite")
    T, E = kf.shape
    if not 1 <= k <= E:
        raise ValueError("oracle top_k: need 1 <= k <= E")
    work = kf.copy()
    ids = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        pick = np.argmax(work, axis=1)
        ids[:, j] = pick
        work[rows, pick] = -np.inf
    return ids


def router_probs(logits, tau: float = 1.0) -> np.ndarray:
    """probs[t, :] = softmax(logits[t, :] / tau) over all experts, float64 (clean logits).

    P2 §3.1 (probs = softmax(scores / temperature)); P4 §3.2 averages these per expert for the
    auxiliary loss.
    """
    s = _f64(logits) / float(np.float32(tau))
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def gate_weights(logits, ids, tau: float = 1.0, renormalize: bool = True, exact: bool = False,
                 straight_through: bool = False) -> np.ndarray:
    """Gate weight of each selected expert, fp32.

    P4 §2.4: the output is the weighted sum of the chosen experts' outputs, weighted by the
    softmax router scores. renormalize=True: softmax over the k selected (clean) logits / tau,
    so a token's weights sum to 1. renormalize=False: the full-softmax probability of each
    selected expert (the page's literal wording). straight_through=True (P2 §3.1's
    straight-through estimator): the routing matrix is the k-hot selection plus
    softmax - detach(softmax), whose value is the k-hot matrix, so every selected expert has
    weight exactly 1 (the softmax only shapes the backward pass).
    """
    ids = np.asarray(ids)
    if straight_through:
        return np.ones(ids.shape, dtype=np.float64 if exact else np.float32)
    if renormalize:
        s = _f64(logits) / float(np.float32(tau))
        sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
        sel = sel - sel.max(axis=1, keepdims=True)
        e = np.exp(sel)
        w = e / e.sum(axis=1, keepdims=True)
    else:
        p = router_probs(logits, tau)
        w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return w if exact else w.astype(np.float32)


def topk_gap(keys, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest key of each row (fp32 keys); +inf when k == E."""
    kf = np.sort(_f64(keys), axis=1)[:, ::-1]
    if k >= kf.shape[1]:
        return np.full(kf.shape[0], np.inf)
    return kf[:, k - 1] - kf[:, k]


def router_entropy(probs) -> np.ndarray:
    """Per-token entropy of the router distribution, -sum_e p_e ln p_e (natural log; 0 ln 0 = 0).

    P4 §3.3 monitors the router entropy next to the expert selection counts and the balance
    loss: an entropy far below its maximum ln E means the routing has become deterministic.
    """
    p = np.asarray(probs, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0.0, p * np.log(np.where(p > 0.0, p, 1.0)), 0.0)
    return -t.sum(axis=1)


@dataclasses.dataclass
class Routing:
    logits: np.ndarray      # [T, E] fp32 (with additive router noise when that mode is on)
    keys: np.ndarray        # [T, E] fp32
    ids: np.ndarray         # [T, k] int32 (-1 for padding tokens)
    weights: np.ndarray     # [T, k] fp32 (0 for padding tokens)
    probs: np.ndarray       # [T, E] float64 (0 rows for padding tokens)
    real: np.ndarray        # [T] bool: token takes part in routing (not padding)
    entropy: np.ndarray     # [T] float64 router entropy (0 for padding tokens)


def route(x=None, w_router=None, bias=None, gumbel=None, tau: float = 1.0, k: int = 2,
          renormalize: bool = True, logits=None, noise_in_logits: bool = False,
          token_mask=None, exact: bool = False, straight_through: bool = False) -> Routing:
    """Router logits -> key -> top-k -> gate weights, plus the full softmax for the aux loss.

    With `logits` given, routing runs on those fp32 logits (the bias, and additive noise when
    noise_in_logits is on, are taken as already in them) instead of computing x W_r^T + b.

    The noise input [T, E] enters in one of two ways. noise_in_logits=False (P2 §3.1, Gumbel
    top-k): it perturbs the selection key only, (logits + g) / tau. noise_in_logits=True (P4
    §3.2: Gaussian noise added to the router logits early in training, then annealed to zero;
    the caller passes the already scaled noise): logits = fp32(logits + n), and everything
    downstream (key, weights, probabilities, aux and entropy) uses the noisy logits.

    token_mask [T] (nonzero = real token; P4 §4.1: padding tokens take no part in expert
    selection): a padding token gets ids -1 and weights 0 in every slot, and is left out of the
    probabilities, the entropy and the aux statistics. Its logits are still computed.

    exact=True keeps logits, keys and weights in float64 (the exact layer of the finite-difference
    checks of the backward pass).
    """
    if exact:
        logits = router_logits(x, w_router, bias, exact=True) if logits is None else _f64(logits)
        if noise_in_logits and gumbel is not None:
            logits = logits + _f64(gumbel)
        keys = logits if (gumbel is None or noise_in_logits) else (logits + _f64(gumbel)) / float(tau)
    else:
        if logits is None:
            logits = router_logits(x, w_router, bias)
            if noise_in_logits and gumbel is not None:
                logits = np.add(_f32(logits), _f32(gumbel), dtype=np.float32)
        logits = _f32(logits)
        keys = selection_keys(logits, None if noise_in_logits else gumbel, tau)
    T, E = logits.shape
    real = np.ones(T, dtype=bool) if token_mask is None else (np.asarray(token_mask) != 0)
    ids = np.full((T, k), -1, dtype=np.int32)
    weights = np.zeros((T, k), dtype=np.float64 if exact else np.float32)
    probs = np.zeros((T, E), dtype=np.float64)
    entropy = np.zeros(T, dtype=np.float64)
    if np.any(real):
        ids[real] = top_k(keys[real], k)
        weights[real] = gate_weights(logits[real], ids[real], tau, renormalize, exact, straight_through)
        probs[real] = router_probs(logits[real], tau)
        entropy[real] = router_entropy(probs[real])
    return Routing(logits, keys, ids, weights, probs, real, entropy)


# ---------------------------------------------------------------------------------------------
# capacity and dispatch  ([P3 §3.1, §3.4, §5.1], [P4 §2.4])
# ---------------------------------------------------------------------------------------------

def capacity_from_factor(T: int, k: int, E: int, factor: Optional[tuple]) -> int:
    """Per-expert capacity C = ceil(cf * T * k / E), exact in integers for cf = num / den.

    P3 gives capacity factors (1.2 in its MoE config, "default 1.0, use 1.2 to 1.5") and an
    absolute per-expert cap flag, but no formula; this is the plain reading. No limit -> C = T.
    """
    if factor is None:
        return T
    num, den = factor
    return -((-num * T * k) // (den * E))


@dataclasses.dataclass
class Dispatch:
    counts_pre: np.ndarray  # [E] int32: assignments per expert before the capacity cut
    counts: np.ndarray      # [E] int32: kept assignments per expert
    offsets: np.ndarray     # [E+1] int32: exclusive scan of counts
    perm_token: np.ndarray  # [N] int32: token of each permuted row
    row_of: np.ndarray      # [T, k] int32: permuted row of each kept slot, -1 if dropped
    dropped: np.ndarray     # [T, k] uint8
    n_dropped: int
    xp: Optional[np.ndarray]  # [N, d] gathered rows (same dtype as x), or None


def dispatch(ids, num_experts: int, capacity: int, x=None) -> Dispatch:
    """Counting sort of the (token, slot) assignments by expert, in token order, with capacity.

    P4 §2.4: sort the [B, K] index by expert id, count tokens per expert, split into
    per-expert segments and gather the tokens with a table lookup. P3: at most `capacity`
    assignments per expert are kept; the rest are dropped. Kept assignments of expert e fill
    rows offsets[e] .. offsets[e] + counts[e] - 1 in token order. An id of -1 (a padding token's
    slot) is skipped: it is neither counted, kept nor dropped.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    E = num_experts
    counts_pre = np.zeros(E, dtype=np.int64)
    pos = np.full((T, k), -1, dtype=np.int64)
    dropped = np.zeros((T, k), dtype=np.uint8)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e == -1:
                continue
            if not 0 <= e < E:
                raise ValueError("oracle dispatch: expert id out of range")
            if counts_pre[e] < capacity:
                pos[t, j] = counts_pre[e]
            else:
                dropped[t, j] = 1
            counts_pre[e] += 1
    counts = np.minimum(counts_pre, max(capacity, 0))
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    N = int(offsets[-1])
    row_of = np.full((T, k), -1, dtype=np.int64)
    perm_token = np.full(N, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if pos[t, j] >= 0:
                row = offsets[ids[t, j]] + pos[t, j]
                row_of[t, j] = row
                perm_token[row] = t
    xp = None
    if x is not None:
        if hasattr(x, "detach"):      # torch tensor: keep its dtype (a bitwise row copy)
            import torch
            xp = x.detach().cpu()[torch.from_numpy(perm_token.astype(np.int64))]
        else:
            xp = np.asarray(x)[perm_token]
    return Dispatch(counts_pre.astype(np.int32), counts.astype(np.int32), offsets.astype(np.int32),
                    perm_token.astype(np.int32), row_of.astype(np.int32), dropped,
                    int(dropped.sum()), xp)


# ---------------------------------------------------------------------------------------------
# 4-bit expert weights  ([P4 §5.2])
# ---------------------------------------------------------------------------------------------

Q4_GROUP = 64


def quantize_int4(w):
    """Symmetric group-wise int4 codes of bf16 weights w [..., K] (K a multiple of 64).

    P4 §5.2 proposes 4-bit expert weights. Per group of 64 consecutive in-features: the scale is
    s = bf16(fp32(amax / 7)) (an fp32 divide, then one round-to-nearest-even to bf16); the codes
    are q = clamp(rint(fp32(w / s)), -8, 7), ties to even, and 0 where s = 0. Returns (codes as
    int8 [..., K], scales as float64 [..., K / 64] holding bf16 values).
    """
    w32 = _f32(w)
    K = w32.shape[-1]
    if K % Q4_GROUP:
        raise ValueError("oracle quantize_int4: K must be a multiple of 64")
    g = w32.reshape(*w32.shape[:-1], K // Q4_GROUP, Q4_GROUP)
    amax = np.abs(g).max(axis=-1)
    s = round_bf16(np.divide(amax, np.float32(7.0), dtype=np.float32).astype(np.float64))
    s32 = s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s32 > 0, np.divide(g, np.where(s32 > 0, s32, np.float32(1.0)), dtype=np.float32), 0)
    q = np.clip(np.rint(r.astype(np.float64)), -8, 7).astype(np.int8)
    return q.reshape(w32.shape), s


def dequantize_int4(codes, scales) -> np.ndarray:
    """w' = bf16(q * s) per element (q * s is exact in float64), float64 result."""
    q = np.asarray(codes, dtype=np.float64)
    K = q.shape[-1]
    s = np.repeat(np.asarray(scales, dtype=np.float64), Q4_GROUP, axis=-1)
    assert s.shape[-1] == K
    return round_bf16(q * s)


def pack_int4(codes, scales) -> np.ndarray:
    """The packed byte layout of a 4-bit weight [rows, K] (rows a multiple of 16, K of 128), tiled
    so that one 1 KiB block holds 16 rows x 128 columns in the order the GEMM's lanes read them.

    Codes: block (t, s) of rows 16 t .. 16 t + 15 and columns 128 s .. 128 s + 127 sits at byte
    1024 (t K/128 + s); inside it, the 16 bytes at 16 (16 g + r) hold row 16 t + r, columns
    128 s + 32 g .. + 31, two per byte (low nibble = even column, two's complement nibbles).
    Scales (bf16, little-endian) follow from the next 256-byte boundary (zero bytes between):
    block (t, s) holds 32 scales at 64 (t K/128 + s) bytes, row r's two groups at 2 r and 2 r + 1.
    Used to build inputs for the library's 4-bit path and to check its quantiser.
    """
    q = np.asarray(codes, dtype=np.int8)
    rows, K = q.shape
    if rows % 16 or K % 128:
        raise ValueError("oracle pack_int4: rows must be a multiple of 16 and K of 128")
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    nib = nib.reshape(rows // 16, 16, K // 128, 4, 32).transpose(0, 2, 3, 1, 4)   # [t, s, g, r, j]
    code_bytes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8).reshape(-1)
    sc = np.asarray(scales, dtype=np.float64).astype(np.float32)
    sc = sc.reshape(rows // 16, 16, K // 128, 2).transpose(0, 2, 1, 3).reshape(-1)   # [t, s, r, h]
    bits = (np.ascontiguousarray(sc).view(np.uint32) >> 16).astype(np.uint16)
    off = (code_bytes.size + 255) // 256 * 256
    out = np.zeros(off + 2 * bits.size, dtype=np.uint8)
    out[:code_bytes.size] = code_bytes
    out[off:] = bits.view(np.uint8)
    return out


# ---------------------------------------------------------------------------------------------
# experts and combine  ([P4 §2.4])
# ---------------------------------------------------------------------------------------------

def silu(a) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a)), float64 (in place on a temporary)."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        if a.ndim == 0:
            return np.float64(a / (1.0 + np.exp(-a)))
        den = np.negative(a)
        np.exp(den, out=den)
    den += 1.0
    return np.divide(a, den, out=den)


def expert_ffn(xp, offsets, w1, w2, storage: str):
    """Per-expert two-layer FFN over the permuted rows: Y_e = W2_e SiLU(W1_e x).

    P4 §2.4: each expert is a two-layer FFN like a standard Transformer FFN. W1 is [E, f, d]
    and W2 is [E, d, f] (out-features by in-features). H = SiLU(Xp_e W1_e^T) is rounded to the
    storage dtype, then Y_e = H_e W2_e^T is rounded to the storage dtype. Returns float64
    arrays (H [N, f], Y [N, d]) holding storage-representable values.
    """
    xp = _f64(xp)
    w1 = _f64(w1)
    w2 = _f64(w2)
    E, f, d = w1.shape
    N = xp.shape[0]
    h = np.zeros((N, f), dtype=np.float64)
    y = np.zeros((N, d), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        h[r0:r1] = round_storage(silu(xp[r0:r1] @ w1[e].T), storage)
        y[r0:r1] = round_storage(h[r0:r1] @ w2[e].T, storage)
    return h, y


def shared_ffn(x, w1s, w2s, storage: str):
    """The shared expert on every token: Hs = SiLU(x W1s^T), Ys = Hs W2s^T.

    P4 §5.2: shared experts are fixed experts that join every token's computation. They are
    FFNs of the same two-layer form as the routed experts (W1s [fs, d], W2s [d, fs]); several
    shared experts of width f are one of width n f. Hs and Ys are rounded to the storage dtype
    like H and Y. Returns float64 arrays (Hs [T, fs], Ys [T, d]).
    """
    hs = round_storage(silu(_f64(x) @ _f64(w1s).T), storage)
    ys = round_storage(hs @ _f64(w2s).T, storage)
    return hs, ys


def combine(y, row_of, weights, storage: str, d: Optional[int] = None, y_shared=None) -> np.ndarray:
    """out[t] = sum over kept slots j (ascending) of w[t, j] * Y[row_of[t, j]] (+ Ys[t]), rounded once.

    P4 §2.4: each token's output is the weighted sum of its chosen experts' outputs. A dropped
    slot adds nothing and the remaining weights are not rescaled; a token whose slots are all
    dropped gets zeros. P4 §5.2: a shared expert's output Ys[t] joins every token's output, with
    no gate weight.
    """
    y = _f64(y)
    row_of = np.asarray(row_of)
    w = _f64(weights)
    T, k = row_of.shape
    d = y.shape[1] if d is None else d
    out = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        kept = row_of[:, j] >= 0
        if np.any(kept):
            out[kept] += w[kept, j][:, None] * y[row_of[kept, j]]
    if y_shared is not None:
        out += _f64(y_shared)
    return round_storage(out, storage)


# ---------------------------------------------------------------------------------------------
# auxiliary load-balance losses  ([P4 §3.2], [P3 §3.2])
# ---------------------------------------------------------------------------------------------

def aux_loss(probs, counts_pre, k: int, coef: float, real=None, entropy=None):
    """(aux_switch, aux_balance, mean router entropy), float64, over the n real tokens.

    aux_switch (P4 §3.2): coef * E * sum_i f_i * P_i with f_i = counts_pre[i] / (n k), the
    fraction of routed assignments that chose expert i, and P_i the mean router probability of
    expert i over the tokens. Uniform routing gives coef * sum_i P_i = coef.
    aux_balance (P3 §3.2): coef * sum_i (p_i - k/E)^2 with p_i = counts_pre[i] / n, the
    per-token probability that expert i is selected; its uniform value is k/E, so it is zero
    for perfectly uniform routing.
    The entropy term is the mean over real tokens of the per-token router entropy (P4 §3.3).
    Padding tokens (real == False) are left out of n, P_i and the entropy; with no real token
    all three values are 0.
    """
    probs = np.asarray(probs, dtype=np.float64)
    T, E = probs.shape
    real = np.ones(T, dtype=bool) if real is None else np.asarray(real, dtype=bool)
    n = int(real.sum())
    if n == 0:
        return 0.0, 0.0, 0.0
    cp = np.asarray(counts_pre, dtype=np.float64)
    P = probs[real].sum(axis=0) / n
    f = cp / (n * k)
    aux_switch = coef * E * float(np.sum(f * P))
    aux_balance = coef * float(np.sum((cp / n - k / E) ** 2))
    ent = router_entropy(probs[real]) if entropy is None else np.asarray(entropy, dtype=np.float64)[real]
    return aux_switch, aux_balance, float(ent.sum() / n)


# ---------------------------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------------------------

@dataclasses.dataclass
class Forward:
    routing: Routing
    dispatch: Dispatch
    capacity: int
    h: np.ndarray
    y: np.ndarray
    out: np.ndarray
    aux: tuple
    y_shared: Optional[np.ndarray] = None


def forward(x, w_router, w1, w2, *, k: int, storage: str, bias=None, gumbel=None,
            tau: float = 1.0, capacity: Optional[int] = None, renormalize: bool = True,
            aux_coef: float = 0.01, logits=None, noise_in_logits: bool = False,
            token_mask=None, w1_shared=None, w2_shared=None, exact: bool = False,
            straight_through: bool = False) -> Forward:
    """Router -> top-k -> capacity + dispatch -> expert FFN -> weighted combine, plus aux.

    aux = (aux_switch, aux_balance, mean router entropy). With w1_shared / w2_shared, a shared
    expert runs on every token (padding included: it involves no selection) and its output is
    added in the combine."""
    T = x.shape[0]
    E = w1.shape[0]
    C = T if capacity is None or capacity < 0 else capacity
    r = route(x, w_router, bias, gumbel, tau, k, renormalize, logits, noise_in_logits, token_mask, exact,
              straight_through=straight_through)
    dp = dispatch(r.ids, E, C, x)
    h, y = expert_ffn(dp.xp, dp.offsets, w1, w2, storage)
    ys = None
    if w1_shared is not None:
        _, ys = shared_ffn(x, w1_shared, w2_shared, storage)
    out = combine(y, dp.row_of, r.weights, storage, d=x.shape[1], y_shared=ys)
    aux = aux_loss(r.probs, dp.counts_pre, k, aux_coef, r.real, r.entropy)
    return Forward(r, dp, C, h, y, out, aux, ys)


def forward_rows(x, w1, w2, ids, weights, dropped, token_idx, storage: str, w1_shared=None,
                 w2_shared=None) -> np.ndarray:
    """Output rows of selected tokens only, straight from the layer's definition.

    out[t] = sum over kept j of w[t, j] * W2_e SiLU(W1_e x_t) (+ W2s SiLU(W1s x_t)) with the
    storage roundings of H and Y; used to check sampled tokens at full size without running
    the whole oracle.
    """
    ids = np.asarray(ids)
    w = _f64(weights)
    dropped = np.asarray(dropped)
    expert_cache = {}

    def expert(e):
        if e not in expert_cache:
            expert_cache[e] = (_f64(w1[e]), _f64(w2[e]))
        return expert_cache[e]

    rows = []
    for t in token_idx:
        xt = _f64(x[t])
        acc = np.zeros(xt.shape[0], dtype=np.float64)
        for j in range(ids.shape[1]):
            if dropped[t, j] or ids[t, j] < 0:
                continue
            e = int(ids[t, j])
            w1e, w2e = expert(e)
            h = round_storage(silu(w1e @ xt), storage)
            y = round_storage(w2e @ h, storage)
            acc += w[t, j] * y
        if w1_shared is not None:
            hs = round_storage(silu(_f64(w1_shared) @ xt), storage)
            acc += round_storage(_f64(w2_shared) @ hs, storage)
        rows.append(round_storage(acc, storage))
    return np.stack(rows) if rows else np.zeros((0, x.shape[1]))


# ---------------------------------------------------------------------------------------------
# backward pass  ([P4 §2.4, §3.2; P2 §3.1])
# ---------------------------------------------------------------------------------------------

def silu_grad(a) -> np.ndarray:
    """d SiLU(a) / da = sigmoid(a) (1 + a (1 - sigmoid(a))), float64."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-a))
    return sg * (1.0 + a * (1.0 - sg))


def combine_backward(d_out, y, row_of, weights, storage: str):
    """The combine's backward: dY[row_of[t, j]] = w[t, j] dOut[t] (rounded to the storage dtype)
    and dw[t, j] = <dOut[t], Y[row_of[t, j]]> (float64; 0 for a slot without a row)."""
    go, y, w = _f64(d_out), _f64(y), _f64(weights)
    row_of = np.asarray(row_of)
    T, k = row_of.shape
    dy = np.zeros((y.shape[0], go.shape[1]), dtype=np.float64)
    dw = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        kept = row_of[:, j] >= 0
        dy[row_of[kept, j]] = w[kept, j][:, None] * go[kept]
        dw[kept, j] = np.sum(go[kept] * y[row_of[kept, j]], axis=1)
    return round_storage(dy, storage), dw


def expert_ffn_backward(xp, offsets, w1, w2, h, dy, storage: str):
    """The expert FFNs' backward over each expert's rows: with A = Xp W1_e^T (recomputed),
    dA = (dY W2_e) * SiLU'(A), dXp = dA W1_e (rounded to the storage dtype), dW2_e = dY^T H,
    dW1_e = dA^T Xp (float64)."""
    xp, w1, w2, h, dy = _f64(xp), _f64(w1), _f64(w2), _f64(h), _f64(dy)
    E = w1.shape[0]
    N = int(offsets[-1])
    dxp = np.zeros((N, xp.shape[1]), dtype=np.float64)
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        a1 = xp[r0:r1] @ w1[e].T
        dw2[e] = dy[r0:r1].T @ h[r0:r1]
        da = (dy[r0:r1] @ w2[e]) * silu_grad(a1)
        dw1[e] = da.T @ xp[r0:r1]
        dxp[r0:r1] = da @ w1[e]
    return round_storage(dxp, storage), dw1, dw2


def dispatch_backward(dxp, row_of, T: int, storage: str):
    """The gather's backward: dx[t] = sum over the token's kept slots of dXp[row_of[t, j]], in slot
    order, rounded once to the storage dtype."""
    dxp = _f64(dxp)
    row_of = np.asarray(row_of)
    dx = np.zeros((T, dxp.shape[1]), dtype=np.float64)
    for j in range(row_of.shape[1]):
        kept = row_of[:, j] >= 0
        dx[kept] += dxp[row_of[kept, j]]
    return round_storage(dx, storage)


@dataclasses.dataclass
class Grads:
    dx: np.ndarray          # [T, d]
    dw_router: np.ndarray   # [E, d]
    dbias: np.ndarray       # [E]
    dw1: np.ndarray         # [E, f, d]
    dw2: np.ndarray         # [E, d, f]
    dlogits: np.ndarray     # [T, E]
    dweights: np.ndarray    # [T, k] gradient of the gate weights (0 for dropped and padding slots)
    dw1_shared: Optional[np.ndarray] = None
    dw2_shared: Optional[np.ndarray] = None


def backward(fw: Forward, x, w_router, w1, w2, d_out, *, storage: str, tau: float = 1.0,
             renormalize: bool = True, aux_coef: float = 0.01, d_aux: float = 1.0, w1_shared=None,
             w2_shared=None, straight_through: bool = False) -> Grads:
    """Gradients of  L = sum(d_out * out) + d_aux * aux_switch  with respect to x, the router
    weight and bias, the expert weights and the shared expert's weights, float64.

    P4 §2.4 trains the layer end to end: the output is the gate-weighted sum of the chosen
    experts' FFN outputs, so the gradient reaches the experts through their outputs and the
    router through the gate weights (the selection itself, the capacity cut and the noise are
    piecewise constant: they pass no gradient). P4 §3.2 adds aux_switch = coef E sum_i f_i P_i
    to the loss: f_i (counts) is constant, P_i is the mean router probability, so the aux term
    reaches the router through the probabilities (aux_balance depends on counts only).
    The forward's stored values are used as they are (H, Y after their storage rounding; the
    shared expert's Hs is recomputed with the same rounding); the pre-activations W1 Xp and
    W1s x are recomputed in float64.
    straight_through (P2 §3.1): the forward's weights are the k-hot selection (all 1) and the
    gradient goes through the full softmax of logits / tau, as for full-softmax weights: the
    derivative of softmax - detach(softmax) is the softmax's. A non-selected (or dropped) expert
    gets no gradient: its output is not computed for the token (P2 §3.2 runs each expert on its
    own tokens only).
    """
    r, dp = fw.routing, fw.dispatch
    x64, wr64 = _f64(x), _f64(w_router)
    w1_64, w2_64 = _f64(w1), _f64(w2)
    go = _f64(d_out)
    T, d = x64.shape
    E, f, _ = w1_64.shape
    k = r.ids.shape[1]
    w = _f64(r.weights)
    y = _f64(fw.y)
    h = _f64(fw.h)
    row_of = np.asarray(dp.row_of)
    dy, dwts = combine_backward(go, y, row_of, w, "f64")
    perm = np.asarray(dp.perm_token).astype(np.int64)
    dxp, dw1, dw2 = expert_ffn_backward(x64[perm], dp.offsets, w1_64, w2_64, h, dy, "f64")
    dx = dispatch_backward(dxp, row_of, T, "f64")
    # shared expert: its output joins every token's with weight 1
    dw1s = dw2s = None
    if w1_shared is not None:
        w1s, w2s = _f64(w1_shared), _f64(w2_shared)
        a_s = x64 @ w1s.T
        hs = round_storage(silu(a_s), storage)
        dw2s = go.T @ hs
        das = (go @ w2s) * silu_grad(a_s)
        dw1s = das.T @ x64
        dx += das @ w1s
    dl = router_backward(r.probs, r.ids, w, r.real, dwts, dp.counts_pre, tau=tau,
                         renormalize=renormalize and not straight_through, aux_coef=aux_coef, d_aux=d_aux)
    dwr, db, dx_r = router_input_grads(dl, x64, wr64)
    dx += dx_r
    return Grads(dx, dwr, db, dw1, dw2, dl, dwts, dw1s, dw2s)


def router_backward(probs, ids, weights, real, dweights, counts_pre, *, tau: float, renormalize: bool,
                    aux_coef: float, d_aux: float) -> np.ndarray:
    """Gradient of the router logits [T, E], float64, from the gate-weight gradients and the aux term.

    P2 §3.1: the gate weights are a softmax of logits / tau, over the k selected logits when
    renormalised (w_j = exp(z_j) / sum_sel exp(z_i)), else over all E (w_j = p_j); the softmax
    Jacobian gives dz = w (dw - <w, dw>) on the selected entries (the renormalised case) or
    p (g - <p, g>) with g the dw scattered over the experts. P4 §3.2's aux_switch
    = coef E sum_i f_i P_i with constant f_i = counts_pre_i / (n k) and P_i the mean of p_i over
    the n real tokens has d aux / d p[t, i] = coef E f_i / n, which reaches the logits through the
    same softmax Jacobian. The chain rule through z = logits / tau divides both by tau. Padding
    tokens (real False) get zeros.
    """
    probs = np.asarray(probs, dtype=np.float64)
    w = _f64(weights)
    dwts = _f64(dweights)
    T, E = probs.shape
    k = np.asarray(ids).shape[1]
    dl = np.zeros((T, E), dtype=np.float64)
    real = np.asarray(real, dtype=bool)
    ids = np.asarray(ids).astype(np.int64)
    for t in np.flatnonzero(real):
        sel = ids[t]
        if renormalize:
            ww = w[t]
            dl[t, sel] += ww * (dwts[t] - np.dot(ww, dwts[t]))
        else:
            p = probs[t]
            g = np.zeros(E)
            g[sel] = dwts[t]
            dl[t] += p * (g - np.dot(p, g))
    n = int(real.sum())
    if n > 0 and d_aux != 0.0:
        f_i = np.asarray(counts_pre, dtype=np.float64) / (n * k)
        g = d_aux * aux_coef * E * f_i / n
        p = probs[real]
        dl[real] += p * (g[None, :] - (p @ g)[:, None])
    dl /= float(np.float32(tau))
    return dl


def router_input_grads(dl, x, w_router):
    """The linear router's gradients from dL = d loss / d logits (logits = x W_r^T + b): dW_r = dL^T x,
    db = sum over tokens of dL, dx = dL W_r; float64."""
    dl = np.asarray(dl, dtype=np.float64)
    x64, wr64 = _f64(x), _f64(w_router)
    return dl.T @ x64, dl.sum(axis=0), dl @ wr64
