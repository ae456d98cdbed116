/*
 * moe.h -- C ABI of the MI355X (gfx950) forward pass of a top-k routed MoE FFN layer.
 *
 * Pages cited (by title):
 *   [P2] "Twinkle首发适配Deepseek-V4系列模型高效训练" (www.wmrh.cn/news/44033)
 *   [P3] "DeepSpeed ZeRO-3与MoE显存精算实战指南" (m.nlpx.cn/news/237350)
 *   [P4] "手搓一个LLaMA4-MoE" (www.nxmr.cn/news/140631)
 *
 * Notation: T tokens, d = d_model, f = d_ffn, E experts, k = top-k, C = per-expert capacity,
 * N = number of kept (token, slot) assignments (N <= T*k). All matrices are row-major and
 * contiguous. "act" is the activation storage type (x, Xp, H, Y, out) and "wt" the expert
 * weight type (W1, W2); both are fp32 or both are bf16. Router weight, bias, Gumbel noise,
 * logits, probabilities and gate weights are always fp32.
 *
 * Conventions shared by every call:
 *  - Ownership: every buffer is caller-owned device memory (except where "host" is stated).
 *    The library never allocates or frees device memory. Scratch space comes from the
 *    caller's workspace `ws` of at least moe_workspace_bytes(cfg) bytes, 256-byte aligned.
 *  - Streams: each call enqueues its kernels on `stream` and returns without synchronising;
 *    outputs are valid once the stream has reached that point. Calls that overlap on the same
 *    buffers or the same workspace race; the library keeps no state between calls.
 *  - Errors: every call returns a moe_status_t. Arguments are validated on the host before any
 *    launch; on a validation error nothing is launched. A failed kernel launch returns
 *    MOE_ERR_HIP. Inputs must be finite; results for NaN/Inf inputs are unspecified.
 *  - Determinism: two calls with the same inputs give bitwise equal outputs. Floating-point
 *    atomics appear in one place only: the backward's weight gradients, when there are fewer
 *    output tiles than CUs, add the two halves of a tile's reduction into a zeroed output with
 *    fp32 atomic adds; 0 + a is exact and a + b commutes, so the bits do not depend on which half
 *    lands first.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* a null required pointer or a size/value out of range     */
  MOE_ERR_UNSUPPORTED = 2,        /* a valid but unsupported combination (e.g. mixed dtypes)    */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed                 */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_INT4 = 2 } moe_dtype_t;

/* Capacity value meaning "no limit" (C = T). */
#define MOE_NO_CAPACITY (-1)

/* Limits checked by moe_validate_config. */
#define MOE_MAX_EXPERTS 64
#define MOE_MAX_TOP_K 8
#define MOE_MAX_TOKENS (1 << 24)

/*
 * Layer configuration. Parameter names follow P4 §2.1 (num_experts, num_experts_per_token,
 * aux_loss_coef), P3 (capacity: an absolute per-expert cap, its --moe_expert_capacity) and
 * P2 (router_temperature).
 */
typedef struct {
  int32_t T;             /* tokens, 1 .. MOE_MAX_TOKENS                                        */
  int32_t d_model;       /* d, a positive multiple of 8                                         */
  int32_t d_ffn;         /* f, a positive multiple of 8                                         */
  int32_t num_experts;   /* E, 1 .. MOE_MAX_EXPERTS                                             */
  int32_t top_k;         /* k, 1 .. min(E, MOE_MAX_TOP_K)                                       */
  int32_t capacity;      /* C >= 0 kept assignments per expert, or MOE_NO_CAPACITY              */
  float   temperature;   /* tau > 0: softmax and Gumbel keys use logits / tau (P2 §3.1)         */
  int32_t renormalize;   /* 1: gate weights = softmax over the k selected logits / tau;
                            0: gate weights = full softmax probability of each selected expert  */
  float   aux_coef;      /* coefficient of both aux losses (P4 §2.1 uses 0.01)                 */
  moe_dtype_t act_dtype;     /* x, Xp, H, Y, out: MOE_F32 or MOE_BF16                          */
  moe_dtype_t weight_dtype;  /* W1, W2: act_dtype, or MOE_INT4 with bf16 activations (packed
                                4-bit weights, see moe_quantize_int4)                          */
  int32_t noise_in_logits;   /* how the noise input enters (0 or 1):
                                0: Gumbel top-k (P2 §3.1), it perturbs the selection key only;
                                1: additive router noise (P4 §3.2), logits = fp32(logits + n)
                                   and the noisy logits are used everywhere downstream         */
  int32_t d_ffn_shared;      /* fs: width of the shared expert (P4 §5.2), 0 = none, else a
                                positive multiple of 8; moe_forward then adds
                                W2s SiLU(W1s x) to every token's output                      */
  int32_t straight_through;  /* 0 or 1. 1: P2 §3.1's straight-through estimator. The routing
                                matrix k-hot + softmax - detach(softmax) has the k-hot value,
                                so every selected expert's gate weight is exactly 1
                                (renormalize is not used). The backward calls take the gradient
                                through the full softmax of logits / tau, as for renormalize 0. */
  int32_t keep_preact;       /* 0 or 1. 1 (training): moe_forward also keeps the pre-activation
                                A = Xp W1^T (rounded once to act) in its workspace, and
                                moe_backward reads it instead of recomputing it: one grouped GEMM
                                less per backward for one [T*k, f] write per forward. The values
                                are the ones a recompute would give, bit for bit. Not with
                                MOE_INT4 weights (MOE_ERR_UNSUPPORTED).                      */
} moe_config_t;

/* Static text for a status code (never NULL). Host only. */
const char* moe_status_string(moe_status_t status);

/* Checks a configuration on the host; touches no GPU. Returns MOE_OK, MOE_ERR_INVALID_ARGUMENT
 * (cfg NULL, a size out of the ranges above, tau not finite and > 0, capacity < -1,
 * renormalize, noise_in_logits, straight_through or keep_preact not 0 or 1, an unknown dtype) or MOE_ERR_UNSUPPORTED
 * (act_dtype != weight_dtype, except MOE_INT4 weights with bf16 activations; MOE_INT4 weights
 * also need d and f multiples of 512, T * k <= 64 * E (the weight-streaming regime) and no
 * shared expert). */
moe_status_t moe_validate_config(const moe_config_t* cfg);

/* C = ceil(cf * T * k / E) for the decimal capacity factor cf = cf_num / cf_den, in exact
 * integer arithmetic (P3 §3.4 and §5.1 give factors such as 1.2 but no formula; this is the
 * plain reading). Returns -1 if T, k, E, cf_num or cf_den is not positive. Host only. */
int32_t moe_capacity_from_factor(int32_t T, int32_t k, int32_t E, int32_t cf_num, int32_t cf_den);

/*
 * 4-bit expert weights [P4 §5.2]. A [rows, K] bf16 weight (rows a multiple of 16, K of 128) is
 * stored as symmetric group-wise int4 along K, groups of 64: per (row, group) a bf16 scale
 * s = bf16(fp32(amax / 7)) and codes q = clamp(rint(fp32(w / s)), -8, 7) (0 where s = 0),
 * two's complement nibbles, two per byte (low nibble = even column). The layer uses
 * w' = bf16(q * s). Layout, tiled so that each GEMM load instruction reads 1 KiB contiguously:
 * the codes of rows 16 t .. + 15 and columns 128 s .. + 127 form the 1 KiB block
 * t * K/128 + s, in which the 16 bytes at 16 * (16 g + r) hold row 16 t + r, columns
 * 128 s + 32 g .. + 31; the scales follow from the next 256-byte boundary (the bytes in between
 * are zero), 32 per block: row r's two groups at 2 r and 2 r + 1. For the expert weights
 * rows = E * f, K = d (W1) and rows = E * d, K = f (W2).
 * moe_int4_bytes: size of that buffer (0 for other sizes).
 * moe_quantize_int4: fills it from w (device, 16-byte aligned) on `stream`; returns
 * MOE_ERR_INVALID_ARGUMENT for other sizes or null/misaligned pointers.
 */
size_t moe_int4_bytes(int64_t rows, int32_t K);
moe_status_t moe_quantize_int4(int64_t rows, int32_t K, const void* w, void* packed, hipStream_t stream);

/* Workspace bytes that every call below accepts for this configuration (0 if cfg is invalid).
 * moe_forward keeps Xp, H and Y there: about (2 d + f) * T * k * sizeof(act) plus O(T k). */
size_t moe_workspace_bytes(const moe_config_t* cfg);

/*
 * Router: logits, selection key, top-k and gate weights for every token.
 * [P2 §3.1] scores = W_router x, probs = softmax(scores / tau), top-k; with Gumbel noise the
 * ranked key is (logits + g) / tau. [P4 §2.4] a linear router, top-k, softmax weights.
 *   x          [T, d] act          token hidden states (ignored when logits_in != NULL)
 *   w_router   [E, d] fp32         router weight, 16-byte aligned (ignored when logits_in != NULL)
 *   bias       [E] fp32 or NULL    per-expert logit bias, added after the product
 *   noise      [T, E] fp32 or NULL noise, entering as cfg->noise_in_logits says. Mode 0 (Gumbel):
 *                                  key = fl32(fl32(logit + g) / tau), the noise changes the
 *                                  selection only. Mode 1 (additive): logit = fl32(logit + n)
 *                                  (not added again to logits_in) and key = logit. Without
 *                                  noise, key = logit.
 *   token_mask [T] uint8 or NULL   nonzero = real token; a padding token (0) gets ids -1 and
 *                                  weights 0 in every slot and probs_out row 0 [P4 §4.1]
 *   logits_in  [T, E] fp32 or NULL route these final logits instead of computing x W_r^T + b
 *   logits_out [T, E] fp32 or NULL the router logits (fp32 accumulation of x W_r^T, + bias,
 *                                  + additive noise in mode 1), padding tokens included
 *   probs_out  [T, E] fp32 or NULL softmax(logits / tau) over all E
 *   ids        [T, k] int32        selected experts, descending key, lowest index on ties
 *                                  (-0.0 ties +0.0)
 *   weights    [T, k] fp32         gate weight of each selected expert (see renormalize)
 * Workspace: per-block probability sums used by moe_forward's aux loss (unused here).
 */
moe_status_t moe_route(const moe_config_t* cfg, const void* x, const float* w_router,
                       const float* bias, const float* noise, const uint8_t* token_mask,
                       const float* logits_in, float* logits_out, float* probs_out, int32_t* ids,
                       float* weights, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Dispatch: per-expert histogram, capacity cut, offsets and stable permutation, and the row
 * gather Xp[row] = x[perm_token[row]]. [P4 §2.4] sort the [T, k] index by expert id, count
 * tokens per expert, split into segments, gather tokens by table lookup; [P3 §3.1] cap the
 * tokens per expert. Assignments are taken in (token, slot) order; the first C of each expert
 * are kept, the rest dropped.
 *   ids        [T, k] int32 device, each in [0, E) and distinct within a token, or -1 in
 *                                  every slot of a padding token (as moe_route gives). A -1
 *                                  slot is neither counted, kept nor dropped (row_of -1,
 *                                  dropped 0). Other values are not checked and give
 *                                  unspecified results.
 *   x          [T, d] act
 *   counts_pre [E] int32           assignments per expert before the cut
 *   counts     [E] int32           kept per expert = min(counts_pre, C)
 *   offsets    [E+1] int32         exclusive scan of counts; offsets[E] = N
 *   perm_token [T*k] int32         token of row r for r < N (entries >= N untouched)
 *   row_of     [T, k] int32        row of each kept slot, -1 if dropped
 *   dropped    [T, k] uint8        1 if the slot was dropped by the capacity cut
 *   n_dropped  [1] int32           assignments dropped by the cut (sum of counts_pre - N)
 *   xp         [T*k, d] act        gathered rows; rows >= N untouched
 */
moe_status_t moe_dispatch(const moe_config_t* cfg, const int32_t* ids, const void* x,
                          int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* row_of, uint8_t* dropped,
                          int32_t* n_dropped, void* xp, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Expert FFN as two grouped GEMMs over the expert segments given by offsets (w1/w2 are packed
 * 4-bit buffers when cfg->weight_dtype is MOE_INT4).
 * [P4 §2.4] each expert is a two-layer FFN. For rows r in [offsets[e], offsets[e+1]):
 *   H[r] = SiLU(Xp[r] W1[e]^T)   (fp32 accumulate, SiLU in fp32, one rounding to act)
 *   Y[r] = H[r] W2[e]^T          (fp32 accumulate, one rounding to act)
 *   xp      [T*k, d] act   w1 [E, f, d] wt   w2 [E, d, f] wt   offsets [E+1] int32 device
 *   h       [T*k, f] act   (scratch output, rows >= N untouched)
 *   y       [T*k, d] act   (rows >= N untouched)
 * offsets must be non-decreasing with offsets[0] = 0 and offsets[E] <= T*k.
 */
moe_status_t moe_expert_ffn(const moe_config_t* cfg, const void* xp, const int32_t* offsets,
                            const void* w1, const void* w2, void* h, void* y, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Weighted combine (unpermute). [P4 §2.4] a token's output is the sum of its selected
 * experts' outputs weighted by the gate weights, [P4 §5.2] plus a shared expert's output:
 *   out[t] = sum_{j = 0..k-1, row_of[t,j] >= 0} weights[t,j] * y[row_of[t,j]] (+ y_shared[t])
 * accumulated in fp32 in slot order, the shared term last, rounded once to act. A token with
 * every slot dropped and no shared term gets zeros. y [T*k, d] act, row_of [T, k] int32
 * (entries < T*k), weights [T, k] fp32, y_shared [T, d] act or NULL, out [T, d] act.
 */
moe_status_t moe_combine(const moe_config_t* cfg, const void* y, const int32_t* row_of,
                         const float* weights, const void* y_shared, void* out, hipStream_t stream);

/*
 * Auxiliary load-balance losses and the router entropy over the n real tokens (n = T without a
 * mask), aux[0] = aux_switch, aux[1] = aux_balance, aux[2] = mean router entropy (device fp32):
 *   P_i = (1/n) sum_t softmax(logits_t / tau)_i  (from probs when given, else from logits)
 *   aux_switch  = coef * E * sum_i (counts_pre[i] / (n k)) * P_i            [P4 §3.2]
 *   aux_balance = coef * sum_i (counts_pre[i] / n - k / E)^2                [P3 §3.2]
 *   entropy     = (1/n) sum_t -sum_i p_ti ln p_ti                            [P4 §3.3]
 * aux_switch is coef for uniform routing; aux_balance is 0 for perfectly uniform counts. With
 * no real token all three are 0.
 *   probs [T, E] fp32 or NULL, logits [T, E] fp32 (used when probs is NULL),
 *   token_mask [T] uint8 or NULL (padding tokens, 0, are left out),
 *   counts_pre [E] int32 (pre-capacity counts from moe_dispatch), aux [3] fp32.
 */
moe_status_t moe_aux_loss(const moe_config_t* cfg, const float* probs, const float* logits,
                          const uint8_t* token_mask, const int32_t* counts_pre, float* aux,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Optional outputs and timing hooks of moe_forward. Every pointer may be NULL; a non-NULL
 * device pointer receives the named tensor (shapes as in the calls above). When `events` is
 * non-NULL it holds n_events >= MOE_FORWARD_NUM_KERNELS + 1 created hipEvent_t; events[i] is
 * recorded on `stream` before kernel i and events[MOE_FORWARD_NUM_KERNELS] after the last, so
 * hipEventElapsedTime gives per-kernel times. Kernel order: route (it also counts each token
 * group's selections per expert), dispatch-histogram (empty: the router's counts are used),
 * dispatch-scan (the capacity cut and the aux losses when the histogram is too large for every
 * dispatch workgroup to sum it itself, else empty), dispatch (ranks, row map, gather; it also
 * forms the capacity cut, the offsets and the aux losses when the scan step is empty), gemm1
 * (W1 + SiLU), gemm2 (W2, with the reduction of its split tail when it has one), shared expert
 * (both of its GEMMs; empty without one), combine.
 */
#define MOE_FORWARD_NUM_KERNELS 8
typedef struct {
  float*   logits;      /* [T, E] */
  float*   probs;       /* [T, E] */
  int32_t* ids;         /* [T, k] */
  float*   weights;     /* [T, k] */
  int32_t* counts_pre;  /* [E]    */
  int32_t* counts;      /* [E]    */
  int32_t* offsets;     /* [E+1]  */
  int32_t* perm_token;  /* [T*k]  */
  int32_t* row_of;      /* [T, k] */
  uint8_t* dropped;     /* [T, k] */
  int32_t* n_dropped;   /* [1]    */
  void*    xp;          /* [T*k, d] act */
  void*    h;           /* [T*k, f] act */
  void*    y;           /* [T*k, d] act */
  void*    y_shared;    /* [T, d] act, the shared expert's output (with d_ffn_shared > 0) */
  hipEvent_t* events;
  int32_t  n_events;
} moe_debug_outputs;

/*
 * The whole layer: route -> dispatch -> expert FFN (and the shared expert) -> combine, plus both
 * aux losses and the router entropy (P4 §2.4, §3.2, §3.3, §4.1 and §5.2, P2 §3.1, P3
 * §3.1-3.2). Inputs as in the calls above; w1_shared [fs, d] wt and w2_shared [d, fs] wt are
 * required when cfg->d_ffn_shared > 0 and ignored otherwise (the shared expert runs on every
 * token, padding included). out [T, d] act (routed part zero for padding tokens); aux [3] fp32
 * device as moe_aux_loss. dbg may be NULL.
 */
moe_status_t moe_forward(const moe_config_t* cfg, const void* x, const float* w_router,
                         const float* bias, const float* noise, const uint8_t* token_mask,
                         const void* w1, const void* w2, const void* w1_shared,
                         const void* w2_shared, void* out, float* aux, moe_debug_outputs* dbg,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward without a caller workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It runs the
 * same kernels as moe_forward with dbg NULL and gives bitwise the same out and aux, with the
 * workspace taken from a static device array of MOE_NOALLOC_SCRATCH_BYTES bytes: one per GPU the
 * library runs on, on the device current at the call (x, the weights, out and aux must live
 * there), located on the first call on each device and held until the process ends. It calls
 * no allocating routine. The caller still owns and passes every input and output.
 * Limit: a configuration whose moe_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES (e.g. the
 * large-batch layers whose grouped GEMM keeps split partial sums) returns
 * MOE_ERR_WORKSPACE_TOO_SMALL before any launch; small-batch layers (the weight-streaming
 * regime: 256 tokens, d 2048, f 4096, 16 experts, top-2 needs about 9 MiB) fit.
 * The array keeps the last call's contents; nothing in it needs clearing between calls. Calls
 * that overlap on one GPU (on different streams, or from several threads without ordering) share
 * the array and race: serialise them. The intermediates are not exposed, so moe_backward cannot
 * follow this call.
 * moe_forward_noalloc_max_bytes: MOE_NOALLOC_SCRATCH_BYTES. Host only.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
size_t moe_forward_noalloc_max_bytes(void);
moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const void* x, const float* w_router,
                                 const float* bias, const float* noise, const uint8_t* token_mask,
                                 const void* w1, const void* w2, const void* w1_shared,
                                 const void* w2_shared, void* out, float* aux, hipStream_t stream);

/*
 * Backward pass [P4 §2.4: the layer is trained end to end]. Gradients of
 * L = sum(d_out * out) (+ d_aux * aux_switch) flow back through the combine, the expert FFNs and
 * the gather; the selection, the capacity cut and the noise pass none. The calls mirror the
 * forward ones and take the forward's intermediates (moe_forward's debug outputs). Products
 * accumulate in fp32; stored gradients are rounded once to act.
 * moe_backward_workspace_bytes: the workspace the backward calls take (0 if cfg is invalid).
 * moe_combine_backward: dy[row_of[t,j]] = weights[t,j] * d_out[t] (act; rows of dropped slots
 *   untouched) and dweights[t,j] = <d_out[t], y[row_of[t,j]]> (fp32; 0 without a row).
 *   d_out [T, d] act, y [T*k, d] act, row_of [T, k], weights [T, k] fp32, dy [T*k, d] act,
 *   dweights [T, k] fp32.
 * moe_expert_ffn_backward: over each expert's rows, with A = xp W1_e^T (recomputed) and
 *   dA = (dy W2_e) * SiLU'(A) (the product dy W2_e rounded to act, then dA rounded to act):
 *   dxp = dA W1_e (act; rows >= N untouched), and when not NULL
 *   dw2[e] = dy^T h (fp32 [E, d, f], needs h) and dw1[e] = dA^T xp (fp32 [E, f, d]); an expert
 *   with no rows gets zero weight gradients. bf16/fp32 weights only. xp, dy, dxp [T*k, d] act,
 *   h [T*k, f] act (the forward's H), offsets [E+1] as in the forward.
 * moe_dispatch_backward: dx[t] = sum over kept slots of dxp[row_of[t,j]] (fp32, one rounding);
 *   dx [T, d] act.
 * moe_route_backward: the router's share [P2 §3.1 softmax gating with temperature; P4 §3.2
 *   aux_switch through the mean probabilities]. Per real token (token_mask NULL or nonzero),
 *   with the gate weights w and their gradients dw (moe_combine_backward's dweights):
 *   renormalised weights (softmax over the k selected logits / tau) give
 *   dL[t, sel_j] = w_j (dw_j - sum_i w_i dw_i) / tau; otherwise (w = the full softmax p, or
 *   cfg.straight_through, whose forward weights are 1) dL[t] = p * (g - <p, g>) / tau with g
 *   the dw scattered to the selected experts. d_aux != 0
 *   adds p * (a - <p, a>) / tau with a_e = d_aux coef E f_e / n, f_e = counts_pre[e] / (n k),
 *   n = sum(counts_pre) / k the real tokens. Padding tokens get dL = 0. Then, each when not
 *   NULL: dx[t] += dL[t] W_r (fp32 products, the sum added to dx's act value with one more
 *   rounding), dw_router = dL^T x (fp32 [E, d], deterministic order), dbias = sum_t dL[t].
 *   logits [T, E] fp32 are the forward's (moe_route's logits_out: bias and additive noise in
 *   them); ids, weights [T, k] as moe_route wrote them; dweights [T, k] fp32; counts_pre [E]
 *   (needed when d_aux != 0); dlogits [T, E] fp32 out (required). dx needs w_router; dw_router
 *   needs x and the backward workspace. Noise and the selection pass no gradient.
 */
size_t moe_backward_workspace_bytes(const moe_config_t* cfg);
moe_status_t moe_combine_backward(const moe_config_t* cfg, const void* d_out, const void* y,
                                  const int32_t* row_of, const float* weights, void* dy,
                                  float* dweights, hipStream_t stream);
moe_status_t moe_expert_ffn_backward(const moe_config_t* cfg, const void* xp, const int32_t* offsets,
                                     const void* w1, const void* w2, const void* h, const void* dy,
                                     void* dxp, float* dw1, float* dw2, void* ws, size_t ws_bytes,
                                     hipStream_t stream);
moe_status_t moe_dispatch_backward(const moe_config_t* cfg, const void* dxp, const int32_t* row_of,
                                   void* dx, hipStream_t stream);
/*
 * moe_backward: the whole layer's backward pass in one call (the five steps above plus the shared
 * expert's: dHs = d_out W2s, dAs = dHs * SiLU'(x W1s^T), dx += dAs W1s, dW2s = d_out^T Hs,
 * dW1s = dAs^T x). It reads the forward's intermediates (logits, ids, weights, counts, row map,
 * Xp, H, Y, Hs) from fwd_ws, the workspace of a moe_forward call with the same cfg, inputs and
 * token_mask, made with dbg NULL or with only its events set (debug buffers divert those
 * intermediates) and not reused since. d_out [T, d] act; dx [T, d] act out (required); the
 * weight gradients are fp32 outputs written when not NULL: dw_router [E, d], dbias [E],
 * dw1 [E, f, d], dw2 [E, d, f], dw1_shared [fs, d], dw2_shared [d, fs]. ws is the backward
 * workspace (moe_backward_workspace_bytes). bf16/fp32 weights only (MOE_ERR_UNSUPPORTED for
 * 4-bit weights). Calls that share fwd_ws or ws must not overlap. dx: with bf16 activations,
 * top-1 or top-2 and at most 16 experts, the kept slots' dxp rows (slot order), the shared
 * expert's term and the router's dL W_r are summed in fp32 and rounded to act once; otherwise dx
 * is formed as moe_dispatch_backward and then moe_route_backward form it (two roundings).
 */
moe_status_t moe_backward(const moe_config_t* cfg, const void* x, const float* w_router,
                          const uint8_t* token_mask, const void* w1, const void* w2,
                          const void* w1_shared, const void* w2_shared, const void* d_out,
                          float d_aux, const void* fwd_ws, size_t fwd_ws_bytes, void* dx,
                          float* dw_router, float* dbias, float* dw1, float* dw2,
                          float* dw1_shared, float* dw2_shared, void* ws, size_t ws_bytes,
                          hipStream_t stream);
moe_status_t moe_route_backward(const moe_config_t* cfg, const void* x, const float* w_router,
                                const float* logits, const int32_t* ids, const float* weights,
                                const float* dweights, const int32_t* counts_pre,
                                const uint8_t* token_mask, float d_aux, float* dlogits, void* dx,
                                float* dw_router, float* dbias, void* ws, size_t ws_bytes,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
