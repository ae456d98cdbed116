// Host side of the C ABI declared in include/moe.h: validation, workspace carve-up and the
// kernel sequence of each call. No call allocates device memory or synchronises the stream.
#include "../../include/moe.h"

#include <math.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxDim = 32768;

struct Layout {
  size_t psum, blk_hist, blk_base, probsum;
  size_t logits, ids, weights, counts_pre, counts, offsets, perm, row_of, dropped, ndrop;
  size_t xp, h, y;
  size_t hs, ys, sh_off;   // shared expert: Hs [T, fs], Ys [T, d], its segment offsets [2]
  size_t a1;               // keep_preact: the pre-activation A = Xp W1^T [T k, f]
  size_t sk_part;   // partial sums of the 256 x 256 grouped GEMM's split tail (empty if unused)
  size_t total;
};

size_t act_size(const moe_config_t& c) { return c.act_dtype == MOE_BF16 ? 2 : 4; }

Layout layout(const moe_config_t& c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t T = (size_t)c.T, k = (size_t)c.top_k, E = (size_t)c.num_experts;
  const size_t d = (size_t)c.d_model, f = (size_t)c.d_ffn, TK = T * k, a = act_size(c);
  L.psum = take((size_t)route_max_parts(c.T, c.num_experts) * (E + 2) * sizeof(double));
  // histogram blocks: the router's token groups (moe_forward) or moe_dispatch's own blocks
  const size_t nb_route = (size_t)dispatch_blocks(c.T, route_block_tokens(c.T, c.num_experts, c.act_dtype == MOE_BF16, false));
  const size_t nb_own = (size_t)dispatch_blocks(c.T, DISPATCH_BLOCK_TOKENS);
  const size_t nb = nb_route > nb_own ? nb_route : nb_own;
  L.blk_hist = take(nb * E * 4);
  L.blk_base = take(nb * E * 4);
  L.probsum = take((size_t)probsum_num_blocks(c.T) * (E + 2) * sizeof(double));
  L.logits = take(T * E * 4);
  L.ids = take(TK * 4);
  L.weights = take(TK * 4);
  L.counts_pre = take(E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(TK * 4);
  L.row_of = take(TK * 4);
  L.dropped = take(TK);
  L.ndrop = take(4);
  L.xp = take(TK * d * a);
  L.h = take(TK * f * a);
  L.y = take(TK * d * a);
  const size_t fs = c.d_ffn_shared > 0 ? (size_t)c.d_ffn_shared : 0;
  L.hs = take(T * fs * a);
  L.ys = take(fs ? T * d * a : 0);
  L.sh_off = take(fs ? 8 : 0);
  L.a1 = take(c.keep_preact ? TK * f * a : 0);
  const bool bf16 = c.act_dtype == MOE_BF16;
  const bool big = gemm_uses_big(bf16, c.d_model, c.T * c.top_k, c.num_experts) ||
                   gemm_uses_big(bf16, c.d_ffn, c.T * c.top_k, c.num_experts) ||
                   (fs && (gemm_uses_big(bf16, c.d_model, c.T, 1) || gemm_uses_big(bf16, c.d_ffn_shared, c.T, 1)));
  L.sk_part = take(big ? gemm_big_part_bytes() : 0);
  L.total = off;
  return L;
}

// Backward-pass workspace: transposed expert weights (for the GEMM paths that need them, see
// run_gemm_kn), the recomputed pre-activation and the gradient of H (turned into the gradient of
// the pre-activation in place).
struct BwdLayout {
  size_t w1t, w2t, a1, dh, sk_part, rw_part;
  size_t dy, dwts, dxp, dlogits;              // moe_backward's own intermediates
  size_t w1st, w2st, as, dhs, dxs;            // the shared expert's (empty without one)
  size_t total;
};

BwdLayout bwd_layout(const moe_config_t& c) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t a = act_size(c), E = (size_t)c.num_experts, d = (size_t)c.d_model, f = (size_t)c.d_ffn;
  const size_t TK = (size_t)c.T * (size_t)c.top_k;
  L.w1t = take(E * d * f * a);
  L.w2t = take(E * d * f * a);
  L.a1 = take(TK * f * a);
  L.dh = take(TK * f * a);
  const bool bf16 = c.act_dtype == MOE_BF16;
  const size_t T = (size_t)c.T, fs = c.d_ffn_shared > 0 ? (size_t)c.d_ffn_shared : 0;
  const bool big = gemm_uses_big(bf16, c.d_model, c.T * c.top_k, c.num_experts) ||
                   gemm_uses_big(bf16, c.d_ffn, c.T * c.top_k, c.num_experts) ||
                   (fs && (gemm_uses_big(bf16, c.d_model, c.T, 1) || gemm_uses_big(bf16, c.d_ffn_shared, c.T, 1)));
  L.sk_part = take(big ? gemm_big_part_bytes() : 0);
  L.rw_part = take(route_bwd_part_bytes(c.T, c.d_model, c.num_experts));
  L.dy = take(TK * d * a);
  L.dwts = take(TK * 4);
  L.dxp = take(TK * d * a);
  L.dlogits = take(T * E * 4);
  L.w1st = take(fs * d * a);
  L.w2st = take(fs * d * a);
  L.as = take(T * fs * a);
  L.dhs = take(T * fs * a);
  L.dxs = take(fs ? T * d * a : 0);
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                         \
  do {                                        \
    const moe_status_t st_ = (expr);          \
    if (st_ != MOE_OK) return st_;            \
  } while (0)

#define MOE_LAUNCH(expr) MOE_TRY(hip_status(expr))

moe_status_t check_ws(const moe_config_t* cfg, const void* ws, size_t ws_bytes) {
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < layout(*cfg).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

uint8_t* at(void* ws, size_t off) { return (uint8_t*)ws + off; }

int capacity_of(const moe_config_t& c) { return c.capacity < 0 ? -1 : c.capacity; }

// The integer a caller stored in an enum-typed field or argument. A C caller may store any int
// there, and in C++ loading a value outside the enumerators' range through the enum type is
// undefined, so values not yet validated are read as their bytes.
template <typename En>
int enum_int(const En& v) {
  static_assert(sizeof(En) == sizeof(int), "C enums are int-sized");
  int i;
  memcpy(&i, &v, sizeof i);
  return i;
}

// The configuration and the required pointers of a whole-layer forward (host only).
moe_status_t forward_args_status(const moe_config_t* cfg, const void* x, const float* w_router, const void* w1,
                                 const void* w2, const void* w1_shared, const void* w2_shared, const void* out,
                                 const float* aux) {
  MOE_TRY(moe_validate_config(cfg));
  if (!x || !w_router || !w1 || !w2 || !out || !aux) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w1) || !aligned16(w2) || !aligned16(out))
    return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->d_ffn_shared > 0 && (!w1_shared || !w2_shared || !aligned16(w1_shared) || !aligned16(w2_shared)))
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

// ---- the kernel sequences, shared by the single-step calls and moe_forward

moe_status_t run_route(const moe_config_t& c, const void* x, const float* w_router, const float* bias,
                       const float* noise, const uint8_t* token_mask, const float* logits_in,
                       float* logits_out, float* probs_out, int32_t* ids, float* weights, double* psum,
                       hipStream_t s, int32_t* blk_hist = nullptr) {
  RouteParams p{};
  p.T = c.T;
  p.d = c.d_model;
  p.E = c.num_experts;
  p.k = c.top_k;
  p.tau = c.temperature;
  p.renormalize = c.renormalize;
  p.straight_through = c.straight_through;
  p.x = x;
  p.w_router = w_router;
  p.bias = logits_in ? nullptr : bias;
  p.gumbel = noise;
  p.noise_in_logits = c.noise_in_logits;
  p.token_mask = token_mask;
  p.logits_in = logits_in;
  p.logits_out = logits_out;
  p.probs_out = probs_out;
  p.ids = ids;
  p.weights = weights;
  p.psum = psum;
  p.blk_hist = blk_hist;
  MOE_LAUNCH(launch_route(p, c.act_dtype == MOE_BF16, s));
  return MOE_OK;
}

ScanParams scan_params(const moe_config_t& c, int nb, int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                       int32_t* n_dropped, void* ws) {
  const Layout L = layout(c);
  ScanParams p{};
  p.TK = c.T * c.top_k;
  p.nb = nb;
  p.E = c.num_experts;
  p.capacity = capacity_of(c);
  p.blk_hist = (const int32_t*)at(ws, L.blk_hist);
  p.blk_base = (int32_t*)at(ws, L.blk_base);
  p.counts_pre = counts_pre;
  p.counts = counts;
  p.offsets = offsets;
  p.n_dropped = n_dropped;
  return p;
}

// The dispatch of blocks of bt tokens whose histograms are in the workspace. When the histogram is
// small every dispatch workgroup sums it itself (blk_base null; the aux losses, when `aux` is
// given, and the shared expert's offsets come from its block 0); otherwise the one-workgroup scan
// (with the aux losses) runs first. `scan_mark` records the timing event between the two.
template <typename Mark>
moe_status_t run_dispatch(const moe_config_t& c, int bt, const int32_t* ids, const void* x, int32_t* counts_pre,
                          int32_t* counts, int32_t* offsets, int32_t* n_dropped, int32_t* perm_token, int32_t* row_of,
                          uint8_t* dropped, void* xp, void* ws, const AuxParams* aux, int32_t* shared_offsets,
                          Mark scan_mark, hipStream_t s) {
  const Layout L = layout(c);
  const int nb = dispatch_blocks(c.T, bt);
  DispatchParams p{};
  p.T = c.T;
  p.k = c.top_k;
  p.E = c.num_experts;
  p.row_bytes = (int)(c.d_model * act_size(c));
  p.capacity = capacity_of(c);
  p.bt = bt;
  p.nb = nb;
  p.ids = ids;
  p.blk_hist = (const int32_t*)at(ws, L.blk_hist);
  p.counts_pre = counts_pre;
  p.counts = counts;
  p.offsets = offsets;
  p.n_dropped = n_dropped;
  p.x = (const uint8_t*)x;
  p.row_of = row_of;
  p.dropped = dropped;
  p.perm_token = perm_token;
  p.xp = (uint8_t*)xp;
  if (dispatch_fused(nb, c.num_experts)) {
    if (aux) p.aux = *aux;
    p.shared_offsets = shared_offsets;
    MOE_TRY(scan_mark());
  } else {
    const ScanParams sp = scan_params(c, nb, counts_pre, counts, offsets, n_dropped, ws);
    if (aux) {
      ScanAuxParams sa{};
      sa.s = sp;
      sa.a = *aux;
      sa.shared_offsets = shared_offsets;
      MOE_LAUNCH(launch_scan_aux(sa, s));
    } else {
      MOE_LAUNCH(launch_scan(sp, s));
    }
    MOE_TRY(scan_mark());
    p.blk_base = (const int32_t*)at(ws, L.blk_base);
  }
  MOE_LAUNCH(launch_dispatch(p, s));
  return MOE_OK;
}

// One grouped GEMM over `experts` segments of at most `rows` rows in total (the routed experts:
// E segments of the T k permuted rows; the shared expert: one segment of the T tokens).
// `sk` is the split-tail partial-sum region of the caller's workspace (null: no split tail).
moe_status_t run_gemm_sk(const moe_config_t& c, const void* a, const void* b, void* out, const int32_t* offsets,
                         int n, int kdim, bool silu, void* sk, hipStream_t s, int experts = -1, int rows = -1,
                         bool int4 = false, void* pre = nullptr, bool first_layer = false, bool b_kn = false) {
  if (experts < 0) experts = c.num_experts;
  if (rows < 0) rows = c.T * c.top_k;
  GemmParams p{};
  if (gemm_uses_big(c.act_dtype == MOE_BF16, kdim, rows, experts)) p.sk_part = sk;
  p.E = experts;
  p.N = n;
  p.K = kdim;
  p.max_rows = rows;
  p.A = a;
  p.B = b;
  p.C = out;
  p.C2 = silu ? pre : nullptr;
  p.offsets = offsets;
  p.sort_split = !silu && !first_layer;
  p.b_kn = b_kn ? 1 : 0;
  if (int4) {
    p.q4_scale_off = q4_scale_offset((size_t)experts * (size_t)n, kdim);
    MOE_LAUNCH(launch_gemm_q4(p, silu, s));
  } else {
    MOE_LAUNCH(launch_gemm(p, c.act_dtype == MOE_BF16, silu, s));
  }
  return MOE_OK;
}

// out = a w_e over each expert's rows, with the other layer's weights as they are: w is
// [E, kdim, n] (for dH: W2 [E, d, f]; for dXp: W1 [E, f, d]). The 256 x 256 and weight-streaming
// kernels read that layout directly; the other GEMM path takes its transpose [E, n, kdim], made
// here in wt.
moe_status_t run_gemm_kn(const moe_config_t& c, const void* a, const void* w, void* wt, void* out,
                         const int32_t* offsets, int n, int kdim, void* sk, hipStream_t s, int experts = -1,
                         int rows = -1) {
  const int E = experts < 0 ? c.num_experts : experts;
  const int R = rows < 0 ? c.T * c.top_k : rows;
  const bool bf16 = c.act_dtype == MOE_BF16;
  if (gemm_uses_big(bf16, kdim, R, E) || gemm_uses_stream(bf16, kdim, R, E))
    return run_gemm_sk(c, a, w, out, offsets, n, kdim, false, sk, s, experts, rows, false, nullptr, false, true);
  MOE_LAUNCH(launch_transpose(w, wt, E, kdim, n, (int)act_size(c), s));
  return run_gemm_sk(c, a, wt, out, offsets, n, kdim, false, sk, s, experts, rows);
}

moe_status_t run_gemm(const moe_config_t& c, const void* a, const void* b, void* out, const int32_t* offsets,
                      int n, int kdim, bool silu, void* ws, hipStream_t s, int experts = -1, int rows = -1,
                      void* pre = nullptr) {
  return run_gemm_sk(c, a, b, out, offsets, n, kdim, silu, at(ws, layout(c).sk_part), s, experts, rows,
                     c.weight_dtype == MOE_INT4 && experts < 0, pre);
}

moe_status_t run_combine(const moe_config_t& c, const void* y, const int32_t* row_of, const float* weights,
                         const void* y_shared, void* out, hipStream_t s) {
  CombineParams p{};
  p.T = c.T;
  p.d = c.d_model;
  p.k = c.top_k;
  p.max_rows = c.T * c.top_k;
  p.y = y;
  p.y_shared = y_shared;
  p.row_of = row_of;
  p.weights = weights;
  p.out = out;
  MOE_LAUNCH(launch_combine(p, c.act_dtype == MOE_BF16, s));
  return MOE_OK;
}

AuxParams aux_params(const moe_config_t& c, const double* psum, int nparts, const int32_t* counts_pre, float* aux) {
  AuxParams p{};
  p.T = c.T;
  p.E = c.num_experts;
  p.k = c.top_k;
  p.nparts = nparts;
  p.coef = c.aux_coef;
  p.tau = c.temperature;
  p.psum = psum;
  p.counts_pre = counts_pre;
  p.aux = aux;
  return p;
}

moe_status_t run_aux_final(const moe_config_t& c, const double* psum, int nparts, const int32_t* counts_pre,
                           float* aux, hipStream_t s) {
  MOE_LAUNCH(launch_aux_final(aux_params(c, psum, nparts, counts_pre, aux), s));
  return MOE_OK;
}

// The routed experts' backward: dXp, and dW1 / dW2 when asked for (shared by moe_expert_ffn_backward
// and moe_backward).
moe_status_t expert_ffn_bwd(const moe_config_t& c, const BwdLayout& L, const void* xp, const int32_t* offsets,
                            const void* w1, const void* w2, const void* h, const void* dy, void* dxp, float* dw1,
                            float* dw2, void* ws, hipStream_t stream, const void* a_kept = nullptr) {
  const bool bf16 = c.act_dtype == MOE_BF16;
  const int E = c.num_experts, d = c.d_model, f = c.d_ffn;
  void* w1t = at(ws, L.w1t);   // [E, d, f], when the GEMM path needs the transpose (run_gemm_kn)
  void* w2t = at(ws, L.w2t);   // [E, f, d], likewise
  void* a1 = at(ws, L.a1);     // [T k, f] pre-activation Xp W1^T
  void* dh = at(ws, L.dh);     // [T k, f] dH, then dA in place
  void* sk = at(ws, L.sk_part);
  if (a_kept) a1 = const_cast<void*>(a_kept);   // the forward's own pre-activation (read only)
  else MOE_TRY(run_gemm_sk(c, xp, w1, a1, offsets, f, d, false, sk, stream, -1, -1, false, nullptr, true));
  MOE_TRY(run_gemm_kn(c, dy, w2, w2t, dh, offsets, f, d, sk, stream));   // dH = dY W2_e
  GradWParams g{};
  g.E = E;
  g.max_rows = c.T * c.top_k;
  g.offsets = offsets;
  if (dw2) {   // dW2_e = dY^T H over the expert's rows: [d, f]
    g.M = d;
    g.N = f;
    g.P = dy;
    g.Q = h;
    g.G = dw2;
    MOE_LAUNCH(launch_grad_w(g, bf16, stream));
  }
  // dA = dH SiLU'(A), in place (an elementwise pass: measured faster than multiplying in the GEMM's
  // epilogue, whose reads of A wait a round trip per 16-row block)
  MOE_LAUNCH(launch_silu_bwd(dh, a1, dh, offsets + E, c.T * c.top_k, f, bf16, stream));
  MOE_TRY(run_gemm_kn(c, dh, w1, w1t, dxp, offsets, d, f, sk, stream));   // dXp = dA W1_e
  if (dw1) {   // dW1_e = dA^T Xp over the expert's rows: [f, d]
    g.M = f;
    g.N = d;
    g.P = dh;
    g.Q = xp;
    g.G = dw1;
    MOE_LAUNCH(launch_grad_w(g, bf16, stream));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t status) {
  switch (enum_int(status)) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

moe_status_t moe_validate_config(const moe_config_t* c) {
  if (!c) return MOE_ERR_INVALID_ARGUMENT;
  if (c->T < 1 || c->T > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARGUMENT;
  if (c->d_model < 8 || c->d_model > kMaxDim || c->d_model % 8) return MOE_ERR_INVALID_ARGUMENT;
  if (c->d_ffn < 8 || c->d_ffn > kMaxDim || c->d_ffn % 8) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_experts < 1 || c->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARGUMENT;
  const int kmax = c->num_experts < MOE_MAX_TOP_K ? c->num_experts : MOE_MAX_TOP_K;
  if (c->top_k < 1 || c->top_k > kmax) return MOE_ERR_INVALID_ARGUMENT;
  if (c->capacity < MOE_NO_CAPACITY) return MOE_ERR_INVALID_ARGUMENT;
  if (!(isfinite(c->temperature) && c->temperature > 0.0f)) return MOE_ERR_INVALID_ARGUMENT;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->noise_in_logits != 0 && c->noise_in_logits != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->straight_through != 0 && c->straight_through != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->keep_preact != 0 && c->keep_preact != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->d_ffn_shared < 0 || c->d_ffn_shared > kMaxDim || c->d_ffn_shared % 8) return MOE_ERR_INVALID_ARGUMENT;
  if (!isfinite(c->aux_coef)) return MOE_ERR_INVALID_ARGUMENT;
  const int act = enum_int(c->act_dtype), wt = enum_int(c->weight_dtype);
  const bool dt_ok = (act == MOE_F32 || act == MOE_BF16) && (wt == MOE_F32 || wt == MOE_BF16 || wt == MOE_INT4);
  if (!dt_ok) return MOE_ERR_INVALID_ARGUMENT;
  if (wt == MOE_INT4) {
    // 4-bit weights: bf16 activations, whole groups of four 128-column stages, the
    // weight-streaming regime (at most 64 rows per expert on average), no shared expert
    const bool ok = act == MOE_BF16 && c->d_model % 512 == 0 && c->d_ffn % 512 == 0 &&
                    (long long)c->T * c->top_k <= 64LL * c->num_experts && c->d_ffn_shared == 0 &&
                    c->keep_preact == 0;
    return ok ? MOE_OK : MOE_ERR_UNSUPPORTED;
  }
  if (act != wt) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int32_t moe_capacity_from_factor(int32_t T, int32_t k, int32_t E, int32_t cf_num, int32_t cf_den) {
  if (T <= 0 || k <= 0 || E <= 0 || cf_num <= 0 || cf_den <= 0) return -1;
  const long long num = (long long)cf_num * T * k;
  const long long den = (long long)cf_den * E;
  const long long c = (num + den - 1) / den;
  return c > 0x7fffffffLL ? 0x7fffffff : (int32_t)c;
}

size_t moe_int4_bytes(int64_t rows, int32_t K) {
  if (rows < 16 || rows % 16 || K < 128 || K % 128) return 0;
  return q4_bytes((size_t)rows, K);
}

moe_status_t moe_quantize_int4(int64_t rows, int32_t K, const void* w, void* packed, hipStream_t stream) {
  if (rows < 16 || rows % 16 || K < 128 || K % 128 || K > kMaxDim || !w || !packed || !aligned16(w) ||
      !aligned16(packed))
    return MOE_ERR_INVALID_ARGUMENT;
  MOE_LAUNCH(launch_quantize_q4(w, (size_t)rows, K, packed, stream));
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_config_t* cfg) {
  if (moe_validate_config(cfg) != MOE_OK) return 0;
  return layout(*cfg).total;
}

moe_status_t moe_route(const moe_config_t* cfg, const void* x, const float* w_router, const float* bias,
                       const float* noise, const uint8_t* token_mask, const float* logits_in,
                       float* logits_out, float* probs_out,
                       int32_t* ids, float* weights, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (!ids || !weights) return MOE_ERR_INVALID_ARGUMENT;
  if (!logits_in && (!x || !w_router || !aligned16(x) || !aligned16(w_router))) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  return run_route(*cfg, x, w_router, bias, noise, token_mask, logits_in, logits_out, probs_out, ids, weights, nullptr,
                   stream);
}

moe_status_t moe_dispatch(const moe_config_t* cfg, const int32_t* ids, const void* x, int32_t* counts_pre,
                          int32_t* counts, int32_t* offsets, int32_t* perm_token, int32_t* row_of,
                          uint8_t* dropped, int32_t* n_dropped, void* xp, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (!ids || !x || !counts_pre || !counts || !offsets || !perm_token || !row_of || !dropped || !n_dropped ||
      !xp)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(xp)) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  const Layout L = layout(*cfg);
  HistParams hp{};
  hp.TK = cfg->T * cfg->top_k;
  hp.E = cfg->num_experts;
  hp.k = cfg->top_k;
  hp.bt = DISPATCH_BLOCK_TOKENS;
  hp.ids = ids;
  hp.blk_hist = (int32_t*)at(ws, L.blk_hist);
  MOE_LAUNCH(launch_hist(hp, stream));
  return run_dispatch(*cfg, DISPATCH_BLOCK_TOKENS, ids, x, counts_pre, counts, offsets, n_dropped, perm_token,
                      row_of, dropped, xp, ws, nullptr, nullptr, [] { return MOE_OK; }, stream);
}

moe_status_t moe_expert_ffn(const moe_config_t* cfg, const void* xp, const int32_t* offsets, const void* w1,
                            const void* w2, void* h, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (!xp || !offsets || !w1 || !w2 || !h || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(xp) || !aligned16(w1) || !aligned16(w2) || !aligned16(h) || !aligned16(y))
    return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  MOE_TRY(run_gemm(*cfg, xp, w1, h, offsets, cfg->d_ffn, cfg->d_model, true, ws, stream));
  return run_gemm(*cfg, h, w2, y, offsets, cfg->d_model, cfg->d_ffn, false, ws, stream);
}

moe_status_t moe_combine(const moe_config_t* cfg, const void* y, const int32_t* row_of, const float* weights,
                         const void* y_shared, void* out, hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (!y || !row_of || !weights || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y) || !aligned16(out) || (y_shared && !aligned16(y_shared))) return MOE_ERR_INVALID_ARGUMENT;
  return run_combine(*cfg, y, row_of, weights, y_shared, out, stream);
}

moe_status_t moe_aux_loss(const moe_config_t* cfg, const float* probs, const float* logits,
                          const uint8_t* token_mask, const int32_t* counts_pre, float* aux, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if ((!probs && !logits) || !counts_pre || !aux) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  const Layout L = layout(*cfg);
  ProbSumParams p{};
  p.T = cfg->T;
  p.E = cfg->num_experts;
  p.tau = cfg->temperature;
  p.probs = probs;
  p.logits = logits;
  p.token_mask = token_mask;
  p.psum = (double*)at(ws, L.probsum);
  MOE_LAUNCH(launch_probsum(p, stream));
  return run_aux_final(*cfg, p.psum, probsum_num_blocks(cfg->T), counts_pre, aux, stream);
}

moe_status_t moe_forward(const moe_config_t* cfg, const void* x, const float* w_router, const float* bias,
                         const float* noise, const uint8_t* token_mask, const void* w1, const void* w2,
                         const void* w1_shared, const void* w2_shared, void* out, float* aux,
                         moe_debug_outputs* dbg, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(forward_args_status(cfg, x, w_router, w1, w2, w1_shared, w2_shared, out, aux));
  const bool shared = cfg->d_ffn_shared > 0;
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  moe_debug_outputs none{};
  const moe_debug_outputs& D = dbg ? *dbg : none;
  if (D.events && D.n_events < MOE_FORWARD_NUM_KERNELS + 1) return MOE_ERR_INVALID_ARGUMENT;
  if ((D.xp && !aligned16(D.xp)) || (D.h && !aligned16(D.h)) || (D.y && !aligned16(D.y)) ||
      (D.y_shared && !aligned16(D.y_shared)))
    return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout(*cfg);
  const moe_config_t& c = *cfg;
  auto pick = [&](void* user, size_t off) { return user ? user : (void*)at(ws, off); };
  float* logits = (float*)pick(D.logits, L.logits);   // kept for moe_backward
  float* probs = D.probs;
  int32_t* ids = (int32_t*)pick(D.ids, L.ids);
  float* weights = (float*)pick(D.weights, L.weights);
  int32_t* counts_pre = (int32_t*)pick(D.counts_pre, L.counts_pre);
  int32_t* counts = (int32_t*)pick(D.counts, L.counts);
  int32_t* offsets = (int32_t*)pick(D.offsets, L.offsets);
  int32_t* perm = (int32_t*)pick(D.perm_token, L.perm);
  int32_t* row_of = (int32_t*)pick(D.row_of, L.row_of);
  uint8_t* dropped = (uint8_t*)pick(D.dropped, L.dropped);
  int32_t* ndrop = (int32_t*)pick(D.n_dropped, L.ndrop);
  void* xp = pick(D.xp, L.xp);
  void* h = pick(D.h, L.h);
  void* y = pick(D.y, L.y);
  double* psum = (double*)at(ws, L.psum);
  int ev = 0;
  auto mark = [&]() -> moe_status_t {
    if (!D.events) return MOE_OK;
    return hip_status(hipEventRecord(D.events[ev++], stream));
  };
  MOE_TRY(mark());
  // the router also counts each of its token groups' selections per expert (the dispatch histogram)
  MOE_TRY(run_route(c, x, w_router, bias, noise, token_mask, nullptr, logits, probs, ids, weights, psum, stream,
                    (int32_t*)at(ws, L.blk_hist)));
  MOE_TRY(mark());
  MOE_TRY(mark());   // no separate histogram step
  const AuxParams ap =
      aux_params(c, psum, route_num_parts(c.T, c.num_experts, c.act_dtype == MOE_BF16, false), counts_pre, aux);
  int32_t* sh_off = shared ? (int32_t*)at(ws, L.sh_off) : nullptr;
  MOE_TRY(run_dispatch(c, route_block_tokens(c.T, c.num_experts, c.act_dtype == MOE_BF16, false), ids, x, counts_pre,
                       counts, offsets, ndrop, perm, row_of, dropped, xp, ws, &ap, sh_off, mark, stream));
  MOE_TRY(mark());
  MOE_TRY(run_gemm(c, xp, w1, h, offsets, c.d_ffn, c.d_model, true, ws, stream, -1, -1,
                   c.keep_preact ? at(ws, L.a1) : nullptr));
  MOE_TRY(mark());
  MOE_TRY(run_gemm(c, h, w2, y, offsets, c.d_model, c.d_ffn, false, ws, stream));
  MOE_TRY(mark());
  void* ys = nullptr;
  if (shared) {   // one segment of all T tokens, straight from x
    void* hs = at(ws, L.hs);
    ys = pick(D.y_shared, L.ys);
    MOE_TRY(run_gemm(c, x, w1_shared, hs, sh_off, c.d_ffn_shared, c.d_model, true, ws, stream, 1, c.T));
    MOE_TRY(run_gemm(c, hs, w2_shared, ys, sh_off, c.d_model, c.d_ffn_shared, false, ws, stream, 1, c.T));
  }
  MOE_TRY(mark());
  MOE_TRY(run_combine(c, y, row_of, weights, ys, out, stream));
  MOE_TRY(mark());
  return MOE_OK;
}

}  // extern "C"

// ---- the forward without a caller workspace

// The no-allocation variant's workspace: one array per GPU the library runs on, held until the
// process ends. In host code this name only stands in for the array; its device address comes
// from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up on the first call on that device.
moe_status_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_forward_noalloc_max_bytes(void) { return (size_t)MOE_NOALLOC_SCRATCH_BYTES; }

moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const void* x, const float* w_router, const float* bias,
                                 const float* noise, const uint8_t* token_mask, const void* w1, const void* w2,
                                 const void* w1_shared, const void* w2_shared, void* out, float* aux,
                                 hipStream_t stream) {
  // every argument is checked before anything touches the GPU; a layer whose workspace is larger
  // than the array is rejected
  MOE_TRY(forward_args_status(cfg, x, w_router, w1, w2, w1_shared, w2_shared, out, aux));
  if (layout(*cfg).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  MOE_TRY(scratch_of_current_device(&ws));
  // the same kernels as moe_forward, on the array's memory; no step needs it cleared first (each
  // kernel writes every workspace element that a later one reads)
  return moe_forward(cfg, x, w_router, bias, noise, token_mask, w1, w2, w1_shared, w2_shared, out, aux, nullptr,
                     ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

// ---- backward pass

size_t moe_backward_workspace_bytes(const moe_config_t* cfg) {
  if (moe_validate_config(cfg) != MOE_OK) return 0;
  return bwd_layout(*cfg).total;
}

moe_status_t moe_combine_backward(const moe_config_t* cfg, const void* d_out, const void* y, const int32_t* row_of,
                                  const float* weights, void* dy, float* dweights, hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (!d_out || !y || !row_of || !weights || !dy || !dweights) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(d_out) || !aligned16(y) || !aligned16(dy)) return MOE_ERR_INVALID_ARGUMENT;
  CombineBwdParams p{};
  p.T = cfg->T;
  p.d = cfg->d_model;
  p.k = cfg->top_k;
  p.max_rows = cfg->T * cfg->top_k;
  p.d_out = d_out;
  p.y = y;
  p.row_of = row_of;
  p.weights = weights;
  p.dy = dy;
  p.dweights = dweights;
  MOE_LAUNCH(launch_combine_bwd(p, cfg->act_dtype == MOE_BF16, stream));
  return MOE_OK;
}

moe_status_t moe_expert_ffn_backward(const moe_config_t* cfg, const void* xp, const int32_t* offsets,
                                     const void* w1, const void* w2, const void* h, const void* dy, void* dxp,
                                     float* dw1, float* dw2, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (cfg->weight_dtype == MOE_INT4) return MOE_ERR_UNSUPPORTED;
  if (!xp || !offsets || !w1 || !w2 || !dy || !dxp || !ws || (dw2 && !h)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(xp) || !aligned16(w1) || !aligned16(w2) || !aligned16(dy) || !aligned16(dxp) || !aligned16(ws) ||
      (h && !aligned16(h)))
    return MOE_ERR_INVALID_ARGUMENT;
  const BwdLayout L = bwd_layout(*cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return expert_ffn_bwd(*cfg, L, xp, offsets, w1, w2, h, dy, dxp, dw1, dw2, ws, stream);
}

moe_status_t moe_dispatch_backward(const moe_config_t* cfg, const void* dxp, const int32_t* row_of, void* dx,
                                   hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (!dxp || !row_of || !dx || !aligned16(dxp) || !aligned16(dx)) return MOE_ERR_INVALID_ARGUMENT;
  return run_combine(*cfg, dxp, row_of, nullptr, nullptr, dx, stream);
}

moe_status_t moe_route_backward(const moe_config_t* cfg, const void* x, const float* w_router, const float* logits,
                                const int32_t* ids, const float* weights, const float* dweights,
                                const int32_t* counts_pre, const uint8_t* token_mask, float d_aux, float* dlogits,
                                void* dx, float* dw_router, float* dbias, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  if (!logits || !ids || !weights || !dweights || !dlogits || !isfinite(d_aux)) return MOE_ERR_INVALID_ARGUMENT;
  if (d_aux != 0.0f && !counts_pre) return MOE_ERR_INVALID_ARGUMENT;
  if ((dx && (!w_router || !aligned16(dx))) || (dw_router && (!x || !aligned16(x) || !ws || !aligned16(ws))))
    return MOE_ERR_INVALID_ARGUMENT;
  const moe_config_t& c = *cfg;
  const BwdLayout L = bwd_layout(c);
  if (dw_router && ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  RouteBwdParams p{};
  p.T = c.T;
  p.d = c.d_model;
  p.E = c.num_experts;
  p.k = c.top_k;
  p.tau = c.temperature;
  p.coef = c.aux_coef;
  p.d_aux = d_aux;
  p.renormalize = c.renormalize && !c.straight_through;   // the estimator: full-softmax gradient
  p.x = x;
  p.w_router = w_router;
  p.logits = logits;
  p.ids = ids;
  p.weights = weights;
  p.dweights = dweights;
  p.counts_pre = d_aux != 0.0f ? counts_pre : nullptr;
  p.token_mask = token_mask;
  p.dlogits = dlogits;
  p.dx = dx;
  p.dw_router = dw_router;
  p.dbias = dbias;
  p.part = dw_router ? (float*)at(ws, L.rw_part) : nullptr;
  MOE_LAUNCH(launch_route_bwd(p, c.act_dtype == MOE_BF16, stream));
  return MOE_OK;
}

moe_status_t moe_backward(const moe_config_t* cfg, const void* x, const float* w_router, const uint8_t* token_mask,
                          const void* w1, const void* w2, const void* w1_shared, const void* w2_shared,
                          const void* d_out, float d_aux, const void* fwd_ws, size_t fwd_ws_bytes, void* dx,
                          float* dw_router, float* dbias, float* dw1, float* dw2, float* dw1_shared,
                          float* dw2_shared, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(moe_validate_config(cfg));
  const moe_config_t& c = *cfg;
  if (c.weight_dtype == MOE_INT4) return MOE_ERR_UNSUPPORTED;
  const bool shared = c.d_ffn_shared > 0;
  if (!x || !w_router || !w1 || !w2 || !d_out || !fwd_ws || !dx || !ws || !isfinite(d_aux))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w1) || !aligned16(w2) || !aligned16(d_out) ||
      !aligned16(fwd_ws) || !aligned16(dx) || !aligned16(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (shared && (!w1_shared || !w2_shared || !aligned16(w1_shared) || !aligned16(w2_shared)))
    return MOE_ERR_INVALID_ARGUMENT;
  const Layout F = layout(c);
  const BwdLayout L = bwd_layout(c);
  if (fwd_ws_bytes < F.total || ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const bool bf16 = c.act_dtype == MOE_BF16;
  const int T = c.T, d = c.d_model;
  void* fw = const_cast<void*>(fwd_ws);   // read only
  const float* logits = (const float*)at(fw, F.logits);
  const int32_t* ids = (const int32_t*)at(fw, F.ids);
  const float* weights = (const float*)at(fw, F.weights);
  const int32_t* counts_pre = (const int32_t*)at(fw, F.counts_pre);
  const int32_t* offsets = (const int32_t*)at(fw, F.offsets);
  const int32_t* row_of = (const int32_t*)at(fw, F.row_of);
  const void* xp = at(fw, F.xp);
  const void* h = at(fw, F.h);
  const void* y = at(fw, F.y);
  void* dy = at(ws, L.dy);
  float* dwts = (float*)at(ws, L.dwts);
  void* dxp = at(ws, L.dxp);
  float* dlogits = (float*)at(ws, L.dlogits);
  // combine: dY = w dOut on each kept slot's row, dw = <dOut, Y>
  CombineBwdParams cp{};
  cp.T = T;
  cp.d = d;
  cp.k = c.top_k;
  cp.max_rows = T * c.top_k;
  cp.d_out = d_out;
  cp.y = y;
  cp.row_of = row_of;
  cp.weights = weights;
  cp.dy = dy;
  cp.dweights = dwts;
  MOE_LAUNCH(launch_combine_bwd(cp, bf16, stream));
  // routed experts
  MOE_TRY(expert_ffn_bwd(c, L, xp, offsets, w1, w2, h, dy, dxp, dw1, dw2, ws, stream,
                         c.keep_preact ? at(fw, F.a1) : nullptr));
  // shared expert: one segment of all T tokens; its output joined every token's with weight 1
  void* dxs = nullptr;
  if (shared) {
    const int fs = c.d_ffn_shared;
    const int32_t* sh_off = (const int32_t*)at(fw, F.sh_off);
    const void* hs = at(fw, F.hs);
    void* w1st = at(ws, L.w1st);   // [d, fs]
    void* w2st = at(ws, L.w2st);   // [fs, d]
    void* as = at(ws, L.as);       // [T, fs] pre-activation x W1s^T (recomputed)
    void* dhs = at(ws, L.dhs);     // [T, fs] dHs, then dAs in place
    void* sk = at(ws, L.sk_part);
    dxs = at(ws, L.dxs);
    MOE_TRY(run_gemm_sk(c, x, w1_shared, as, sh_off, fs, d, false, sk, stream, 1, T, false, nullptr, true));
    MOE_TRY(run_gemm_kn(c, d_out, w2_shared, w2st, dhs, sh_off, fs, d, sk, stream, 1, T));
    GradWParams g{};
    g.E = 1;
    g.max_rows = T;
    g.offsets = sh_off;
    if (dw2_shared) {   // dW2s = dOut^T Hs: [d, fs]
      g.M = d;
      g.N = fs;
      g.P = d_out;
      g.Q = hs;
      g.G = dw2_shared;
      MOE_LAUNCH(launch_grad_w(g, bf16, stream));
    }
    MOE_LAUNCH(launch_silu_bwd(dhs, as, dhs, sh_off + 1, T, fs, bf16, stream));
    MOE_TRY(run_gemm_kn(c, dhs, w1_shared, w1st, dxs, sh_off, d, fs, sk, stream, 1, T));
    if (dw1_shared) {   // dW1s = dAs^T x: [fs, d]
      g.M = fs;
      g.N = d;
      g.P = dhs;
      g.Q = x;
      g.G = dw1_shared;
      MOE_LAUNCH(launch_grad_w(g, bf16, stream));
    }
  }
  // gather backward (plus the shared expert's dx) and the router's share: one pass that writes dx
  // where the router backward can form it from the rows (route_bwd_fuses_gather), else the gather
  // first and the router's share added to dx
  const bool fused = route_bwd_fuses_gather(bf16, c.num_experts, c.top_k);
  if (!fused) MOE_TRY(run_combine(c, dxp, row_of, nullptr, dxs, dx, stream));
  RouteBwdParams p{};
  p.T = T;
  p.d = d;
  p.E = c.num_experts;
  p.k = c.top_k;
  p.tau = c.temperature;
  p.coef = c.aux_coef;
  p.d_aux = d_aux;
  p.renormalize = c.renormalize && !c.straight_through;   // the estimator: full-softmax gradient
  p.x = x;
  p.w_router = w_router;
  p.logits = logits;
  p.ids = ids;
  p.weights = weights;
  p.dweights = dwts;
  p.counts_pre = counts_pre;
  p.token_mask = token_mask;
  p.dlogits = dlogits;
  p.dx = dx;
  p.dw_router = dw_router;
  p.dbias = dbias;
  p.part = dw_router ? (float*)at(ws, L.rw_part) : nullptr;
  if (fused) {
    p.dxp = dxp;
    p.row_of = row_of;
    p.max_rows = T * c.top_k;
    p.dxs = dxs;
  }
  MOE_LAUNCH(launch_route_bwd(p, bf16, stream));
  return MOE_OK;
}

}  // extern "C"
