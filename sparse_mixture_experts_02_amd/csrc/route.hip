// Router kernels: logits = x W_r^T + b on MFMA, selection key, wavefront top-k, gate weights,
// full softmax and partial probability sums (per workgroup or per wave) for the aux loss -- one pass
// over x.
//
// [P2 §3.1] scores = W_router x, probs = softmax(scores / tau), top-k (k = 2); with Gumbel
// noise the ranked value is (logits + g) / tau. [P4 §2.4] a linear router with softmax, the
// top-k experts per token, weights = softmax router scores.
//
// bf16 activations: each fp32 router weight w is split into three bf16 values hi + mid + lo
// (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid); the residual is below 2^-26 |w|),
// so x W_r^T = x hi^T + x mid^T + x lo^T runs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16) with
// exact products and fp32 accumulation. fp32 activations use v_mfma_f32_16x16x4_f32.
//
// Lane layout of a 16x16 MFMA result: lane l holds rows 4*(l/16) .. 4*(l/16)+3 of column l%16.
// Rows are tokens and columns are experts, so the 16 lanes of a row group hold all (up to 16)
// experts of 4 tokens: top-k and softmax are reductions over those 16 lanes (DPP moves within
// the row), with more experts held in extra registers (ET tiles of 16).
//
// Two kernels compute the logits:
//  * route_ksplit_kernel (bf16): an 8-wave workgroup routes 1, 2 or 4 tiles of 16 tokens, each
//    wave over its own range of K, with x and the fp32 weight read straight from global memory (the weight is split
//    into its planes in registers, so no separate split pass and no staged copy of the weight).
//  * route_kernel (fp32 activations, or given logits): one wave per 32 tokens, operands straight
//    from global memory.
#include "moe_internal.h"

namespace moe {

// Order-preserving map of a finite fp32 key to uint32 (larger key -> larger code), with -0.0
// and +0.0 mapped to the same code. Every finite key maps above 0, so 0 marks "not a candidate".
__device__ __forceinline__ uint32_t key_code(float key) {
  uint32_t u = __float_as_uint(key);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Reductions over the 16 lanes of a row (one token's experts) with DPP moves, so the data stays in
// the vector registers: partners lane ^ 1 and lane ^ 2 (quad permutes), then the mirror within
// each half row (lane i of 8 with 7 - i) and within the row (i of 16 with 15 - i). Each step
// combines a value with its partner's by a commutative op, so every lane of the row ends with the
// same bits.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f32<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f32<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp_f32<DPP_MIRROR>(v));
}

__device__ __forceinline__ float row16_sum(float v) {
  v = __fadd_rn(v, dpp_f32<DPP_XOR1>(v));
  v = __fadd_rn(v, dpp_f32<DPP_XOR2>(v));
  v = __fadd_rn(v, dpp_f32<DPP_HALF_MIRROR>(v));
  return __fadd_rn(v, dpp_f32<DPP_MIRROR>(v));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<DPP_XOR1>(v));
  v = max_u64(v, dpp_u64<DPP_XOR2>(v));
  v = max_u64(v, dpp_u64<DPP_HALF_MIRROR>(v));
  return max_u64(v, dpp_u64<DPP_MIRROR>(v));
}

// Per-lane running sums for the aux statistics: the lane's probabilities of real tokens (its
// expert column of each ET tile) and, in column 0 lanes only, the router entropy of its real
// tokens and their count.
template <int ET>
struct RouteStats {
  double p[ET];
  double ent, cnt;
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int et = 0; et < ET; ++et) p[et] = 0.0;
    ent = 0.0;
    cnt = 0.0;
  }
};

// Routing of one 16-token MFMA tile whose logits (before the bias) are in acc[et]: lane l holds
// tokens t16 + 4*(l/16) + r, r = 0..3, for expert et*16 + l%16. Adds the bias (and the additive
// noise in that mode), forms the keys, selects the top-k, computes the gate weights,
// probabilities and entropy, writes the outputs and adds the statistics of real tokens to st.
// Padding tokens (token_mask 0) are not routed: ids -1, weights 0, probabilities 0. cnt[et] counts
// the lane's selections (expert et * 16 + l % 16 over its 4 tokens), for the dispatch histogram.
template <int ET>
__device__ __forceinline__ void finish_tile(const RouteParams& p, f32x4_t (&acc)[ET], int t16, bool add_bias,
                                            RouteStats<ET>& st, int (&cnt)[ET]) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int T = p.T, E = p.E, K = p.k;
  const bool additive = p.noise_in_logits && p.gumbel && add_bias;   // computed logits only
  if (add_bias && p.bias) {
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      const int e = et * 16 + col;
      const float b = (e < E) ? p.bias[e] : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[et][r] = __fadd_rn(acc[et][r], b);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t16 + 4 * grp + r;
    const bool in_range = t < T;
    const bool real = in_range && (!p.token_mask || p.token_mask[t] != 0);
    float L[ET];
    bool valid[ET];
    uint64_t pk[ET];
    int slot[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      const int e = et * 16 + col;
      const bool ok = in_range && e < E;
      L[et] = acc[et][r];
      if (additive && ok) L[et] = __fadd_rn(L[et], p.gumbel[(size_t)t * E + e]);
      valid[et] = real && e < E;
      slot[et] = -1;
      float key = L[et];
      if (p.gumbel && !p.noise_in_logits && valid[et])
        key = __fdiv_rn(__fadd_rn(L[et], p.gumbel[(size_t)t * E + e]), p.tau);
      pk[et] = valid[et] ? (((uint64_t)key_code(key) << 8) | (uint64_t)(255 - e)) : 0ull;
      if (ok && p.logits_out) p.logits_out[(size_t)t * E + e] = L[et];
    }
    // k rounds of "largest remaining key": a max over the 16 lanes of the group; the low byte
    // (255 - expert) makes the lowest expert index win equal keys.
    for (int j = 0; j < K; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int et = 0; et < ET; ++et) best = max_u64(best, pk[et]);
      best = row16_max_u64(best);
#pragma unroll
      for (int et = 0; et < ET; ++et)
        if (best != 0ull && pk[et] == best) {
          pk[et] = 0ull;
          slot[et] = j;
        }
    }
#pragma unroll
    for (int et = 0; et < ET; ++et) cnt[et] += slot[et] >= 0 ? 1 : 0;
    // full softmax of logits / tau (probs, aux sums, entropy, unnormalised weights) and the
    // softmax restricted to the selected experts (normalised weights). Exponents are formed as
    // (L - max) / tau, subtracting before scaling.
    float mx_all = -INFINITY, mx_sel = -INFINITY;
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      if (valid[et]) mx_all = fmaxf(mx_all, L[et]);
      if (slot[et] >= 0) mx_sel = fmaxf(mx_sel, L[et]);
    }
    mx_all = row16_max(mx_all);
    mx_sel = row16_max(mx_sel);
    float z[ET], ex_all[ET], ex_sel[ET];
    float s_all = 0.0f, s_sel = 0.0f;
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      z[et] = valid[et] ? __fdiv_rn(__fsub_rn(L[et], mx_all), p.tau) : 0.0f;
      ex_all[et] = valid[et] ? expf(z[et]) : 0.0f;
      ex_sel[et] = (slot[et] >= 0) ? expf(__fdiv_rn(__fsub_rn(L[et], mx_sel), p.tau)) : 0.0f;
      s_all = __fadd_rn(s_all, ex_all[et]);
      s_sel = __fadd_rn(s_sel, ex_sel[et]);
    }
    s_all = row16_sum(s_all);
    s_sel = row16_sum(s_sel);
    // entropy -sum p ln p = ln s - sum p z, with ln p = z - ln s (no logarithm of a small p)
    float pz = 0.0f;
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      const int e = et * 16 + col;
      if (in_range && !real && col < K && et == 0) {   // padding token: no selection in any slot
        p.ids[(size_t)t * K + col] = -1;
        p.weights[(size_t)t * K + col] = 0.0f;
      }
      if (in_range && e < E && !real && p.probs_out) p.probs_out[(size_t)t * E + e] = 0.0f;
      if (!valid[et]) continue;
      const float prob = __fdiv_rn(ex_all[et], s_all);
      pz = __fadd_rn(pz, prob * z[et]);
      if (p.probs_out) p.probs_out[(size_t)t * E + e] = prob;
      st.p[et] += (double)prob;
      if (slot[et] >= 0) {
        const float w = p.straight_through ? 1.0f : (p.renormalize ? __fdiv_rn(ex_sel[et], s_sel) : prob);
        p.ids[(size_t)t * K + slot[et]] = e;
        p.weights[(size_t)t * K + slot[et]] = w;
      }
    }
    pz = row16_sum(pz);
    if (real && col == 0) {
      st.ent += (double)__fsub_rn(logf(s_all), pz);
      st.cnt += 1.0;
    }
  }
}

// Row of the aux statistics of one part: [E] probability sums, entropy sum, real-token count.
__host__ __device__ constexpr int psum_row(int E) { return E + 2; }

// Adds the 4 row groups of a wave (fixed order) and stores the wave's statistics row.
template <int ET>
__device__ __forceinline__ void store_psum(const RouteParams& p, RouteStats<ET>& st, int part) {
  if (!p.psum) return;
  const int lane = threadIdx.x & 63;
  double* row = p.psum + (size_t)part * psum_row(p.E);
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    double v = st.p[et];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    const int e = et * 16 + (lane & 15);
    if (lane < 16 && e < p.E) row[e] = v;
  }
  double h = st.ent, c = st.cnt;
  h += __shfl_xor(h, 16);
  h += __shfl_xor(h, 32);
  c += __shfl_xor(c, 16);
  c += __shfl_xor(c, 32);
  if (lane == 0) {
    row[p.E] = h;
    row[p.E + 1] = c;
  }
}

// Sums a wave's selection counts over its 4 row groups: lane l < 16 then holds the count of expert
// et * 16 + l in cnt[et].
template <int ET>
__device__ __forceinline__ void reduce_counts(int (&cnt)[ET]) {
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    cnt[et] += __shfl_xor(cnt[et], 16);
    cnt[et] += __shfl_xor(cnt[et], 32);
  }
}

// ------------------------------------------------------------------------------ generic kernel

template <int ET>
__global__ __launch_bounds__(64) void route_kernel(RouteParams p) {
  const int lane = threadIdx.x;
  const int col = lane & 15;   // expert column within a 16-wide tile
  const int grp = lane >> 4;   // row group
  const int T = p.T, E = p.E, d = p.d;
  const int ntiles = (T + ROUTE_TILE - 1) / ROUTE_TILE;

  RouteStats<ET> st;
  st.clear();

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t0 = tile * ROUTE_TILE;
    f32x4_t acc[2][ET];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[mt][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (p.logits_in) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = t0 + mt * 16 + 4 * grp + r;
            const int e = et * 16 + col;
            acc[mt][et][r] = (t < T && e < E) ? p.logits_in[(size_t)t * E + e] : 0.0f;
          }
    } else {
      const float* __restrict__ x = (const float*)p.x;
      const float* __restrict__ wr = p.w_router;
      const int row0 = t0 + col;
      const int row1 = t0 + 16 + col;
#pragma unroll 4
      for (int k0 = 0; k0 < d; k0 += 4) {
        const int kc = k0 + grp;   // d is a multiple of 8, so kc < d always
        const float a0 = (row0 < T) ? x[(size_t)row0 * d + kc] : 0.0f;
        const float a1 = (row1 < T) ? x[(size_t)row1 * d + kc] : 0.0f;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const int e = et * 16 + col;
          const float b = (e < E) ? wr[(size_t)e * d + kc] : 0.0f;
          acc[0][et] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b, acc[0][et], 0, 0, 0);
          acc[1][et] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b, acc[1][et], 0, 0, 0);
        }
      }
    }
    int cnt[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) cnt[et] = 0;
    finish_tile<ET>(p, acc[0], t0, !p.logits_in, st, cnt);
    finish_tile<ET>(p, acc[1], t0 + 16, !p.logits_in, st, cnt);
    if (p.blk_hist) {   // the tile is one block of the dispatch histogram
      reduce_counts<ET>(cnt);
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const int e = et * 16 + lane;
        if (lane < 16 && e < E) p.blk_hist[(size_t)tile * E + e] = cnt[et];
      }
    }
  }
  store_psum<ET>(p, st, blockIdx.x);
}

// ------------------------------------------------------------------------------ K-split kernel

namespace {
constexpr int KS_WAVES = 8;             // waves per workgroup, each taking one K range
constexpr int KS_MAX_BLOCKS = 2048;     // grid cap (one row of probability sums per workgroup)

// hi + mid + lo split of 8 fp32 router weights into three bf16x8 MFMA operands (the products with
// bf16 activations are exact in fp32, and hi + mid + lo equals w to within 2^-26 |w|)
__device__ __forceinline__ void split3(const float4& a, const float4& b, bf16x8_t& hi, bf16x8_t& mid, bf16x8_t& lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    const float r0 = __fsub_rn(v[2 * i], bf16_bits_to_f32(h[i] & 0xffffu));
    const float r1 = __fsub_rn(v[2 * i + 1], bf16_bits_to_f32(h[i] >> 16));
    m[i] = pack_bf16x2(r0, r1);
    const float q0 = __fsub_rn(r0, bf16_bits_to_f32(m[i] & 0xffffu));
    const float q1 = __fsub_rn(r1, bf16_bits_to_f32(m[i] >> 16));
    l[i] = pack_bf16x2(q0, q1);
  }
  hi = __builtin_bit_cast(bf16x8_t, uint4{h[0], h[1], h[2], h[3]});
  mid = __builtin_bit_cast(bf16x8_t, uint4{m[0], m[1], m[2], m[3]});
  lo = __builtin_bit_cast(bf16x8_t, uint4{l[0], l[1], l[2], l[3]});
}
}  // namespace

// bf16 activations, E <= 64. A workgroup of 8 waves routes MT tiles of 16 tokens: wave w
// multiplies them by the router weight over its own range of K (a contiguous run of 32-column
// MFMA steps), reading x and the fp32 weight straight from global memory and splitting the
// weight into its three bf16 planes in registers (once per step for all MT tiles); all loads of a
// batch of steps are issued before its MFMAs. The 8 partial products of each tile meet in LDS and
// wave q adds those of tile q in wave order and finishes it; the probability sums of the MT
// finishing waves are added in wave order. MT > 1 reads each weight element once per 16 MT
// tokens (large T); MT = 1 spreads small T over as many workgroups as possible.
template <int ET, int MT>
__global__ __launch_bounds__(512) void route_ksplit_kernel(RouteParams p) {
  static_assert(MT <= KS_WAVES, "one finishing wave per tile");
  constexpr int NB = (ET * (MT + 2) <= 6) ? 4 : ((ET * (MT + 2) <= 12) ? 2 : 1);   // k-steps per load batch
  __shared__ f32x4_t red[KS_WAVES][MT][ET][64];
  __shared__ double wsum[MT][ET * 16 + 2];
  __shared__ int hc[MT][ET * 16];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = p.T, d = p.d, E = p.E;
  const int nsteps = (d + 31) / 32;
  const int per = (nsteps + KS_WAVES - 1) / KS_WAVES;
  const int s0 = w * per;
  const int s1 = min(nsteps, s0 + per);
  const int col = lane & 15, kq = 8 * (lane >> 4);
  const uint16_t* __restrict__ X = (const uint16_t*)p.x;
  const float* __restrict__ W = p.w_router;

  RouteStats<ET> st;
  st.clear();

  const int ngroups = (T + 16 * MT - 1) / (16 * MT);
  for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int t0 = grp * 16 * MT;
    const uint16_t* __restrict__ xr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xr[mt] = X + (size_t)min(t0 + mt * 16 + col, T - 1) * d;   // rows past T: discarded
    f32x4_t acc[MT][ET];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[mt][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int sb = s0; sb < s1; sb += NB) {
      uint4 xa[NB][MT];
      float4 wv[NB][ET][2];
      // Every load is issued unconditionally from a valid address (column 0 for steps past the
      // range, the last expert for lanes past E) and masked afterwards: loads behind branches
      // make the compiler wait for all outstanding loads at the join.
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int kr = (sb + u) * 32 + kq;
        const bool kin = sb + u < s1 && kr < d;   // d is a multiple of 8: a chunk is all in or all out
        const int kc = kin ? kr : 0;
        // the masks are opaque to the compiler, so it cannot turn the masking back into a branch
        uint32_t mk = kin ? 0xffffffffu : 0u;
        asm volatile("" : "+v"(mk));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint4 v = *(const uint4*)(xr[mt] + kc);
          xa[u][mt] = make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk);
        }
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const int e = et * 16 + col;
          uint32_t mw = (kin && e < E) ? 0xffffffffu : 0u;
          asm volatile("" : "+v"(mw));
          const uint4* src = (const uint4*)(W + (size_t)min(e, E - 1) * d + kc);
          const uint4 w0 = src[0], w1 = src[1];
          wv[u][et][0] = make_float4(__uint_as_float(w0.x & mw), __uint_as_float(w0.y & mw),
                                     __uint_as_float(w0.z & mw), __uint_as_float(w0.w & mw));
          wv[u][et][1] = make_float4(__uint_as_float(w1.x & mw), __uint_as_float(w1.y & mw),
                                     __uint_as_float(w1.z & mw), __uint_as_float(w1.w & mw));
        }
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          bf16x8_t hi, mid, lo;
          split3(wv[u][et][0], wv[u][et][1], hi, mid, lo);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const bf16x8_t A = __builtin_bit_cast(bf16x8_t, xa[u][mt]);
            // smallest plane first
            acc[mt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, lo, acc[mt][et], 0, 0, 0);
            acc[mt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, mid, acc[mt][et], 0, 0, 0);
            acc[mt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, hi, acc[mt][et], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int et = 0; et < ET; ++et) red[w][mt][et][lane] = acc[mt][et];
    __syncthreads();
    if (w < MT) {
      f32x4_t s[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        s[et] = red[0][w][et][lane];
#pragma unroll
        for (int q = 1; q < KS_WAVES; ++q) {
          const f32x4_t v = red[q][w][et][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) s[et][r] = __fadd_rn(s[et][r], v[r]);
        }
      }
      int cnt[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et) cnt[et] = 0;
      finish_tile<ET>(p, s, t0 + 16 * w, true, st, cnt);
      if (p.blk_hist) {
        reduce_counts<ET>(cnt);
#pragma unroll
        for (int et = 0; et < ET; ++et)
          if (lane < 16) hc[w][et * 16 + lane] = cnt[et];
      }
    }
    __syncthreads();   // red is rewritten by the next group
    // the group is one block of the dispatch histogram: its MT tiles' counts (hc is rewritten
    // only after the next group's first barrier, which wave 0 passes after these reads)
    if (p.blk_hist && w == 0) {
      for (int e = lane; e < E; e += 64) {
        int v = 0;
#pragma unroll
        for (int q = 0; q < MT; ++q) v += hc[q][e];
        p.blk_hist[(size_t)grp * E + e] = v;
      }
    }
  }
  if (p.psum) {
    if (w < MT) {
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        double v = st.p[et];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane < 16) wsum[w][et * 16 + lane] = v;
      }
      double h = st.ent, c = st.cnt;
      h += __shfl_xor(h, 16);
      h += __shfl_xor(h, 32);
      c += __shfl_xor(c, 16);
      c += __shfl_xor(c, 32);
      if (lane == 0) {
        wsum[w][ET * 16] = h;
        wsum[w][ET * 16 + 1] = c;
      }
    }
    __syncthreads();
    if (w == 0) {
      double* row = p.psum + (size_t)blockIdx.x * psum_row(E);
      for (int i = lane; i < ET * 16 + 2; i += 64) {
        double v = wsum[0][i];
#pragma unroll
        for (int q = 1; q < MT; ++q) v += wsum[q][i];
        if (i < ET * 16) {
          if (i < E) row[i] = v;
        } else {
          row[E + (i - ET * 16)] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------ host side

int route_expert_tiles(int E) { return (E + 15) / 16; }


static bool use_ksplit(bool bf16, bool logits_in) { return bf16 && !logits_in; }

// Tiles of 16 tokens per K-split workgroup: as many workgroups as possible while they fill the
// chip, more tiles per workgroup (fewer weight re-reads) once there are enough tokens; at most 2
// when E > 32 (LDS of the partial products).
static int ksplit_mt(int T, int E) {
  const int tiles = (T + 15) / 16;
  const int mt = tiles >= 4 * 256 ? 4 : (tiles >= 2 * 256 ? 2 : 1);
  return (route_expert_tiles(E) > 2 && mt > 2) ? 2 : mt;
}

static int ksplit_blocks(int T, int E) {
  const int mt = ksplit_mt(T, E);
  const int n = (T + 16 * mt - 1) / (16 * mt);
  return n < KS_MAX_BLOCKS ? n : KS_MAX_BLOCKS;
}

static int generic_blocks(int T) {
  const int n = (T + ROUTE_TILE - 1) / ROUTE_TILE;
  return n < ROUTE_MAX_WAVES ? n : ROUTE_MAX_WAVES;
}

int route_block_tokens(int T, int E, bool bf16, bool logits_in) {
  return use_ksplit(bf16, logits_in) ? 16 * ksplit_mt(T, E) : ROUTE_TILE;
}

int route_num_parts(int T, int E, bool bf16, bool logits_in) {
  return use_ksplit(bf16, logits_in) ? ksplit_blocks(T, E) : generic_blocks(T);
}

int route_max_parts(int T, int E) {
  const int a = ksplit_blocks(T, E), b = generic_blocks(T);
  return a > b ? a : b;
}

template <int ET>
static void launch_ksplit(const RouteParams& p, hipStream_t s) {
  const int grid = ksplit_blocks(p.T, p.E);
  switch (ksplit_mt(p.T, p.E)) {
    case 1: route_ksplit_kernel<ET, 1><<<grid, 64 * KS_WAVES, 0, s>>>(p); break;
    case 2: route_ksplit_kernel<ET, 2><<<grid, 64 * KS_WAVES, 0, s>>>(p); break;
    default:
      if constexpr (ET <= 2) route_ksplit_kernel<ET, 4><<<grid, 64 * KS_WAVES, 0, s>>>(p);
      break;
  }
}

static hipError_t launch_route_generic(const RouteParams& p, hipStream_t s) {
  const int grid = generic_blocks(p.T);
  switch (route_expert_tiles(p.E)) {
    case 1: route_kernel<1><<<grid, 64, 0, s>>>(p); break;
    case 2: route_kernel<2><<<grid, 64, 0, s>>>(p); break;
    case 3: route_kernel<3><<<grid, 64, 0, s>>>(p); break;
    case 4: route_kernel<4><<<grid, 64, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteParams& p, bool bf16, hipStream_t s) {
  if (use_ksplit(bf16, p.logits_in != nullptr)) {
    switch (route_expert_tiles(p.E)) {
      case 1: launch_ksplit<1>(p, s); break;
      case 2: launch_ksplit<2>(p, s); break;
      case 3: launch_ksplit<3>(p, s); break;
      case 4: launch_ksplit<4>(p, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return launch_route_generic(p, s);
}

}  // namespace moe
