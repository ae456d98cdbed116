// Router kernel: logits = x W_r^T + b on MFMA, selection key, wavefront top-k, gate weights,
// full softmax and per-wave probability sums for the aux loss -- one pass over x.
//
// [P2 §3.1] scores = W_router x, probs = softmax(scores / tau), top-k (k = 2); with Gumbel
// noise the ranked value is (logits + g) / tau. [P4 §2.4] a linear router with softmax, the
// top-k experts per token, weights = softmax router scores.
//
// bf16 activations: W_r (fp32) is split once per call into three bf16 planes hi + mid + lo
// (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid); the residual is below 2^-26 |w|),
// so x W_r^T = x hi^T + x mid^T + x lo^T runs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16) with
// exact products and fp32 accumulation. fp32 activations use v_mfma_f32_16x16x4_f32.
//
// Lane layout of a 16x16 MFMA result: lane l holds rows 4*(l/16) .. 4*(l/16)+3 of column l%16.
// Rows are tokens and columns are experts, so the 16 lanes of a row group hold all (up to 16)
// experts of 4 tokens: top-k and softmax are reductions over those 16 lanes (xor 1, 2, 4, 8),
// with more experts held in extra registers (ET tiles of 16).
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void route_split_kernel(const float* __restrict__ w, int E, int EP,
                                                          int d, uint16_t* __restrict__ out) {
  const size_t n = (size_t)EP * d;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / d);
    const float v = (e < E) ? w[i] : 0.0f;  // [EP, d] and [E, d] share the row stride d
    const uint32_t hi = f32_to_bf16_bits(v);
    const float r1 = __fsub_rn(v, bf16_bits_to_f32(hi));
    const uint32_t mid = f32_to_bf16_bits(r1);
    const float r2 = __fsub_rn(r1, bf16_bits_to_f32(mid));
    const uint32_t lo = f32_to_bf16_bits(r2);
    out[i] = (uint16_t)hi;
    out[n + i] = (uint16_t)mid;
    out[2 * n + i] = (uint16_t)lo;
  }
}

// Order-preserving map of a finite fp32 key to uint32 (larger key -> larger code), with -0.0
// and +0.0 mapped to the same code. Every finite key maps above 0, so 0 marks "not a candidate".
__device__ __forceinline__ uint32_t key_code(float key) {
  uint32_t u = __float_as_uint(key);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <bool BF16, int ET>
__global__ __launch_bounds__(64) void route_kernel(RouteParams p) {
  const int lane = threadIdx.x;
  const int col = lane & 15;   // expert column within a 16-wide tile
  const int grp = lane >> 4;   // row group: tokens 4*grp .. 4*grp+3 of a 16-token tile
  constexpr int EP = 16 * ET;
  const int T = p.T, E = p.E, d = p.d, K = p.k;
  const int ntiles = (T + ROUTE_TILE - 1) / ROUTE_TILE;

  double psum_acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) psum_acc[et] = 0.0;

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
      if constexpr (BF16) {
        const uint16_t* __restrict__ x = (const uint16_t*)p.x;
        const uint16_t* __restrict__ ws = (const uint16_t*)p.wsplit;
        const size_t plane = (size_t)EP * d;
        const int row0 = t0 + col;
        const int row1 = t0 + 16 + col;
#pragma unroll 4
        for (int k0 = 0; k0 < d; k0 += 32) {
          const int kc = k0 + 8 * grp;
          const bool kin = kc < d;
          uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
          if (kin && row0 < T) a0 = *(const uint4*)(x + (size_t)row0 * d + kc);
          if (kin && row1 < T) a1 = *(const uint4*)(x + (size_t)row1 * d + kc);
          const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, a0);
          const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, a1);
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            const size_t wrow = (size_t)(et * 16 + col) * d + kc;
#pragma unroll
            for (int s = 2; s >= 0; --s) {   // smallest plane first
              uint4 b = make_uint4(0, 0, 0, 0);
              if (kin) b = *(const uint4*)(ws + s * plane + wrow);
              const bf16x8_t B = __builtin_bit_cast(bf16x8_t, b);
              acc[0][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc[0][et], 0, 0, 0);
              acc[1][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc[1][et], 0, 0, 0);
            }
          }
        }
      } else {
        const float* __restrict__ x = (const float*)p.x;
        const float* __restrict__ wr = (const float*)p.wsplit;
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
      if (p.bias) {
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const int e = et * 16 + col;
          const float b = (e < E) ? p.bias[e] : 0.0f;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][et][r] = __fadd_rn(acc[mt][et][r], b);
        }
      }
    }

    // ---- per-token routing: 4 row groups each handle one token at a time
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + mt * 16 + 4 * grp + r;
        const bool tok_ok = t < T;
        float L[ET];
        bool valid[ET];
        uint64_t pk[ET];
        int slot[ET];
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const int e = et * 16 + col;
          L[et] = acc[mt][et][r];
          valid[et] = tok_ok && e < E;
          slot[et] = -1;
          float key = L[et];
          if (p.gumbel && valid[et]) key = __fdiv_rn(__fadd_rn(L[et], p.gumbel[(size_t)t * E + e]), p.tau);
          pk[et] = valid[et] ? (((uint64_t)key_code(key) << 8) | (uint64_t)(255 - e)) : 0ull;
          if (valid[et] && p.logits_out) p.logits_out[(size_t)t * E + e] = L[et];
        }
        // k rounds of "largest remaining key": a max over the 16 lanes of the group; the low
        // byte (255 - expert) makes the lowest expert index win equal keys.
        for (int j = 0; j < K; ++j) {
          uint64_t best = 0;
#pragma unroll
          for (int et = 0; et < ET; ++et) best = max_u64(best, pk[et]);
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) best = max_u64(best, __shfl_xor(best, m));
#pragma unroll
          for (int et = 0; et < ET; ++et)
            if (best != 0ull && pk[et] == best) {
              pk[et] = 0ull;
              slot[et] = j;
            }
        }
        // full softmax of logits / tau (for probs, the aux sums and unnormalised weights), and
        // the softmax restricted to the selected experts (normalised weights). Exponents are
        // formed as (L - max) / tau so that the subtraction is done before the scaling.
        float mx_all = -INFINITY, mx_sel = -INFINITY;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          if (valid[et]) mx_all = fmaxf(mx_all, L[et]);
          if (slot[et] >= 0) mx_sel = fmaxf(mx_sel, L[et]);
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          mx_all = fmaxf(mx_all, __shfl_xor(mx_all, m));
          mx_sel = fmaxf(mx_sel, __shfl_xor(mx_sel, m));
        }
        float ex_all[ET], ex_sel[ET];
        float s_all = 0.0f, s_sel = 0.0f;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          ex_all[et] = valid[et] ? expf(__fdiv_rn(__fsub_rn(L[et], mx_all), p.tau)) : 0.0f;
          ex_sel[et] = (slot[et] >= 0) ? expf(__fdiv_rn(__fsub_rn(L[et], mx_sel), p.tau)) : 0.0f;
          s_all = __fadd_rn(s_all, ex_all[et]);
          s_sel = __fadd_rn(s_sel, ex_sel[et]);
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          s_all = __fadd_rn(s_all, __shfl_xor(s_all, m));
          s_sel = __fadd_rn(s_sel, __shfl_xor(s_sel, m));
        }
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const int e = et * 16 + col;
          if (!valid[et]) continue;
          const float prob = __fdiv_rn(ex_all[et], s_all);
          if (p.probs_out) p.probs_out[(size_t)t * E + e] = prob;
          psum_acc[et] += (double)prob;
          if (slot[et] >= 0) {
            const float w = p.renormalize ? __fdiv_rn(ex_sel[et], s_sel) : prob;
            p.ids[(size_t)t * K + slot[et]] = e;
            p.weights[(size_t)t * K + slot[et]] = w;
          }
        }
      }
    }
  }

  if (p.psum) {
    // combine the 4 row groups (fixed order) and store this wave's sums
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      double v = psum_acc[et];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      const int e = et * 16 + col;
      if (grp == 0 && e < E) p.psum[(size_t)blockIdx.x * E + e] = v;
    }
  }
}

int route_num_waves(int T) {
  const int ntiles = (T + ROUTE_TILE - 1) / ROUTE_TILE;
  return ntiles < ROUTE_MAX_WAVES ? ntiles : ROUTE_MAX_WAVES;
}

int route_expert_tiles(int E) { return (E + 15) / 16; }

hipError_t launch_route_split(const float* w_router, int E, int d, void* wsplit, hipStream_t s) {
  const int EP = 16 * route_expert_tiles(E);
  const size_t n = (size_t)EP * d;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  route_split_kernel<<<blocks, 256, 0, s>>>(w_router, E, EP, d, (uint16_t*)wsplit);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_route_t(const RouteParams& p, hipStream_t s) {
  const int grid = route_num_waves(p.T);
  switch (route_expert_tiles(p.E)) {
    case 1: route_kernel<BF16, 1><<<grid, 64, 0, s>>>(p); break;
    case 2: route_kernel<BF16, 2><<<grid, 64, 0, s>>>(p); break;
    case 3: route_kernel<BF16, 3><<<grid, 64, 0, s>>>(p); break;
    case 4: route_kernel<BF16, 4><<<grid, 64, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteParams& p, bool bf16, hipStream_t s) {
  return bf16 ? launch_route_t<true>(p, s) : launch_route_t<false>(p, s);
}

}  // namespace moe
