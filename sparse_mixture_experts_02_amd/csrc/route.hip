// Router kernels: logits = x W_r^T + b on MFMA, selection key, wavefront top-k, gate weights,
// full softmax and partial probability sums (per workgroup or per wave) for the aux loss -- one pass
// over x.
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
//
// Two kernels compute the logits:
//  * route_fast_kernel (bf16, E <= 32): a 4-wave workgroup routes 64 tokens. x rows and the
//    split weight pass through an LDS ring of 128-column chunks (5 stages for E <= 16, 4 for
//    E <= 32), filled with direct global -> LDS loads issued as many chunks ahead as the ring
//    holds, so each weight chunk is read once per 64 tokens and x streams with 48-64 KiB in flight
//    per workgroup.
//  * route_kernel (fp32 activations, E > 32, or given logits): one wave per 32 tokens, operands
//    straight from global memory.
#include "moe_internal.h"

namespace moe {

namespace {
// fast kernel geometry
constexpr int FR_TOK = 64;           // tokens per workgroup tile (16 per wave)
constexpr int FR_COLS = 128;         // columns of x and of the weight per stage
constexpr int FR_ROWB = 256;         // staged bytes per row per stage
// LDS ring depth: as many stages as fit in 160 KiB (5 x 28 KiB for one 16-expert tile, 4 x 40
// KiB for two), so that NSTAGE - 1 chunks of x are in flight per workgroup
template <int ET>
constexpr int fr_nstage() { return ET == 1 ? 5 : 4; }
constexpr int FR_MAX_BLOCKS = 1024;
}  // namespace

__global__ __launch_bounds__(256) void route_split_kernel(const float* __restrict__ w, int E, int EP,
                                                          int d, int dpad, uint16_t* __restrict__ out) {
  const size_t n = (size_t)EP * dpad;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / dpad);
    const int c = (int)(i % dpad);
    const float v = (e < E && c < d) ? w[(size_t)e * d + c] : 0.0f;   // zero padding
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

// Routing of one 16-token MFMA tile whose logits (before the bias) are in acc[et]: lane l holds
// tokens t16 + 4*(l/16) + r, r = 0..3, for expert et*16 + l%16. Adds the bias, forms the keys,
// selects the top-k, computes the gate weights and probabilities, writes the outputs and adds
// each lane's probabilities of valid tokens to psum_acc.
template <int ET>
__device__ __forceinline__ void finish_tile(const RouteParams& p, f32x4_t (&acc)[ET], int t16, bool add_bias,
                                            double (&psum_acc)[ET]) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int T = p.T, E = p.E, K = p.k;
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
    const bool tok_ok = t < T;
    float L[ET];
    bool valid[ET];
    uint64_t pk[ET];
    int slot[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      const int e = et * 16 + col;
      L[et] = acc[et][r];
      valid[et] = tok_ok && e < E;
      slot[et] = -1;
      float key = L[et];
      if (p.gumbel && valid[et]) key = __fdiv_rn(__fadd_rn(L[et], p.gumbel[(size_t)t * E + e]), p.tau);
      pk[et] = valid[et] ? (((uint64_t)key_code(key) << 8) | (uint64_t)(255 - e)) : 0ull;
      if (valid[et] && p.logits_out) p.logits_out[(size_t)t * E + e] = L[et];
    }
    // k rounds of "largest remaining key": a max over the 16 lanes of the group; the low byte
    // (255 - expert) makes the lowest expert index win equal keys.
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
    // full softmax of logits / tau (probs, aux sums, unnormalised weights) and the softmax
    // restricted to the selected experts (normalised weights). Exponents are formed as
    // (L - max) / tau, subtracting before scaling.
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

// Adds the 4 row groups of a wave (fixed order) and stores the wave's per-expert sums.
template <int ET>
__device__ __forceinline__ void store_psum(const RouteParams& p, double (&psum_acc)[ET], int part) {
  if (!p.psum) return;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    double v = psum_acc[et];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    const int e = et * 16 + (lane & 15);
    if (lane < 16 && e < p.E) p.psum[(size_t)part * p.E + e] = v;
  }
}

// ------------------------------------------------------------------------------ generic kernel

template <bool BF16, int ET>
__global__ __launch_bounds__(64) void route_kernel(RouteParams p) {
  const int lane = threadIdx.x;
  const int col = lane & 15;   // expert column within a 16-wide tile
  const int grp = lane >> 4;   // row group
  constexpr int EP = 16 * ET;
  const int T = p.T, E = p.E, d = p.d;
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
        const int dpad = p.dpad;
        const size_t plane = (size_t)EP * dpad;
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
            const size_t wrow = (size_t)(et * 16 + col) * dpad + kc;
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
    }
    finish_tile<ET>(p, acc[0], t0, !p.logits_in, psum_acc);
    finish_tile<ET>(p, acc[1], t0 + 16, !p.logits_in, psum_acc);
  }
  store_psum<ET>(p, psum_acc, blockIdx.x);
}

// ------------------------------------------------------------------------------ fast kernel

namespace {
// One direct global -> LDS 16-byte load per lane (gfx950 global_load_lds_dwordx4): lane l reads
// sbase + voff and writes LDS bytes [lds_addr + 16 l, lds_addr + 16 l + 16). M0 carries the LDS
// address and is restored afterwards. Issued as inline asm so that the compiler does not wait
// on it before unrelated LDS reads; the kernel counts these loads and waits (vmcnt) itself.
__device__ __forceinline__ void route_load_lds16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// staged row r (256 bytes) holds its 16-byte chunk c in slot c ^ (r mod 16): 16 lanes reading 16
// consecutive rows at one chunk hit 16 distinct bank groups
__device__ __forceinline__ int fr_off(int row, int chunk) { return row * FR_ROWB + ((chunk ^ (row & 15)) << 4); }
}  // namespace

template <int ET>
__global__ __launch_bounds__(256, 1) void route_fast_kernel(RouteParams p) {
  constexpr int EP = 16 * ET;
  constexpr int XB = FR_TOK * FR_ROWB;        // x chunk: 64 rows, 16 KiB
  constexpr int WB = 3 * EP * FR_ROWB;        // weight chunk: 3 planes x EP rows, 12 KiB per ET
  constexpr int SB = XB + WB;
  constexpr int XI = 4;                       // x load instructions per wave per stage (16 rows)
  constexpr int WI = 3 * ET;                  // weight load instructions per wave per stage
  constexpr int PER = XI + WI;
  constexpr int NS = fr_nstage<ET>();
  static_assert(NS * SB <= 160 * 1024, "LDS ring too large");
  static_assert((NS - 2) * PER <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, d = p.d, dpad = p.dpad;
  const int nk = dpad / FR_COLS;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const uint8_t* __restrict__ W = (const uint8_t*)p.wsplit;
  const int lr = lane >> 4, ls = lane & 15;   // row within an instruction's 4 rows, slot

  // weight sources of this lane (same for every tile): staged weight row rr = plane * EP + e
  uint32_t woff[WI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int rr = w * (WI * 4) + i * 4 + lr;
    woff[i] = (uint32_t)rr * (uint32_t)(dpad * 2) + ((ls ^ (rr & 15)) << 4);
  }

  double psum_acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) psum_acc[et] = 0.0;

  const int ntiles = (T + FR_TOK - 1) / FR_TOK;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t0 = tile * FR_TOK;
    const uint8_t* __restrict__ X = (const uint8_t*)p.x + (size_t)t0 * d * 2;
    // x sources: staged row = w * 16 + i * 4 + lr; rows past T read token T - 1 (their results
    // are discarded); columns past d read column 0 (the weight is zero there)
    uint32_t xrow[XI];
    int xch[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int row = w * 16 + i * 4 + lr;
      const int tr = min(t0 + row, T - 1) - t0;
      xrow[i] = (uint32_t)tr * (uint32_t)(d * 2);
      xch[i] = ls ^ (row & 15);
    }
    auto issue = [&](int kt) {
      const int st = min(kt, nk - 1);   // past the end: reload the last chunk (uniform counts)
      const uint32_t base = lds0 + (kt % NS) * SB;
#pragma unroll
      for (int i = 0; i < XI; ++i) {
        int c = st * FR_COLS + xch[i] * 8;
        if (c >= d) c = 0;
        route_load_lds16(X, xrow[i] + (uint32_t)c * 2, base + (w * 16 + i * 4) * FR_ROWB);
      }
      const uint8_t* wst = W + (size_t)st * FR_ROWB;
#pragma unroll
      for (int i = 0; i < WI; ++i) route_load_lds16(wst, woff[i], base + XB + (w * (WI * 4) + i * 4) * FR_ROWB);
    };

    f32x4_t acc[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) acc[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int kt = 0; kt < NS - 1; ++kt) issue(kt);
    wait_vmcnt<(NS - 2) * PER>();
    __syncthreads();
    const int arow = w * 16 + (lane & 15);
    for (int s = 0; s < nk; ++s) {
      issue(s + NS - 1);
      const uint8_t* sx = smem + (s % NS) * SB;
      const uint8_t* sw = sx + XB;
#pragma unroll
      for (int ks = 0; ks < FR_COLS / 32; ++ks) {
        const int ch = ks * 4 + (lane >> 4);
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sx + fr_off(arow, ch)));
#pragma unroll
        for (int et = 0; et < ET; ++et) {
#pragma unroll
          for (int pl = 2; pl >= 0; --pl) {   // smallest plane first
            const int wrow = pl * EP + et * 16 + (lane & 15);
            const bf16x8_t B = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sw + fr_off(wrow, ch)));
            acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[et], 0, 0, 0);
          }
        }
      }
      wait_vmcnt<(NS - 2) * PER>();   // chunk s + 1 complete (the NS - 2 after it may be in flight)
      __syncthreads();
    }
    wait_vmcnt<0>();           // the trailing reloads land before the ring is reused
    __syncthreads();
    finish_tile<ET>(p, acc, t0 + w * 16, true, psum_acc);
  }
  // One row of probability sums per workgroup: each wave folds its 4 row groups (as store_psum),
  // the 4 waves' sums meet in LDS (the ring is no longer read: every wave is past the last
  // barrier of the tile loop) and are added in wave order.
  if (p.psum) {
    double* wsum = (double*)smem;   // [4 waves][ET][16]
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      double v = psum_acc[et];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) wsum[(w * ET + et) * 16 + lane] = v;
    }
    __syncthreads();
    if (w == 0 && lane < 16) {
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const int e = et * 16 + lane;
        const double v = ((wsum[(0 * ET + et) * 16 + lane] + wsum[(1 * ET + et) * 16 + lane]) +
                          wsum[(2 * ET + et) * 16 + lane]) +
                         wsum[(3 * ET + et) * 16 + lane];
        if (e < p.E) p.psum[(size_t)blockIdx.x * p.E + e] = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------ host side

int route_expert_tiles(int E) { return (E + 15) / 16; }

int route_padded_d(int d) { return (d + FR_COLS - 1) / FR_COLS * FR_COLS; }

static bool use_fast(int E, bool bf16, bool logits_in) { return bf16 && !logits_in && route_expert_tiles(E) <= 2; }

static int fast_blocks(int T) {
  const int n = (T + FR_TOK - 1) / FR_TOK;
  return n < FR_MAX_BLOCKS ? n : FR_MAX_BLOCKS;
}

static int generic_blocks(int T) {
  const int n = (T + ROUTE_TILE - 1) / ROUTE_TILE;
  return n < ROUTE_MAX_WAVES ? n : ROUTE_MAX_WAVES;
}

int route_num_parts(int T, int E, bool bf16, bool logits_in) {
  return use_fast(E, bf16, logits_in) ? fast_blocks(T) : generic_blocks(T);
}

int route_max_parts(int T) {
  const int a = fast_blocks(T), b = generic_blocks(T);
  return a > b ? a : b;
}

hipError_t launch_route_split(const float* w_router, int E, int d, void* wsplit, hipStream_t s) {
  const int EP = 16 * route_expert_tiles(E);
  const int dpad = route_padded_d(d);
  const size_t n = (size_t)EP * dpad;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  route_split_kernel<<<blocks, 256, 0, s>>>(w_router, E, EP, d, dpad, (uint16_t*)wsplit);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_route_generic(const RouteParams& p, hipStream_t s) {
  const int grid = generic_blocks(p.T);
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
  if (use_fast(p.E, bf16, p.logits_in != nullptr)) {
    const int grid = fast_blocks(p.T);
    if (route_expert_tiles(p.E) == 1) route_fast_kernel<1><<<grid, 256, 0, s>>>(p);
    else route_fast_kernel<2><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  return bf16 ? launch_route_generic<true>(p, s) : launch_route_generic<false>(p, s);
}

}  // namespace moe
