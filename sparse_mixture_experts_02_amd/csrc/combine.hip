// Weighted combine (unpermute) and the probability sums of the stand-alone aux-loss call.
//
// [P4 §2.4] a token's output is the weighted sum of its selected experts' outputs, the weights
// being the softmax router scores; [P4 §5.2] a shared expert's output joins every token's.
// [P4 §3.2] the aux loss averages the router probabilities per expert; [P4 §3.3] the router
// entropy is monitored next to it.
#include "moe_internal.h"

namespace moe {

// One wave per token; each lane owns 8 consecutive columns per step. The k rows of Y are read
// with 16-byte loads (bf16) and accumulated in fp32 in slot order, then rounded once.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int k = p.k;
  int my_row = -1;
  float my_w = 0.0f;
  if (lane < k) {
    my_row = p.row_of[(size_t)t * k + lane];
    my_w = p.weights ? p.weights[(size_t)t * k + lane] : 1.0f;   // no weights: plain sum of the rows
    if (my_row >= p.max_rows) my_row = -1;
  }
  int rows[MOE_MAX_TOP_K_DEV];
  float ws[MOE_MAX_TOP_K_DEV];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K_DEV; ++j) {
    rows[j] = (j < k) ? __shfl(my_row, j) : -1;
    ws[j] = (j < k) ? __shfl(my_w, j) : 0.0f;
  }
  const int d = p.d;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOP_K_DEV; ++j) {
      if (rows[j] < 0) continue;
      float v[8];
      if constexpr (BF16) {
        const uint4 u = *(const uint4*)((const uint16_t*)p.y + (size_t)rows[j] * d + c);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = bf16_bits_to_f32(wd[q] & 0xFFFFu);
          v[2 * q + 1] = bf16_bits_to_f32(wd[q] >> 16);
        }
      } else {
        const float4 a = *(const float4*)((const float*)p.y + (size_t)rows[j] * d + c);
        const float4 b = *(const float4*)((const float*)p.y + (size_t)rows[j] * d + c + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(ws[j], v[q], acc[q]);
    }
    if (p.y_shared) {   // the shared expert's output, weight 1, after the routed slots
      float v[8];
      if constexpr (BF16) {
        const uint4 u = *(const uint4*)((const uint16_t*)p.y_shared + (size_t)t * d + c);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = bf16_bits_to_f32(wd[q] & 0xFFFFu);
          v[2 * q + 1] = bf16_bits_to_f32(wd[q] >> 16);
        }
      } else {
        const float4 a = *(const float4*)((const float*)p.y_shared + (size_t)t * d + c);
        const float4 b = *(const float4*)((const float*)p.y_shared + (size_t)t * d + c + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __fadd_rn(acc[q], v[q]);
    }
    if constexpr (BF16) {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *(uint4*)((uint16_t*)p.out + (size_t)t * d + c) = o;
    } else {
      *(float4*)((float*)p.out + (size_t)t * d + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *(float4*)((float*)p.out + (size_t)t * d + c + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// bf16, top-k <= 2, d a multiple of 512 and at most 4096: one wave per token as above, but every
// load of the token (up to 8 column steps x 2 rows, 16 bytes per lane each) is issued before the
// first use, so a wave keeps all of its row reads in flight at once. Y rows are read once, with the
// non-temporal hint (measured: 3-5% faster; the same hint on the output stores was slower). Same
// arithmetic and order as the general kernel (fp32 FMA in slot order, one rounding).
// The loads are unconditional (a slot without a row reads row 0 and its terms are replaced by 0
// with a select, never multiplied: the row may hold anything), followed by one explicit wait, so
// that the compiler places no wait between the column steps' stores (a wait there would also
// wait for the previous step's store).
__global__ __launch_bounds__(256) void combine_k2_kernel(CombineParams p) {
  constexpr int MAXU = 8;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int k = p.k, d = p.d;
  int my_row = -1;
  float my_w = 0.0f;
  if (lane < k) {
    my_row = p.row_of[(size_t)t * k + lane];
    my_w = p.weights ? p.weights[(size_t)t * k + lane] : 1.0f;   // no weights: plain sum of the rows
    if (my_row >= p.max_rows) my_row = -1;
  }
  const int r0 = __shfl(my_row, 0), r1 = k > 1 ? __shfl(my_row, 1) : -1;
  const float w0 = __shfl(my_w, 0), w1 = k > 1 ? __shfl(my_w, 1) : 0.0f;
  const bool h0 = r0 >= 0, h1 = r1 >= 0;
  const int nu = d >> 9;   // column steps of 512
  const u32x4_t* y0 = (const u32x4_t*)((const uint16_t*)p.y + (size_t)(h0 ? r0 : 0) * d) + lane;
  const u32x4_t* y1 = (const u32x4_t*)((const uint16_t*)p.y + (size_t)(h1 ? r1 : 0) * d) + lane;
  const bool sh = p.y_shared != nullptr;
  const u32x4_t* ys = (const u32x4_t*)((const uint16_t*)(sh ? p.y_shared : p.y) + (size_t)(sh ? t : 0) * d) + lane;
  u32x4_t a[MAXU], b[MAXU], c[MAXU];
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
    if (u < nu) {   // uniform
      a[u] = __builtin_nontemporal_load(y0 + u * 64);
      b[u] = __builtin_nontemporal_load(y1 + u * 64);
      if (sh) c[u] = __builtin_nontemporal_load(ys + u * 64);   // uniform (a kernel argument)
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every row has landed
  u32x4_t* out = (u32x4_t*)((uint16_t*)p.out + (size_t)t * d) + lane;
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
    if (u < nu) {
      float acc[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = fmaf(w0, bf16_bits_to_f32(a[u][q] & 0xFFFFu), 0.0f);
        const float x1 = fmaf(w0, bf16_bits_to_f32(a[u][q] >> 16), 0.0f);
        acc[2 * q] = h0 ? x0 : 0.0f;
        acc[2 * q + 1] = h0 ? x1 : 0.0f;
        const float y0v = fmaf(w1, bf16_bits_to_f32(b[u][q] & 0xFFFFu), acc[2 * q]);
        const float y1v = fmaf(w1, bf16_bits_to_f32(b[u][q] >> 16), acc[2 * q + 1]);
        acc[2 * q] = h1 ? y0v : acc[2 * q];
        acc[2 * q + 1] = h1 ? y1v : acc[2 * q + 1];
        if (sh) {   // the shared expert's output, weight 1, after the routed slots
          acc[2 * q] = __fadd_rn(acc[2 * q], bf16_bits_to_f32(c[u][q] & 0xFFFFu));
          acc[2 * q + 1] = __fadd_rn(acc[2 * q + 1], bf16_bits_to_f32(c[u][q] >> 16));
        }
      }
      const u32x4_t o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                         pack_bf16x2(acc[6], acc[7])};
      out[u * 64] = o;
    }
  }
}

hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s) {
  const int grid = (p.T + 3) / 4;
  if (bf16 && p.k <= 2 && p.d % 512 == 0 && p.d <= 4096) combine_k2_kernel<<<grid, 256, 0, s>>>(p);
  else if (bf16) combine_kernel<true><<<grid, 256, 0, s>>>(p);
  else combine_kernel<false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ aux losses

constexpr int PROBSUM_TOKENS = 256;  // tokens per block of the stand-alone probability sum

// Per-block sums of softmax(logits / tau) (or of given probabilities) per expert, in double.
// Thread layout: EPAD = E rounded up to a power of two lanes per token, 256 / EPAD tokens at a
// time; partial sums are combined in LDS in a fixed order.
__global__ __launch_bounds__(256) void probsum_kernel(ProbSumParams p) {
  __shared__ double part[256];
  __shared__ double hpart[256];
  __shared__ double cpart[256];
  const int tid = threadIdx.x;
  const int E = p.E;
  int EPAD = 1;
  while (EPAD < E) EPAD <<= 1;
  const int e = tid % EPAD;
  const int sub = tid / EPAD;
  const int nsub = 256 / EPAD;
  const int t0 = blockIdx.x * PROBSUM_TOKENS;
  const int t1 = min(p.T, t0 + PROBSUM_TOKENS);
  double acc = 0.0, hacc = 0.0, cacc = 0.0;
  for (int t = t0 + sub; t < t1; t += nsub) {
    if (p.token_mask && p.token_mask[t] == 0) continue;   // padding: left out
    float prob = 0.0f;
    if (p.probs) {
      prob = (e < E) ? p.probs[(size_t)t * E + e] : 0.0f;
      if (e == 0) {   // entropy of the row, -sum p ln p (0 ln 0 = 0)
        float h = 0.0f;
        for (int q = 0; q < E; ++q) {
          const float v = p.probs[(size_t)t * E + q];
          if (v > 0.0f) h = __fsub_rn(h, v * logf(v));
        }
        hacc += (double)h;
      }
    } else {
      const float* row = p.logits + (size_t)t * E;
      float mx = -INFINITY;
      for (int q = 0; q < E; ++q) mx = fmaxf(mx, row[q]);
      float s = 0.0f;
      for (int q = 0; q < E; ++q) s = __fadd_rn(s, expf(__fdiv_rn(__fsub_rn(row[q], mx), p.tau)));
      prob = (e < E) ? __fdiv_rn(expf(__fdiv_rn(__fsub_rn(row[e], mx), p.tau)), s) : 0.0f;
      if (e == 0) {   // entropy = ln s - sum p z, z = (L - max) / tau
        float pz = 0.0f;
        for (int q = 0; q < E; ++q) {
          const float z = __fdiv_rn(__fsub_rn(row[q], mx), p.tau);
          pz = __fadd_rn(pz, __fdiv_rn(expf(z), s) * z);
        }
        hacc += (double)__fsub_rn(logf(s), pz);
      }
    }
    acc += (double)prob;
    if (e == 0) cacc += 1.0;
  }
  part[tid] = acc;
  hpart[tid] = hacc;
  cpart[tid] = cacc;
  __syncthreads();
  double* out = p.psum + (size_t)blockIdx.x * (E + 2);
  if (tid < E) {
    double s = 0.0;
    for (int q = 0; q < nsub; ++q) s += part[q * EPAD + tid];
    out[tid] = s;
  } else if (tid == E || tid == E + 1) {
    const double* src = (tid == E) ? hpart : cpart;
    double s = 0.0;
    for (int q = 0; q < nsub; ++q) s += src[q * EPAD];
    out[tid] = s;
  }
}

int probsum_num_blocks(int T) { return (T + PROBSUM_TOKENS - 1) / PROBSUM_TOKENS; }

hipError_t launch_probsum(const ProbSumParams& p, hipStream_t s) {
  probsum_kernel<<<probsum_num_blocks(p.T), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
