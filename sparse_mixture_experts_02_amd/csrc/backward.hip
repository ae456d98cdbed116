// Backward-pass kernels of the layer (P4 §2.4 trains it end to end): the combine's backward,
// a batched transpose for the expert weights, and the SiLU derivative. The grouped GEMMs of the
// forward pass do the products (with transposed weights), and the combine kernel with unit
// weights sums the permuted rows of each token back (the gather's backward).
#include "moe_internal.h"

namespace moe {

// One wave per token. For each kept slot j: dY[row] = w[t, j] * dOut[t] (fp32 product, one
// rounding) and dw[t, j] = <dOut[t], Y[row]> (fp32 products, lane partial sums added in a fixed
// tree order). Slots without a row get dw = 0.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(CombineBwdParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int k = p.k, d = p.d;
  for (int j = 0; j < k; ++j) {
    int row = p.row_of[(size_t)t * k + j];
    if (row >= p.max_rows) row = -1;
    if (row < 0) {   // uniform across the wave
      if (lane == 0) p.dweights[(size_t)t * k + j] = 0.0f;
      continue;
    }
    const float w = p.weights[(size_t)t * k + j];
    float dot = 0.0f;
    for (int c = lane * 8; c < d; c += 64 * 8) {
      float g[8], y[8];
      if constexpr (BF16) {
        const uint4 ug = *(const uint4*)((const uint16_t*)p.d_out + (size_t)t * d + c);
        const uint4 uy = *(const uint4*)((const uint16_t*)p.y + (size_t)row * d + c);
        const uint32_t wg[4] = {ug.x, ug.y, ug.z, ug.w}, wy[4] = {uy.x, uy.y, uy.z, uy.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          g[2 * q] = bf16_bits_to_f32(wg[q] & 0xFFFFu);
          g[2 * q + 1] = bf16_bits_to_f32(wg[q] >> 16);
          y[2 * q] = bf16_bits_to_f32(wy[q] & 0xFFFFu);
          y[2 * q + 1] = bf16_bits_to_f32(wy[q] >> 16);
        }
      } else {
        const float4* sg = (const float4*)((const float*)p.d_out + (size_t)t * d + c);
        const float4* sy = (const float4*)((const float*)p.y + (size_t)row * d + c);
        const float4 g0 = sg[0], g1 = sg[1], y0 = sy[0], y1 = sy[1];
        g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
        y[0] = y0.x; y[1] = y0.y; y[2] = y0.z; y[3] = y0.w; y[4] = y1.x; y[5] = y1.y; y[6] = y1.z; y[7] = y1.w;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) dot = fmaf(g[q], y[q], dot);
      if constexpr (BF16) {
        uint4 o;
        o.x = pack_bf16x2(w * g[0], w * g[1]);
        o.y = pack_bf16x2(w * g[2], w * g[3]);
        o.z = pack_bf16x2(w * g[4], w * g[5]);
        o.w = pack_bf16x2(w * g[6], w * g[7]);
        *(uint4*)((uint16_t*)p.dy + (size_t)row * d + c) = o;
      } else {
        float4* o = (float4*)((float*)p.dy + (size_t)row * d + c);
        o[0] = make_float4(w * g[0], w * g[1], w * g[2], w * g[3]);
        o[1] = make_float4(w * g[4], w * g[5], w * g[6], w * g[7]);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
    if (lane == 0) p.dweights[(size_t)t * k + j] = dot;
  }
}

hipError_t launch_combine_bwd(const CombineBwdParams& p, bool bf16, hipStream_t s) {
  const int grid = (p.T + 3) / 4;
  if (bf16) combine_bwd_kernel<true><<<grid, 256, 0, s>>>(p);
  else combine_bwd_kernel<false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// 64 x 64 tiles through LDS (one padding column against bank conflicts).
template <typename TE>
__global__ __launch_bounds__(256) void transpose_kernel(const TE* __restrict__ in, TE* __restrict__ out, int R, int C) {
  __shared__ TE tile[64][65];
  const size_t b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const TE* src = in + b * (size_t)R * C;
  TE* dst = out + b * (size_t)R * C;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = src[(size_t)r * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < R && c < C) dst[(size_t)c * R + r] = tile[tx][i];
  }
}

hipError_t launch_transpose(const void* in, void* out, int B, int R, int C, int elem, hipStream_t s) {
  dim3 grid((C + 63) / 64, (R + 63) / 64, B);
  if (elem == 2) transpose_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)in, (uint16_t*)out, R, C);
  else transpose_kernel<float><<<grid, 256, 0, s>>>((const float*)in, (float*)out, R, C);
  return hipGetLastError();
}

// dA = dH * SiLU'(A), SiLU'(a) = s (1 + a (1 - s)) with s = sigmoid(a), in fp32, one rounding.
template <bool BF16>
__global__ __launch_bounds__(256) void silu_bwd_kernel(const void* dh, const void* a, void* da, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    float g, x;
    if constexpr (BF16) {
      g = bf16_bits_to_f32(((const uint16_t*)dh)[i]);
      x = bf16_bits_to_f32(((const uint16_t*)a)[i]);
    } else {
      g = ((const float*)dh)[i];
      x = ((const float*)a)[i];
    }
    const float sg = 1.0f / (1.0f + expf(-x));
    const float v = g * (sg * (1.0f + x * (1.0f - sg)));
    if constexpr (BF16) ((uint16_t*)da)[i] = (uint16_t)f32_to_bf16_bits(v);
    else ((float*)da)[i] = v;
  }
}

hipError_t launch_silu_bwd(const void* dh, const void* a, void* da, size_t n, bool bf16, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks == 0) return hipSuccess;
  if (bf16) silu_bwd_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(dh, a, da, n);
  else silu_bwd_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(dh, a, da, n);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Weight gradients of the grouped GEMMs: for every expert e,
//   G[e][m][n] = sum over the expert's rows r of P[r][m] * Q[r][n]     (fp32 result)
// a product whose reduction runs over the expert's segment of the permuted rows (dW2 = dY^T H,
// dW1 = dA^T Xp). bf16: 64 x 64 output tiles of 4 waves (16 rows each, four 16 x 16 MFMA blocks);
// 32 rows of P and Q per step are staged through LDS transposed (the reduction index becomes
// the contiguous one), then v_mfma_f32_16x16x32_bf16. fp32: one output per thread, fp32 FMA in
// row order.
__global__ __launch_bounds__(256) void grad_w_bf16_kernel(GradWParams p) {
  constexpr int TP = 32 + 8;   // padded row of the transposed tiles (elements)
  __shared__ __attribute__((aligned(16))) uint16_t PT[64 * TP];
  __shared__ __attribute__((aligned(16))) uint16_t QT[64 * TP];
  const int e = blockIdx.y;
  const int tilesN = (p.N + 63) / 64;
  const int m0 = (blockIdx.x / tilesN) * 64, n0 = (blockIdx.x % tilesN) * 64;
  int r0 = p.offsets[e], r1 = p.offsets[e + 1];
  r0 = r0 < 0 ? 0 : (r0 > p.max_rows ? p.max_rows : r0);
  r1 = r1 < r0 ? r0 : (r1 > p.max_rows ? p.max_rows : r1);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const uint16_t* __restrict__ P = (const uint16_t*)p.P;
  const uint16_t* __restrict__ Q = (const uint16_t*)p.Q;
  f32x4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int rr = tid >> 3, cc = (tid & 7) * 8;   // the loader's row within the step and column
  for (int r = r0; r < r1; r += 32) {
    uint4 pv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
    if (r + rr < r1) {
      if (m0 + cc < p.M) pv = *(const uint4*)(P + (size_t)(r + rr) * p.M + m0 + cc);
      if (n0 + cc < p.N) qv = *(const uint4*)(Q + (size_t)(r + rr) * p.N + n0 + cc);
    }
    __syncthreads();   // the previous step's fragments have been read
    const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w}, qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      PT[(cc + 2 * q) * TP + rr] = (uint16_t)(pw[q] & 0xFFFFu);
      PT[(cc + 2 * q + 1) * TP + rr] = (uint16_t)(pw[q] >> 16);
      QT[(cc + 2 * q) * TP + rr] = (uint16_t)(qw[q] & 0xFFFFu);
      QT[(cc + 2 * q + 1) * TP + rr] = (uint16_t)(qw[q] >> 16);
    }
    __syncthreads();
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, *(const uint4*)(PT + (16 * w + fr) * TP + 8 * fg));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t B = __builtin_bit_cast(bf16x8_t, *(const uint4*)(QT + (16 * j + fr) * TP + 8 * fg));
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[j], 0, 0, 0);
    }
  }
  // lane holds rows m0 + 16 w + 4 fg .. + 3 of column n0 + 16 j + fr
  float* __restrict__ G = p.G + (size_t)e * p.M * p.N;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + fr;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = m0 + 16 * w + 4 * fg + t;
      if (m < p.M && n < p.N) G[(size_t)m * p.N + n] = acc[j][t];
    }
  }
}

__global__ __launch_bounds__(256) void grad_w_f32_kernel(GradWParams p) {
  const int e = blockIdx.y;
  int r0 = p.offsets[e], r1 = p.offsets[e + 1];
  r0 = r0 < 0 ? 0 : (r0 > p.max_rows ? p.max_rows : r0);
  r1 = r1 < r0 ? r0 : (r1 > p.max_rows ? p.max_rows : r1);
  const float* __restrict__ P = (const float*)p.P;
  const float* __restrict__ Q = (const float*)p.Q;
  const size_t MN = (size_t)p.M * p.N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / p.N), n = (int)(i % p.N);
    float s = 0.0f;
    for (int r = r0; r < r1; ++r) s = fmaf(P[(size_t)r * p.M + m], Q[(size_t)r * p.N + n], s);
    p.G[(size_t)e * MN + i] = s;
  }
}

hipError_t launch_grad_w(const GradWParams& p, bool bf16, hipStream_t s) {
  if (bf16) {
    dim3 grid(((p.M + 63) / 64) * ((p.N + 63) / 64), p.E);
    grad_w_bf16_kernel<<<grid, 256, 0, s>>>(p);
  } else {
    size_t blocks = ((size_t)p.M * p.N + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    dim3 grid((unsigned)blocks, p.E);
    grad_w_f32_kernel<<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Router backward, per token (one wave, lane e = expert e; E <= 64): the gradient of the logits
// from the gate-weight gradients (softmax over the selected logits / tau, or the full softmax
// when the weights are not renormalised) plus the aux_switch term through the probabilities:
//   d aux_switch / d p[t, i] = d_aux coef E f_i / n,  f_i = counts_pre[i] / (n k),
// with n = sum(counts_pre) / k real tokens. Padding tokens get zero. Everything in fp32.
__global__ __launch_bounds__(256) void route_bwd_kernel(RouteBwdParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int E = p.E, K = p.k;
  const bool ok = lane < E;
  const bool real = !p.token_mask || p.token_mask[t] != 0;
  float dl = 0.0f;
  if (real) {
    const float L = ok ? p.logits[(size_t)t * E + lane] : -INFINITY;
    float mx = L;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    const float z = ok ? __fdiv_rn(__fsub_rn(L, mx), p.tau) : 0.0f;
    const float ex = ok ? expf(z) : 0.0f;
    float s = ex;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s = __fadd_rn(s, __shfl_xor(s, m));
    const float prob = ex / s;
    // this lane's selected slot, its weight and weight gradient
    float wj = 0.0f, gj = 0.0f;
    for (int j = 0; j < K; ++j) {
      if (p.ids[(size_t)t * K + j] == lane) {
        wj = p.weights[(size_t)t * K + j];
        gj = p.dweights[(size_t)t * K + j];
      }
    }
    float g = 0.0f;
    if (p.renormalize) {
      float wg = wj * gj;   // sum over the selected of w_j dw_j
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) wg += __shfl_xor(wg, m);
      g = wj * (gj - wg);
    } else {
      float pg = prob * gj;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) pg += __shfl_xor(pg, m);
      g = prob * (gj - pg);
    }
    // n k = the assignments of all real tokens = the sum of the pre-capacity counts
    const int cnt = (ok && p.counts_pre) ? p.counts_pre[lane] : 0;
    int nk = cnt;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) nk += __shfl_xor(nk, m);
    if (p.d_aux != 0.0f && nk > 0) {
      const float n = (float)(nk / K);
      const float ga = ok ? p.d_aux * p.coef * (float)E * ((float)cnt / (float)nk) / n : 0.0f;
      float pga = prob * ga;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) pga += __shfl_xor(pga, m);
      g += prob * (ga - pga);
    }
    dl = ok ? g / p.tau : 0.0f;
  }
  if (ok) p.dlogits[(size_t)t * E + lane] = dl;
}

// dx[t] += sum_e dL[t, e] W_r[e]: a [T, E] x [E, d] product in fp32 FMAs (the router weight is
// fp32). A block owns 64 tokens x 256 columns: the tokens' dL rows sit in LDS, each thread keeps
// one column's 64 token sums in registers and reads every W_r[e, c] once. The sum is rounded once
// more to act when added to dx.
constexpr int RB_TOK = 64;
template <bool BF16>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(RouteBwdParams p) {
  __shared__ float sdl[RB_TOK][64];
  const int E = p.E, d = p.d;
  const int t0 = blockIdx.y * RB_TOK;
  const int c = blockIdx.x * 256 + threadIdx.x;
  for (int i = threadIdx.x; i < RB_TOK * 64; i += 256) {
    const int tt = i >> 6, e = i & 63;
    const int t = t0 + tt;
    sdl[tt][e] = (t < p.T && e < E) ? p.dlogits[(size_t)t * E + e] : 0.0f;
  }
  __syncthreads();
  if (c >= d) return;
  float acc[RB_TOK];
#pragma unroll
  for (int tt = 0; tt < RB_TOK; ++tt) acc[tt] = 0.0f;
  for (int e = 0; e < E; ++e) {
    const float w = p.w_router[(size_t)e * d + c];
#pragma unroll
    for (int tt = 0; tt < RB_TOK; ++tt) acc[tt] = fmaf(sdl[tt][e], w, acc[tt]);
  }
  const int nt = min(RB_TOK, p.T - t0);
#pragma unroll
  for (int tt = 0; tt < RB_TOK; ++tt) {
    if (tt < nt) {
      const size_t o = (size_t)(t0 + tt) * d + c;
      if constexpr (BF16) {
        uint16_t* dx = (uint16_t*)p.dx;
        dx[o] = (uint16_t)f32_to_bf16_bits(__fadd_rn(bf16_bits_to_f32(dx[o]), acc[tt]));
      } else {
        float* dx = (float*)p.dx;
        dx[o] = __fadd_rn(dx[o], acc[tt]);
      }
    }
  }
}

// dW_r[e, c] = sum_t dL[t, e] x[t, c]: a [E, T] x [T, d] product, split over token chunks. A block
// owns one chunk x 256 columns and keeps, per thread, one column's EM expert sums; the chunk's dL
// rows stream through LDS 64 tokens at a time. Chunk partials [chunks, E, d] are summed in chunk
// order by route_bwd_reduce_kernel (deterministic).
template <bool BF16, int EM>
__global__ __launch_bounds__(256) void route_bwd_w_kernel(RouteBwdParams p) {
  __shared__ float sdl[RB_TOK][EM];
  const int E = p.E, d = p.d;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int tb = blockIdx.y * p.chunk_tokens;
  const int te = min(p.T, tb + p.chunk_tokens);
  float acc[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) acc[e] = 0.0f;
  for (int t0 = tb; t0 < te; t0 += RB_TOK) {
    __syncthreads();
    for (int i = threadIdx.x; i < RB_TOK * EM; i += 256) {
      const int tt = i / EM, e = i % EM;
      const int t = t0 + tt;
      sdl[tt][e] = (t < te && e < E) ? p.dlogits[(size_t)t * E + e] : 0.0f;
    }
    __syncthreads();
    if (c < d) {
      const int nt = min(RB_TOK, te - t0);
      for (int tt = 0; tt < nt; ++tt) {
        const size_t o = (size_t)(t0 + tt) * d + c;
        const float xv = BF16 ? bf16_bits_to_f32(((const uint16_t*)p.x)[o]) : ((const float*)p.x)[o];
#pragma unroll
        for (int e = 0; e < EM; ++e) acc[e] = fmaf(sdl[tt][e], xv, acc[e]);
      }
    }
  }
  if (c < d) {
    float* part = p.part + (size_t)blockIdx.y * E * d;
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) part[(size_t)e * d + c] = acc[e];
  }
}

// dW_r = the chunk partials summed in chunk order; db[e] = sum_t dL[t, e] (a fixed-order tree over
// 256 strided partial sums), from the blocks of the last grid row.
__global__ __launch_bounds__(256) void route_bwd_reduce_kernel(RouteBwdParams p) {
  const size_t n = (size_t)p.E * p.d;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.y == 0) {
    if (i < n && p.dw_router) {
      float acc = 0.0f;
      for (int ch = 0; ch < p.chunks; ++ch) acc += p.part[(size_t)ch * n + i];
      p.dw_router[i] = acc;
    }
    return;
  }
  // blockIdx.y == 1: bias gradient, expert blockIdx.x
  __shared__ float red[256];
  const int e = blockIdx.x;
  if (e >= p.E || !p.dbias) return;
  float acc = 0.0f;
  for (int t = threadIdx.x; t < p.T; t += 256) acc += p.dlogits[(size_t)t * p.E + e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int m = 128; m >= 1; m >>= 1) {
    if ((int)threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.dbias[e] = red[0];
}

// token chunks of the router weight gradient: about 512 blocks in all, chunks a multiple of 64
// tokens long (at most 512 chunks, so the partials take at most 512 * 256 * E fp32 per 256 columns).
void route_bwd_chunks(int T, int d, int* chunks, int* chunk_tokens) {
  const int col_tiles = (d + 255) / 256;
  const int max_chunks = (T + RB_TOK - 1) / RB_TOK;
  int ch = (512 + col_tiles - 1) / col_tiles;
  ch = max(1, min(ch, max_chunks));
  int tok = (T + ch - 1) / ch;
  tok = (tok + RB_TOK - 1) / RB_TOK * RB_TOK;
  *chunk_tokens = tok;
  *chunks = (T + tok - 1) / tok;
}

size_t route_bwd_part_bytes(int T, int d, int E) {
  int ch = 0, tok = 0;
  route_bwd_chunks(T, d, &ch, &tok);
  return (size_t)ch * E * d * sizeof(float);
}

hipError_t launch_route_bwd(const RouteBwdParams& p_in, bool bf16, hipStream_t s) {
  RouteBwdParams p = p_in;
  route_bwd_chunks(p.T, p.d, &p.chunks, &p.chunk_tokens);
  const int grid = (p.T + 3) / 4;
  route_bwd_kernel<<<grid, 256, 0, s>>>(p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int col_tiles = (p.d + 255) / 256;
  if (p.dx) {
    dim3 g(col_tiles, (p.T + RB_TOK - 1) / RB_TOK);
    if (bf16) route_bwd_dx_kernel<true><<<g, 256, 0, s>>>(p);
    else route_bwd_dx_kernel<false><<<g, 256, 0, s>>>(p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (p.dw_router) {
    dim3 g(col_tiles, p.chunks);
#define MOE_RBW(EMV)                                                         \
    if (bf16) route_bwd_w_kernel<true, EMV><<<g, 256, 0, s>>>(p);            \
    else route_bwd_w_kernel<false, EMV><<<g, 256, 0, s>>>(p);
    if (p.E <= 16) { MOE_RBW(16) }
    else if (p.E <= 32) { MOE_RBW(32) }
    else { MOE_RBW(64) }
#undef MOE_RBW
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (p.dw_router || p.dbias) {
    const size_t n = (size_t)p.E * p.d;
    const int gx = (int)std::max<size_t>((n + 255) / 256, (size_t)p.E);
    route_bwd_reduce_kernel<<<dim3(gx, 2), 256, 0, s>>>(p);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
