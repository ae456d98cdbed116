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
