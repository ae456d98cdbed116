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
