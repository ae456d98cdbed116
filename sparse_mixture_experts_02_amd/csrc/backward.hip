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

typedef unsigned cb_u32x4_t __attribute__((ext_vector_type(4)));

// bf16, top-k <= 2, d = 512 NU (NU = 1, 2, 4 or 8): the same arithmetic in the same order (each
// lane's terms in column order, then the same butterfly), with every load of the token (its dOut
// row and the rows of both slots, NU column steps of 16 bytes per lane each) issued before the
// first use and one explicit wait after them, so that no wait of the compiler's sits between the
// stores. The loads are unconditional: a slot without a row reads row 0 and its sum is replaced by
// 0 with a select (the row may hold anything). Y rows are read once, with the non-temporal hint.
// The two slots' reductions are interleaved, so their cross-lane round trips overlap.
template <int NU>
__global__ __launch_bounds__(256) void combine_bwd_k2_kernel(CombineBwdParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int k = p.k, d = p.d;
  int my_row = -1;
  float my_w = 0.0f;
  if (lane < k) {
    my_row = p.row_of[(size_t)t * k + lane];
    my_w = p.weights[(size_t)t * k + lane];
    if (my_row >= p.max_rows) my_row = -1;
  }
  const int r0 = __shfl(my_row, 0), r1 = k > 1 ? __shfl(my_row, 1) : -1;
  const float w0 = __shfl(my_w, 0), w1 = k > 1 ? __shfl(my_w, 1) : 0.0f;
  const bool h0 = r0 >= 0, h1 = r1 >= 0;
  const cb_u32x4_t* gp = (const cb_u32x4_t*)((const uint16_t*)p.d_out + (size_t)t * d) + lane;
  const cb_u32x4_t* y0 = (const cb_u32x4_t*)((const uint16_t*)p.y + (size_t)(h0 ? r0 : 0) * d) + lane;
  const cb_u32x4_t* y1 = (const cb_u32x4_t*)((const uint16_t*)p.y + (size_t)(h1 ? r1 : 0) * d) + lane;
  cb_u32x4_t g[NU], a[NU], b[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    g[u] = gp[u * 64];
    a[u] = __builtin_nontemporal_load(y0 + u * 64);
    if (k > 1) b[u] = __builtin_nontemporal_load(y1 + u * 64);   // uniform (a kernel argument)
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every row has landed
  cb_u32x4_t* o0 = (cb_u32x4_t*)((uint16_t*)p.dy + (size_t)(h0 ? r0 : 0) * d) + lane;
  cb_u32x4_t* o1 = (cb_u32x4_t*)((uint16_t*)p.dy + (size_t)(h1 ? r1 : 0) * d) + lane;
  float dot0 = 0.0f, dot1 = 0.0f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    float gf[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      gf[2 * h] = bf16_bits_to_f32(g[u][h] & 0xFFFFu);
      gf[2 * h + 1] = bf16_bits_to_f32(g[u][h] >> 16);
      dot0 = fmaf(gf[2 * h], bf16_bits_to_f32(a[u][h] & 0xFFFFu), dot0);
      dot0 = fmaf(gf[2 * h + 1], bf16_bits_to_f32(a[u][h] >> 16), dot0);
      if (k > 1) {
        dot1 = fmaf(gf[2 * h], bf16_bits_to_f32(b[u][h] & 0xFFFFu), dot1);
        dot1 = fmaf(gf[2 * h + 1], bf16_bits_to_f32(b[u][h] >> 16), dot1);
      }
    }
    if (h0)
      o0[u * 64] = cb_u32x4_t{pack_bf16x2(w0 * gf[0], w0 * gf[1]), pack_bf16x2(w0 * gf[2], w0 * gf[3]),
                              pack_bf16x2(w0 * gf[4], w0 * gf[5]), pack_bf16x2(w0 * gf[6], w0 * gf[7])};
    if (h1)
      o1[u * 64] = cb_u32x4_t{pack_bf16x2(w1 * gf[0], w1 * gf[1]), pack_bf16x2(w1 * gf[2], w1 * gf[3]),
                              pack_bf16x2(w1 * gf[4], w1 * gf[5]), pack_bf16x2(w1 * gf[6], w1 * gf[7])};
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    dot0 += __shfl_xor(dot0, m);
    dot1 += __shfl_xor(dot1, m);
  }
  if (lane == 0) {
    p.dweights[(size_t)t * k] = h0 ? dot0 : 0.0f;
    if (k > 1) p.dweights[(size_t)t * k + 1] = h1 ? dot1 : 0.0f;
  }
}

hipError_t launch_combine_bwd(const CombineBwdParams& p, bool bf16, hipStream_t s) {
  const int grid = (p.T + 3) / 4;
  const int nu = p.d / 512;
  const bool k2 = bf16 && p.k <= 2 && p.d % 512 == 0 && (nu == 1 || nu == 2 || nu == 4 || nu == 8);
  if (k2 && nu == 1) combine_bwd_k2_kernel<1><<<grid, 256, 0, s>>>(p);
  else if (k2 && nu == 2) combine_bwd_k2_kernel<2><<<grid, 256, 0, s>>>(p);
  else if (k2 && nu == 4) combine_bwd_k2_kernel<4><<<grid, 256, 0, s>>>(p);
  else if (k2) combine_bwd_k2_kernel<8><<<grid, 256, 0, s>>>(p);
  else if (bf16) combine_bwd_kernel<true><<<grid, 256, 0, s>>>(p);
  else combine_bwd_kernel<false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// fp32: 64 x 64 tiles through LDS (one padding column against bank conflicts).
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

// bf16 (R and C multiples of 8): no LDS. Each thread moves one 8 x 8 block: 8 loads of 16 bytes
// (rows 8 rb .. 8 rb + 7), a register transpose (v_perm of half-words) and 8 stores of 16 bytes.
// A wave covers 64 x 64: lane = rb + 8 cb, so each load instruction reads 8 rows x 128
// contiguous bytes and each store writes 8 output rows x 128 contiguous bytes.
__global__ __launch_bounds__(256) void transpose_b16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                            int R, int C) {
  const size_t b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.y * 64 + 8 * (lane & 7);
  const int c = blockIdx.x * 256 + 64 * w + 8 * (lane >> 3);
  if (r >= R || c >= C) return;
  const uint16_t* src = in + b * (size_t)R * C + (size_t)r * C + c;
  uint16_t* dst = out + b * (size_t)R * C + (size_t)c * R + r;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *(const uint4*)(src + (size_t)i * C);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = __builtin_amdgcn_perm(((const uint32_t*)&v[2 * q + 1])[j >> 1], ((const uint32_t*)&v[2 * q])[j >> 1], sel);
    *(uint4*)(dst + (size_t)j * R) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_transpose(const void* in, void* out, int B, int R, int C, int elem, hipStream_t s) {
  if (elem == 2) {
    dim3 grid((C + 255) / 256, (R + 63) / 64, B);
    transpose_b16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)in, (uint16_t*)out, R, C);
  } else {
    dim3 grid((C + 63) / 64, (R + 63) / 64, B);
    transpose_kernel<float><<<grid, 256, 0, s>>>((const float*)in, (float*)out, R, C);
  }
  return hipGetLastError();
}

// dA = dH * SiLU'(A), SiLU'(a) = s (1 + a (1 - s)) with s = sigmoid(a), in fp32, one rounding.
// 16 bytes per thread and step (8 bf16 or 4 fp32 elements; cols is a multiple of 8). Rows past
// *nrows (the kept rows, read on the device; clamped to max_rows) are left alone. bf16: dsilu_mul
// and one packed conversion per two results. (Multiplying in the [K, N] product's epilogue
// instead was measured slower: holding the pre-activation's pieces for a tile there takes
// registers that kernel does not have, and the spills wait on its operand loads.)
template <bool BF16>
__global__ __launch_bounds__(256) void silu_bwd_kernel(const void* dh, const void* a, void* da, const int32_t* nrows,
                                                       int max_rows, int cols) {
  constexpr int V = BF16 ? 8 : 4;
  int r = *nrows;
  r = r < 0 ? 0 : (r > max_rows ? max_rows : r);
  const size_t nv = (size_t)r * cols / V;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 gv = ((const uint4*)dh)[i];
    const uint4 xv = ((const uint4*)a)[i];
    const uint32_t* gw = (const uint32_t*)&gv;
    const uint32_t* xw = (const uint32_t*)&xv;
    uint4 ov;
    uint32_t* ow = (uint32_t*)&ov;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (BF16) {
        float r[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float g = bf16_bits_to_f32((gw[q] >> (16 * h)) & 0xFFFFu);
          const float x = bf16_bits_to_f32((xw[q] >> (16 * h)) & 0xFFFFu);
          r[h] = dsilu_mul(g, x);
        }
        ow[q] = pack_bf16x2(r[0], r[1]);
      } else {
        const float g = __uint_as_float(gw[q]), x = __uint_as_float(xw[q]);
        const float sg = 1.0f / (1.0f + expf(-x));
        ow[q] = __float_as_uint(g * (sg * (1.0f + x * (1.0f - sg))));
      }
    }
    ((uint4*)da)[i] = ov;
  }
}

hipError_t launch_silu_bwd(const void* dh, const void* a, void* da, const int32_t* nrows, int max_rows, int cols,
                           bool bf16, hipStream_t s) {
  const size_t nv = (size_t)max_rows * cols / (bf16 ? 8 : 4);
  size_t blocks = (nv + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks == 0) return hipSuccess;
  if (bf16) silu_bwd_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(dh, a, da, nrows, max_rows, cols);
  else silu_bwd_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(dh, a, da, nrows, max_rows, cols);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Weight gradients of the grouped GEMMs: for every expert e,
//   G[e][m][n] = sum over the expert's rows r of P[r][m] * Q[r][n]     (fp32 result)
// a product whose reduction runs over the expert's segment of the permuted rows (dW2 = dY^T H,
// dW1 = dA^T Xp). bf16 (grad_w_bf16_kernel):
//  * one 256 x 256 output tile of one expert per workgroup; 8 waves in 2 x 4, each 128 x 64 =
//    8 x 4 blocks of v_mfma_f32_16x16x32_bf16. Tiles are numbered so that each XCD takes a
//    contiguous range (the same expert), walked in groups of 8 m-tiles: the tiles in flight on
//    an XCD share their rows of P and Q 8 ways in its L2.
//  * the reduction runs in stages of 64 rows. P and Q are row-major in r; a stage of each operand
//    (64 rows x the tile's 256 columns) sits in LDS as four 64-column blocks of 64 rows x 128
//    bytes, filled row for row by direct buffer -> LDS loads (8 rows x 128 bytes per
//    instruction). An MFMA operand wants 8 consecutive r per lane; the transposing LDS read
//    (ds_read_b64_tr_b16) delivers 4 of them: in each group of 16 lanes, lane s reads 8 bytes of
//    row r0 + s / 4 at column c0 + 4 (s % 4), and lane i receives column c0 + i of rows
//    r0 .. r0 + 3. Within a row the four 32-byte quarters are XOR-swizzled by
//    f(r) = ((r >> 1) & 1) | (((r >> 3) & 1) << 1), which puts the 16 rows x 32 bytes of one such
//    read of a wave on every bank octet exactly twice (two cycles, the minimum for 512 bytes).
//  * ping-pong, as in the forward's grouped GEMM: the two waves of each SIMD (w and w + 4, the
//    tile's two 128-row halves in m, groups 0 and 1) take turns at the matrix core. In one phase a
//    group issues its stage's 64 MFMAs and nothing else while the other reads its next fragments
//    from LDS and issues its share of the direct loads; a barrier ends each phase. Group 1 runs
//    one phase behind group 0. Group 0 loads P, group 1 loads Q: wave wn of a group fills
//    64-column block wn of its operand. P of stage s + 2 goes into stage s's buffer right after
//    the phase in which group 1 read stage s; Q of stage s + 3 goes into stage s + 1's buffer
//    right after wave wn of group 1 has read that block, which its partner in group 0 read one
//    phase before. Each group waits for its loads at the end of its next MFMA phase.
constexpr int GW_TILE = 256, GW_BK = 64;
constexpr int GW_CB_BYTES = GW_BK * 128;            // one 64-column block of one operand: 8 KiB
constexpr int GW_OP_BYTES = 4 * GW_CB_BYTES;        // one operand, one stage: 32 KiB
constexpr int GW_STAGE_BYTES = 2 * GW_OP_BYTES;     // P and Q

typedef short gw_v4i16 __attribute__((ext_vector_type(4)));

// Direct buffer -> LDS 16-byte load per lane (lane l writes LDS [lds_addr + 16 l, + 16)), with a
// uniform byte offset in the scalar offset register; M0 is restored afterwards. The kernel waits
// for these itself (vmcnt).
__device__ __forceinline__ void gw_load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                              uint32_t lds_addr) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}

__device__ __forceinline__ gw_v4i16 gw_read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) gw_v4i16*)(uintptr_t)addr);
}

__global__ __launch_bounds__(512, 1) void grad_w_bf16_kernel(GradWParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * GW_STAGE_BYTES];   // [buffer][P, Q][block]
  const int tilesM = (p.M + GW_TILE - 1) / GW_TILE, tilesN = (p.N + GW_TILE - 1) / GW_TILE;
  const int per_e = tilesM * tilesN, total = per_e * p.E * p.splits;
  int b = blockIdx.x;
  if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);   // contiguous block range per XCD
  const int part = b % p.splits;
  b /= p.splits;
  // within an expert, groups of 8 m-tiles walked n-tile by n-tile
  const int e = b / per_e, rem = b - e * per_e;
  const int grp = rem / (8 * tilesN), gm0 = grp * 8, gsz = min(8, tilesM - gm0);
  const int in = rem - grp * 8 * tilesN;
  const int m0 = (gm0 + in % gsz) * GW_TILE, n0 = (in / gsz) * GW_TILE;
  int r0 = p.offsets[e], r1 = p.offsets[e + 1];
  r0 = r0 < 0 ? 0 : (r0 > p.max_rows ? p.max_rows : r0);
  r1 = r1 < r0 ? r0 : (r1 > p.max_rows ? p.max_rows : r1);
  if (p.splits == 2) {   // this block's half of the segment, split at a whole stage
    const int mid = min(r1, r0 + ((r1 - r0 + 2 * GW_BK - 1) / (2 * GW_BK)) * GW_BK);
    if (part == 0) r1 = mid;
    else r0 = mid;
  }
  r0 = __builtin_amdgcn_readfirstlane(r0);
  r1 = __builtin_amdgcn_readfirstlane(r1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gr = w >> 2, wn = w & 3;
  const int fr = lane & 15, fg = lane >> 4;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // Loader: wave wn of group gr copies 64-column block wn of its operand (P for group 0, Q for
  // group 1). Instruction i (i < 8) fills rows 8 i .. 8 i + 7 of the block; lane l fills 16-byte
  // slot l % 8 of row 8 i + l / 8 with the global chunk the swizzle puts there, chunk
  // (l % 8) ^ 2 f(row) (f of that row is ((l >> 4) & 1) | ((i & 1) << 1)). Offsets relative to the
  // stage's first row; the row offset 16 (i / 2) rows goes in the scalar offset. Columns past M
  // (or N) get an offset outside every resource (zeros, nothing fetched); rows past the segment's
  // end fall outside the stage's resource.
  const int opc = gr == 0 ? p.M : p.N;   // columns of this wave's operand
  const uint32_t rs = (uint32_t)opc * 2u;  // its row stride in bytes
  const int cb0 = (gr == 0 ? m0 : n0) + 64 * wn;
  uint32_t vo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int chunk = (lane & 7) ^ ((((lane >> 4) & 1) << 1) | (h << 2));
    const int c = cb0 + 8 * chunk;
    vo[h] = c < opc ? (uint32_t)(8 * h + (lane >> 3)) * rs + (uint32_t)c * 2u : 0x80000000u;
  }
  const uint16_t* const src = (const uint16_t*)(gr == 0 ? p.P : p.Q);
  auto load_stage = [&](int st, int buf) {   // stage st (< number of stages) into buffer buf
    const int r = r0 + st * GW_BK;
    const int nrows = min(GW_BK, r1 - r);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)r * opc), 0, nrows * rs, 0x00020000);
    const uint32_t base = lds0 + buf * GW_STAGE_BYTES + gr * GW_OP_BYTES + wn * GW_CB_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) gw_load_lds16(rsrc, vo[i & 1], (uint32_t)(i >> 1) * 16u * rs, base + i * 1024);
  };

  // Fragment reads: lane s = fr of group fg reads, for block u (16 columns at 16 u of a 64-column
  // block) and half hh, row 32 ks + 8 fg + 4 hh + fr / 4, bytes 8 (fr % 4) of quarter u ^ f(row);
  // f(row) = (fr >> 3) | ((fg & 1) << 1) for every ks and hh. The per-lane part without the
  // quarter is rd; quarter u is an XOR of bits 5-6, which no other term of the address touches,
  // so each u gets its own address register and the rest are immediate offsets.
  const uint32_t rd = (uint32_t)((8 * fg + (fr >> 2)) * 128 + 8 * (fr & 3) + 32 * ((fr >> 3) | ((fg & 1) << 1)));
  bf16x8_t xa[2][8], wb[2][4];
  auto read_frags = [&](int g) {
    const uint32_t bufb = lds0 + (g & 1) * GW_STAGE_BYTES;
    const uint32_t pb = bufb + gr * 2 * GW_CB_BYTES;          // blocks 2 gr, 2 gr + 1 of P
    const uint32_t qb = bufb + GW_OP_BYTES + wn * GW_CB_BYTES;  // block wn of Q
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t ru = rd ^ (uint32_t)(32 * u);
      asm volatile("" : "+v"(ru));
      const uint32_t pa = pb + ru, qa = qb + ru;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {   // P blocks u (block 2 gr) and 4 + u (block 2 gr + 1)
          const uint32_t a = pa + half * GW_CB_BYTES + ks * 32 * 128;
          const gw_v4i16 lo = gw_read_tr(a), hi = gw_read_tr(a + 4 * 128);
          xa[ks][4 * half + u] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        const uint32_t a = qa + ks * 32 * 128;
        const gw_v4i16 lo = gw_read_tr(a), hi = gw_read_tr(a + 4 * 128);
        wb[ks][u] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  f32x4_t acc[8][4];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&]() {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[mi][ni]) : "v"(xa[ks][mi]), "v"(wb[ks][ni]));
    __builtin_amdgcn_sched_barrier(0);
  };
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  const int ns = (r1 - r0 + GW_BK - 1) / GW_BK;
  if (ns > 0) {
    load_stage(0, 0);
    if (ns > 1) load_stage(1, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    read_frags(0);
    if (gr == 1) {
      phase_end();   // group 0's stage-0 reads are done too: Q of stage 2 may replace stage 0's
      if (ns > 2) load_stage(2, 0);
    }
    for (int s = 0; s < ns; ++s) {
      compute();
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads of its previous memory phase
      phase_end();
      if (gr == 0 && s + 2 < ns) load_stage(s + 2, s & 1);
      if (s + 1 < ns) read_frags(s + 1);
      if (gr == 1 && s + 3 < ns) load_stage(s + 3, (s + 1) & 1);
      phase_end();
    }
    if (gr == 0) phase_end();
    // let the last MFMAs retire before their accumulators are read
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]),
                   "+a"(acc[6][0]), "+a"(acc[6][1]), "+a"(acc[6][2]), "+a"(acc[6][3])
                 :
                 : "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane holds rows m0 + 128 gr + 16 mi + 4 fg .. + 3 of column n0 + 64 wn + 16 ni + fr
  float* __restrict__ G = p.G + (size_t)e * p.M * p.N;
  if (p.splits == 2) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int n = n0 + 64 * wn + 16 * ni + fr;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int m = m0 + 128 * gr + 16 * mi + 4 * fg + t;
          // two halves: each adds its partial sum to the zeroed G (0 + a is exact and a + b
          // commutes, so the result does not depend on which half lands first)
          if (m < p.M && n < p.N) atomicAdd(&G[(size_t)m * p.N + n], acc[mi][ni][t]);
        }
      }
    return;
  }
  // Row-major stores through LDS, one 16-row block at a time: the lane's four values (four rows
  // of one column) go to a per-wave area, and each lane reads back four consecutive columns of
  // one row, so that a store instruction covers 4 rows x 256 contiguous bytes (stored straight
  // from the accumulator layout, an instruction covered 4 rows x 64 bytes with 4-byte stores:
  // measured ~68 us of each main-size launch). Two areas per wave alternate between blocks (LDS
  // operations of one wave complete in order, so a block's reads see its writes and the next
  // block but one may overwrite them). Row pitch 68 floats: the four row groups of a write fall
  // on different banks. The stage buffers are free once every wave is past its last fragment
  // read.
  __syncthreads();
  constexpr int EPF = 68;
  static_assert(8 * 2 * 16 * EPF * 4 <= 2 * GW_STAGE_BYTES, "the epilogue areas lie in the stage buffers");
  float* const ep = (float*)lds + w * 2 * 16 * EPF;
  const int rr = lane >> 4, rc = (lane & 15) * 4;   // read-back: row within 4, first column
  const int n = n0 + 64 * wn + rc;
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) {
    float* const a = ep + (mi & 1) * 16 * EPF;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int t = 0; t < 4; ++t) a[(4 * fg + t) * EPF + 16 * ni + fr] = acc[mi][ni][t];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + rr;
      const f32x4_t v = *(const f32x4_t*)(a + row * EPF + rc);
      const int m = m0 + 128 * gr + 16 * mi + row;
      if (m < p.M && n < p.N) *(f32x4_t*)(G + (size_t)m * p.N + n) = v;   // N % 4 == 0: all or none
    }
  }
}

// fp32: one 128 x 128 output tile of one expert per workgroup; 4 waves in 2 x 2, each 64 x 64 =
// 4 x 4 blocks of v_mfma_f32_16x16x4_f32 (exact fp32 products, fp32 sums). The reduction runs
// in stages of 16 rows: P and Q are row-major in r, which is already the operand order of this
// MFMA (a lane takes one element of one row), so each stage is copied row for row into LDS
// ([r][m] and [r][n], pitch 144 floats: the 4 rows a wave reads at once fall in different
// banks) and the next stage is fetched into registers while the current one is multiplied.
// Rows past the segment's end and columns past M or N read as zeros.
constexpr int GF_TILE = 128, GF_BK = 16, GF_PITCH = GF_TILE + 16;

__global__ __launch_bounds__(256) void grad_w_f32_kernel(GradWParams p) {
  __shared__ __attribute__((aligned(16))) float lds[2][2][GF_BK * GF_PITCH];
  const int tilesM = (p.M + GF_TILE - 1) / GF_TILE, tilesN = (p.N + GF_TILE - 1) / GF_TILE;
  const int per_e = tilesM * tilesN;
  const int e = blockIdx.x / per_e, rem = blockIdx.x - e * per_e;
  const int m0 = (rem % tilesM) * GF_TILE, n0 = (rem / tilesM) * GF_TILE;
  int r0 = p.offsets[e], r1 = p.offsets[e + 1];
  r0 = r0 < 0 ? 0 : (r0 > p.max_rows ? p.max_rows : r0);
  r1 = r1 < r0 ? r0 : (r1 > p.max_rows ? p.max_rows : r1);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  // loader: thread t moves the 16-byte pieces t and t + 256 of each operand's stage (16 rows x
  // 128 columns = 32 pieces per row), through a buffer resource covering the stage's valid rows
  int lrow[2], lcol[2];
  uint32_t voffP[2], voffQ[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = tid + 256 * h;
    lrow[h] = idx >> 5;
    lcol[h] = 4 * (idx & 31);
    voffP[h] = m0 + lcol[h] < p.M ? (uint32_t)(lrow[h] * p.M + m0 + lcol[h]) * 4u : 0x80000000u;
    voffQ[h] = n0 + lcol[h] < p.N ? (uint32_t)(lrow[h] * p.N + n0 + lcol[h]) * 4u : 0x80000000u;
  }
  const float* const P = (const float*)p.P;
  const float* const Q = (const float*)p.Q;
  f32x4_t vp[2], vq[2];
  auto load = [&](int r) {
    const int nrows = r < r1 ? min(GF_BK, r1 - r) : 0;
    const int rb = r < r1 ? r : r0;
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc((void*)(P + (size_t)rb * p.M), 0, nrows * p.M * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Q + (size_t)rb * p.N), 0, nrows * p.N * 4, 0x00020000);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      vp[h] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (int)voffP[h], 0, 0));
      vq[h] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)voffQ[h], 0, 0));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *(f32x4_t*)&lds[buf][0][lrow[h] * GF_PITCH + lcol[h]] = vp[h];
      *(f32x4_t*)&lds[buf][1][lrow[h] * GF_PITCH + lcol[h]] = vq[h];
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wm = w >> 1, wn = w & 1;
  const int ns = (r1 - r0 + GF_BK - 1) / GF_BK;
  if (ns > 0) {
    load(r0);
    store(0);
    __syncthreads();
  }
  for (int s = 0; s < ns; ++s) {
    load(r0 + (s + 1) * GF_BK);   // past the last stage: an empty resource, zeros
    const float* A = &lds[s & 1][0][0];
    const float* B = &lds[s & 1][1][0];
#pragma unroll
    for (int kk = 0; kk < GF_BK / 4; ++kk) {
      float af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = A[(4 * kk + fg) * GF_PITCH + 64 * wm + 16 * i + fr];
        bfr[i] = B[(4 * kk + fg) * GF_PITCH + 64 * wn + 16 * i + fr];
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    store((s + 1) & 1);
    __syncthreads();
  }
  // lane holds rows m0 + 64 wm + 16 mi + 4 fg .. + 3 of column n0 + 64 wn + 16 ni + fr
  float* __restrict__ G = p.G + (size_t)e * p.M * p.N;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int n = n0 + 64 * wn + 16 * ni + fr;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + 64 * wm + 16 * mi + 4 * fg + t;
        if (m < p.M && n < p.N) G[(size_t)m * p.N + n] = acc[mi][ni][t];
      }
    }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) x[i] = 0.0f;
}

hipError_t launch_grad_w(const GradWParams& p_in, bool bf16, hipStream_t s) {
  GradWParams p = p_in;
  p.splits = 1;
  if (bf16) {
    const int tiles = ((p.M + GW_TILE - 1) / GW_TILE) * ((p.N + GW_TILE - 1) / GW_TILE) * p.E;
    if (tiles == 0) return hipSuccess;
    if (tiles < 256) {   // fewer tiles than CUs (a shared expert: E = 1): split each reduction in two
      p.splits = 2;
      const size_t n = (size_t)p.E * p.M * p.N;
      zero_f32_kernel<<<(unsigned)std::min<size_t>((n + 255) / 256, 8192), 256, 0, s>>>(p.G, n);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    grad_w_bf16_kernel<<<tiles * p.splits, 512, 0, s>>>(p);
  } else {
    const int tiles = ((p.M + GF_TILE - 1) / GF_TILE) * ((p.N + GF_TILE - 1) / GF_TILE) * p.E;
    if (tiles == 0) return hipSuccess;
    grad_w_f32_kernel<<<tiles, 256, 0, s>>>(p);
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
// fp32), each token's sum added to dx with one more rounding to act. The tokens' dL rows sit in
// LDS (read back as 16-byte vectors, the same address for every lane).
// Up to 16 experts (route_bwd_dx_kernel): a block owns RB_DX_TOK tokens x 2048 columns, a thread 8
// consecutive columns with their EM x 8 router weights in registers; the dx values of 8 (EM 16:
// 4) tokens are loaded (16 bytes per token for bf16) before any of them is updated, and the
// blocks are short so that several run on each CU. 32 or 64 experts (route_bwd_dx1_kernel): one column per thread,
// 256 columns per block, one token at a time.
constexpr int RB_TOK = 64;
constexpr int RB_DX_COLS = 2048;   // columns per block of route_bwd_dx_kernel (256 threads x 8)
constexpr int RB_DX_TOK = 16;      // tokens per block of route_bwd_dx_kernel
typedef unsigned rb_u32x4 __attribute__((ext_vector_type(4)));
template <bool BF16, int EM>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(RouteBwdParams p) {
  constexpr int NB = EM <= 8 ? 8 : 4;   // tokens whose dx is in flight at once
  __shared__ __attribute__((aligned(16))) float sdl[RB_DX_TOK][EM];
  const int E = p.E, d = p.d;
  const int t0 = blockIdx.y * RB_DX_TOK;
  const int c8 = blockIdx.x * RB_DX_COLS + 8 * threadIdx.x;
  for (int i = threadIdx.x; i < RB_DX_TOK * EM; i += 256) {
    const int tt = i / EM, e = i % EM;
    const int t = t0 + tt;
    sdl[tt][e] = (t < p.T && e < E) ? p.dlogits[(size_t)t * E + e] : 0.0f;
  }
  __syncthreads();
  if (c8 >= d) return;
  float wv[EM][8];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    if (e < E) {
      const float4 a = *(const float4*)&p.w_router[(size_t)e * d + c8];
      const float4 b = *(const float4*)&p.w_router[(size_t)e * d + c8 + 4];
      wv[e][0] = a.x; wv[e][1] = a.y; wv[e][2] = a.z; wv[e][3] = a.w;
      wv[e][4] = b.x; wv[e][5] = b.y; wv[e][6] = b.z; wv[e][7] = b.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[e][q] = 0.0f;
    }
  }
  const int nt = min(RB_DX_TOK, p.T - t0);
  // the sum of token tt's dL row against the 8 columns' weights, expert order
  auto sums = [&](int tt, float (&a)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = 0.0f;
#pragma unroll
    for (int e4 = 0; e4 < EM / 4; ++e4) {
      const float4 v = *(const float4*)&sdl[tt][4 * e4];
      const float lv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = fmaf(lv[u], wv[4 * e4 + u][q], a[q]);
    }
  };
  if constexpr (BF16) {
    uint16_t* const dx = (uint16_t*)p.dx;
    auto update = [&](int tt, const rb_u32x4& v) {
      float a[8];
      sums(tt, a);
      rb_u32x4 o;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float lo = __fadd_rn(bf16_bits_to_f32(v[h] & 0xFFFFu), a[2 * h]);
        const float hi = __fadd_rn(bf16_bits_to_f32(v[h] >> 16), a[2 * h + 1]);
        o[h] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
      }
      *(rb_u32x4*)(dx + (size_t)(t0 + tt) * d + c8) = o;
    };
    int tb = 0;
    for (; tb + NB <= nt; tb += NB) {   // NB tokens' loads, unconditionally, before the updates
      rb_u32x4 v[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) v[j] = *(const rb_u32x4*)(dx + (size_t)(t0 + tb + j) * d + c8);
#pragma unroll
      for (int j = 0; j < NB; ++j) update(tb + j, v[j]);
    }
    for (; tb < nt; ++tb) update(tb, *(const rb_u32x4*)(dx + (size_t)(t0 + tb) * d + c8));
  } else {
    float* const dx = (float*)p.dx;
    auto update = [&](int tt, const float4& v0, const float4& v1) {
      float a[8];
      sums(tt, a);
      const float4 r0 = make_float4(__fadd_rn(v0.x, a[0]), __fadd_rn(v0.y, a[1]), __fadd_rn(v0.z, a[2]),
                                    __fadd_rn(v0.w, a[3]));
      const float4 r1 = make_float4(__fadd_rn(v1.x, a[4]), __fadd_rn(v1.y, a[5]), __fadd_rn(v1.z, a[6]),
                                    __fadd_rn(v1.w, a[7]));
      *(float4*)(dx + (size_t)(t0 + tt) * d + c8) = r0;
      *(float4*)(dx + (size_t)(t0 + tt) * d + c8 + 4) = r1;
    };
    int tb = 0;
    for (; tb + NB <= nt; tb += NB) {   // NB tokens' loads, unconditionally, before the updates
      float4 v[NB][2];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        v[j][0] = *(const float4*)(dx + (size_t)(t0 + tb + j) * d + c8);
        v[j][1] = *(const float4*)(dx + (size_t)(t0 + tb + j) * d + c8 + 4);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) update(tb + j, v[j][0], v[j][1]);
    }
    for (; tb < nt; ++tb)
      update(tb, *(const float4*)(dx + (size_t)(t0 + tb) * d + c8), *(const float4*)(dx + (size_t)(t0 + tb) * d + c8 + 4));
  }
}

// moe_backward's dx in one pass (bf16, top-1 or top-2, up to 16 experts): the sum of the token's
// kept slots' dXp rows in slot order (as the gather backward forms it), then its shared-expert dXs
// row, then the router term sum_e dL[t, e] W_r[e], in fp32, rounded once to act. The gather
// backward and the router's share then need no dx written and read back between them. Layout
// as route_bwd_dx_kernel; the rows of 4 tokens (their slots' and shared rows, 16 bytes each per
// thread) are loaded before any of them is summed, dropped slots' rows clamped to row 0 and masked.
constexpr int RB_DXG_TOK = 32;   // tokens per block of route_bwd_dx_gather_kernel
constexpr int RB_DXG_NB = 4;     // tokens whose rows are in flight at once
template <int EM>
__global__ __launch_bounds__(256) void route_bwd_dx_gather_kernel(RouteBwdParams p) {
  constexpr int NB = RB_DXG_NB;
  __shared__ __attribute__((aligned(16))) float sdl[RB_DXG_TOK][EM];
  __shared__ int srow[RB_DXG_TOK][2];
  const int E = p.E, d = p.d, k = p.k;
  const int t0 = blockIdx.y * RB_DXG_TOK;
  const int c8 = blockIdx.x * RB_DX_COLS + 8 * threadIdx.x;
  for (int i = threadIdx.x; i < RB_DXG_TOK * EM; i += 256) {
    const int tt = i / EM, e = i % EM;
    const int t = t0 + tt;
    sdl[tt][e] = (t < p.T && e < E) ? p.dlogits[(size_t)t * E + e] : 0.0f;
  }
  for (int i = threadIdx.x; i < RB_DXG_TOK * 2; i += 256) {
    const int tt = i >> 1, j = i & 1, t = t0 + tt;
    const int r = (t < p.T && j < k) ? p.row_of[(size_t)t * k + j] : -1;
    srow[tt][j] = (r >= 0 && r < p.max_rows) ? r : -1;
  }
  __syncthreads();
  if (c8 >= d) return;
  float wv[EM][8];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    if (e < E) {
      const float4 a = *(const float4*)&p.w_router[(size_t)e * d + c8];
      const float4 b = *(const float4*)&p.w_router[(size_t)e * d + c8 + 4];
      wv[e][0] = a.x; wv[e][1] = a.y; wv[e][2] = a.z; wv[e][3] = a.w;
      wv[e][4] = b.x; wv[e][5] = b.y; wv[e][6] = b.z; wv[e][7] = b.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[e][q] = 0.0f;
    }
  }
  const int nt = min(RB_DXG_TOK, p.T - t0);
  const uint16_t* const dxp = (const uint16_t*)p.dxp;
  const uint16_t* const dxs = (const uint16_t*)p.dxs;
  uint16_t* const dx = (uint16_t*)p.dx;
  const bool sh = dxs != nullptr;
  auto load = [&](int tt, rb_u32x4 (&v)[3]) {
    v[0] = *(const rb_u32x4*)(dxp + (size_t)max(srow[tt][0], 0) * d + c8);
    v[1] = *(const rb_u32x4*)(dxp + (size_t)max(srow[tt][1], 0) * d + c8);
    if (sh) v[2] = *(const rb_u32x4*)(dxs + (size_t)(t0 + tt) * d + c8);
  };
  auto update = [&](int tt, const rb_u32x4 (&v)[3]) {
    float a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = 0.0f;
#pragma unroll
    for (int e4 = 0; e4 < EM / 4; ++e4) {
      const float4 l = *(const float4*)&sdl[tt][4 * e4];
      const float lv[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = fmaf(lv[u], wv[4 * e4 + u][q], a[q]);
    }
    const bool h0 = srow[tt][0] >= 0, h1 = srow[tt][1] >= 0;
    rb_u32x4 o;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float s2[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int sft = 16 * b;
        float g = h0 ? fmaf(1.0f, bf16_bits_to_f32((v[0][h] >> sft) & 0xFFFFu), 0.0f) : 0.0f;
        g = h1 ? fmaf(1.0f, bf16_bits_to_f32((v[1][h] >> sft) & 0xFFFFu), g) : g;
        if (sh) g = __fadd_rn(g, bf16_bits_to_f32((v[2][h] >> sft) & 0xFFFFu));
        s2[b] = __fadd_rn(g, a[2 * h + b]);
      }
      o[h] = f32_to_bf16_bits(s2[0]) | (f32_to_bf16_bits(s2[1]) << 16);
    }
    *(rb_u32x4*)(dx + (size_t)(t0 + tt) * d + c8) = o;
  };
  int tb = 0;
  for (; tb + NB <= nt; tb += NB) {   // NB tokens' rows, unconditionally, before the sums
    rb_u32x4 v[NB][3];
#pragma unroll
    for (int j = 0; j < NB; ++j) load(tb + j, v[j]);
#pragma unroll
    for (int j = 0; j < NB; ++j) update(tb + j, v[j]);
  }
  for (; tb < nt; ++tb) {
    rb_u32x4 v[3];
    load(tb, v);
    update(tb, v);
  }
}

bool route_bwd_fuses_gather(bool bf16, int E, int k) { return bf16 && E <= 16 && k <= 2; }

template <bool BF16, int EM>
__global__ __launch_bounds__(256) void route_bwd_dx1_kernel(RouteBwdParams p) {
  __shared__ __attribute__((aligned(16))) float sdl[RB_TOK][EM];
  const int E = p.E, d = p.d;
  const int t0 = blockIdx.y * RB_TOK;
  const int c = blockIdx.x * 256 + threadIdx.x;
  for (int i = threadIdx.x; i < RB_TOK * EM; i += 256) {
    const int tt = i / EM, e = i % EM;
    const int t = t0 + tt;
    sdl[tt][e] = (t < p.T && e < E) ? p.dlogits[(size_t)t * E + e] : 0.0f;
  }
  __syncthreads();
  if (c >= d) return;
  float wv[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) wv[e] = e < E ? p.w_router[(size_t)e * d + c] : 0.0f;
  const int nt = min(RB_TOK, p.T - t0);
  for (int tt = 0; tt < nt; ++tt) {
    float a = 0.0f;
#pragma unroll
    for (int e4 = 0; e4 < EM / 4; ++e4) {
      const float4 v = *(const float4*)&sdl[tt][4 * e4];
      a = fmaf(v.x, wv[4 * e4], a);
      a = fmaf(v.y, wv[4 * e4 + 1], a);
      a = fmaf(v.z, wv[4 * e4 + 2], a);
      a = fmaf(v.w, wv[4 * e4 + 3], a);
    }
    const size_t o = (size_t)(t0 + tt) * d + c;
    if constexpr (BF16) {
      uint16_t* dx = (uint16_t*)p.dx;
      dx[o] = (uint16_t)f32_to_bf16_bits(__fadd_rn(bf16_bits_to_f32(dx[o]), a));
    } else {
      float* dx = (float*)p.dx;
      dx[o] = __fadd_rn(dx[o], a);
    }
  }
}

// dW_r[e, c] = sum_t dL[t, e] x[t, c]: a [E, T] x [T, d] product, split over token chunks. A
// column thread owns 8 consecutive columns (one 16-byte load of x per token for bf16, two for
// fp32) and their 8 EM sums; a block covers 2048 columns of one chunk with two such threads per
// column group (512 threads: two waves per SIMD, so one's FMAs overlap the other's loads). The
// chunk's dL rows stream through LDS 64 tokens at a time and are read back as 16-byte vectors
// (the same address for every lane); half h of the block takes tokens 32 h .. 32 h + 31 of every
// 64, with 16 tokens' loads (8 with 16 experts; 4 for fp32) issued before their FMAs. The two
// halves' sums are added (half 0 + half 1) through LDS. Chunk partials [chunks, E, d] are summed
// in a fixed order by route_bwd_reduce_kernel (deterministic).
constexpr int RB_COLS = 2048;   // columns per block (256 column threads x 8)
template <bool BF16, int EM>
__global__ __launch_bounds__(512) void route_bwd_w_kernel(RouteBwdParams p) {
  __shared__ __attribute__((aligned(16))) float sdl[RB_TOK][EM];
  __shared__ __attribute__((aligned(16))) float xch[8][256][8];   // half 1's sums, 8 experts at a time
  const int E = p.E, d = p.d;
  const int ct = threadIdx.x & 255, half = threadIdx.x >> 8;
  const int c8 = blockIdx.x * RB_COLS + 8 * ct;
  const bool active = c8 < d;
  const int tb = blockIdx.y * p.chunk_tokens;
  const int te = min(p.T, tb + p.chunk_tokens);
  float acc[EM][8];
#pragma unroll
  for (int e = 0; e < EM; ++e)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[e][q] = 0.0f;
  auto load8 = [&](int t, float (&xv)[8]) {
    if constexpr (BF16) {
      const uint4 u = *(const uint4*)((const uint16_t*)p.x + (size_t)t * d + c8);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[2 * q] = bf16_bits_to_f32(w4[q] & 0xFFFFu);
        xv[2 * q + 1] = bf16_bits_to_f32(w4[q] >> 16);
      }
    } else {
      const float4 a = *(const float4*)((const float*)p.x + (size_t)t * d + c8);
      const float4 b = *(const float4*)((const float*)p.x + (size_t)t * d + c8 + 4);
      xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
      xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
    }
  };
  auto fma_token = [&](int tt, const float (&xv)[8]) {
#pragma unroll
    for (int e4 = 0; e4 < EM / 4; ++e4) {
      const float4 l = *(const float4*)&sdl[tt][4 * e4];
      const float lv[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[4 * e4 + u][q] = fmaf(lv[u], xv[q], acc[4 * e4 + u][q]);
    }
  };
  for (int t0 = tb; t0 < te; t0 += RB_TOK) {
    __syncthreads();
    for (int i = threadIdx.x; i < RB_TOK * EM; i += 512) {
      const int tt = i / EM, e = i % EM;
      const int t = t0 + tt;
      sdl[tt][e] = (t < te && e < E) ? p.dlogits[(size_t)t * E + e] : 0.0f;
    }
    __syncthreads();
    if (active) {
      const int h0 = half * (RB_TOK / 2);
      const int nt = min(RB_TOK / 2, te - t0 - h0);   // this half's tokens of the batch (may be <= 0)
      int tt = 0;
      if constexpr (BF16) {
        // NB tokens' 16-byte loads before their FMAs (token order is kept for the sums)
        constexpr int NB = EM <= 8 ? 16 : 8;
        for (; tt + NB <= nt; tt += NB) {
          rb_u32x4 u[NB];
#pragma unroll
          for (int j = 0; j < NB; ++j)
            u[j] = *(const rb_u32x4*)((const uint16_t*)p.x + (size_t)(t0 + h0 + tt + j) * d + c8);
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            float xv[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              xv[2 * q] = bf16_bits_to_f32(u[j][q] & 0xFFFFu);
              xv[2 * q + 1] = bf16_bits_to_f32(u[j][q] >> 16);
            }
            fma_token(h0 + tt + j, xv);
          }
        }
      } else {
        for (; tt + 4 <= nt; tt += 4) {   // four tokens' loads before their FMAs, in token order
          float x0[8], x1[8], x2[8], x3[8];
          load8(t0 + h0 + tt, x0);
          load8(t0 + h0 + tt + 1, x1);
          load8(t0 + h0 + tt + 2, x2);
          load8(t0 + h0 + tt + 3, x3);
          fma_token(h0 + tt, x0);
          fma_token(h0 + tt + 1, x1);
          fma_token(h0 + tt + 2, x2);
          fma_token(h0 + tt + 3, x3);
        }
      }
      for (; tt < nt; ++tt) {
        float xv[8];
        load8(t0 + h0 + tt, xv);
        fma_token(h0 + tt, xv);
      }
    }
  }
  // half 0 += half 1, 8 experts at a time through LDS
  float* part = p.part + (size_t)blockIdx.y * E * d;
#pragma unroll
  for (int eb = 0; eb < EM; eb += 8) {
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        *(float4*)&xch[e][ct][0] = make_float4(acc[eb + e][0], acc[eb + e][1], acc[eb + e][2], acc[eb + e][3]);
        *(float4*)&xch[e][ct][4] = make_float4(acc[eb + e][4], acc[eb + e][5], acc[eb + e][6], acc[eb + e][7]);
      }
    }
    __syncthreads();
    if (half == 0 && active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (eb + e >= E) continue;
        const float4 a = *(const float4*)&xch[e][ct][0];
        const float4 b = *(const float4*)&xch[e][ct][4];
        *(float4*)&part[(size_t)(eb + e) * d + c8] =
            make_float4(acc[eb + e][0] + a.x, acc[eb + e][1] + a.y, acc[eb + e][2] + a.z, acc[eb + e][3] + a.w);
        *(float4*)&part[(size_t)(eb + e) * d + c8 + 4] =
            make_float4(acc[eb + e][4] + b.x, acc[eb + e][5] + b.y, acc[eb + e][6] + b.z, acc[eb + e][7] + b.w);
      }
    }
  }
}

// The same product for 32 or 64 experts (8 columns' sums per thread would not fit in registers):
// one column per thread, 256 columns per block, the same chunks and partial layout.
template <bool BF16, int EM>
__global__ __launch_bounds__(256) void route_bwd_w1_kernel(RouteBwdParams p) {
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

// dW_r = the chunk partials summed in a fixed order: the chunks fall into RB_RG contiguous groups,
// each summed in chunk order by one thread (4 consecutive outputs, 16-byte loads, 8 chunks' loads
// in flight), and the group sums are added in group order. A block covers 16 output quads x the
// RB_RG groups. db[e] = sum_t dL[t, e] (a fixed-order tree over 256 strided partial sums), from
// the blocks of the last grid row.
constexpr int RB_RG = 16;
__global__ __launch_bounds__(256) void route_bwd_reduce_kernel(RouteBwdParams p) {
  if (blockIdx.y == 0) {
    __shared__ float4 red[RB_RG][16];
    const int nq = p.E * p.d / 4;   // output quads
    const int oq = threadIdx.x & 15, g = threadIdx.x >> 4;
    const int q = blockIdx.x * 16 + oq;
    if (!p.dw_router) return;
    const int c0 = g * p.chunks / RB_RG, c1 = (g + 1) * p.chunks / RB_RG;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (q < nq) {
      const float4* __restrict__ part = (const float4*)p.part;
      int ch = c0;
      for (; ch + 8 <= c1; ch += 8) {
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = part[(size_t)(ch + j) * nq + q];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc.x += v[j].x;
          acc.y += v[j].y;
          acc.z += v[j].z;
          acc.w += v[j].w;
        }
      }
      for (; ch < c1; ++ch) {
        const float4 v = part[(size_t)ch * nq + q];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
    red[g][oq] = acc;
    __syncthreads();
    if (g == 0 && q < nq) {
      float4 s = red[0][oq];
      for (int j = 1; j < RB_RG; ++j) {
        const float4 v = red[j][oq];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      }
      ((float4*)p.dw_router)[q] = s;
    }
    return;
  }
  // blockIdx.y == 1: bias gradient, expert blockIdx.x
  __shared__ float red[256];
  const int e = blockIdx.x;
  if (e >= p.E || !p.dbias) return;
  float acc = 0.0f;
  int t = threadIdx.x;
  for (; t + 15 * 256 < p.T; t += 16 * 256) {   // 16 loads in flight, added in token order
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p.dlogits[(size_t)(t + j * 256) * p.E + e];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += v[j];
  }
  for (; t < p.T; t += 256) acc += p.dlogits[(size_t)t * p.E + e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int m = 128; m >= 1; m >>= 1) {
    if ((int)threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.dbias[e] = red[0];
}

// token chunks of the router weight gradient: about 512 blocks of 2048 columns in all, chunks a
// multiple of 64 tokens long; the partials take chunks * E * d fp32, chunks <= 512 / ceil(d / 2048).
void route_bwd_chunks(int T, int d, int* chunks, int* chunk_tokens) {
  const int col_tiles = (d + RB_COLS - 1) / RB_COLS;
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
  if (p.dx && p.dxp) {   // dx formed from the gather and the router term (route_bwd_fuses_gather)
    if (!route_bwd_fuses_gather(bf16, p.E, p.k)) return hipErrorInvalidValue;
    dim3 g((p.d + RB_DX_COLS - 1) / RB_DX_COLS, (p.T + RB_DXG_TOK - 1) / RB_DXG_TOK);
    if (p.E <= 8) route_bwd_dx_gather_kernel<8><<<g, 256, 0, s>>>(p);
    else route_bwd_dx_gather_kernel<16><<<g, 256, 0, s>>>(p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  } else if (p.dx) {
    dim3 g((p.d + RB_DX_COLS - 1) / RB_DX_COLS, (p.T + RB_DX_TOK - 1) / RB_DX_TOK);
#define MOE_RBDX(K, EMV)                                                     \
    if (bf16) K<true, EMV><<<g, 256, 0, s>>>(p);                             \
    else K<false, EMV><<<g, 256, 0, s>>>(p);
    if (p.E <= 8) { MOE_RBDX(route_bwd_dx_kernel, 8) }
    else if (p.E <= 16) { MOE_RBDX(route_bwd_dx_kernel, 16) }
    else {
      g.x = (p.d + 255) / 256;
      g.y = (p.T + RB_TOK - 1) / RB_TOK;
      if (p.E <= 32) { MOE_RBDX(route_bwd_dx1_kernel, 32) }
      else { MOE_RBDX(route_bwd_dx1_kernel, 64) }
    }
#undef MOE_RBDX
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (p.dw_router) {
    dim3 g((p.d + RB_COLS - 1) / RB_COLS, p.chunks);
#define MOE_RBW(K, EMV, NT)                                                  \
    if (bf16) K<true, EMV><<<g, NT, 0, s>>>(p);                              \
    else K<false, EMV><<<g, NT, 0, s>>>(p);
    if (p.E <= 8) { MOE_RBW(route_bwd_w_kernel, 8, 512) }
    else if (p.E <= 16) { MOE_RBW(route_bwd_w_kernel, 16, 512) }
    else {
      g.x = (p.d + 255) / 256;
      if (p.E <= 32) { MOE_RBW(route_bwd_w1_kernel, 32, 256) }
      else { MOE_RBW(route_bwd_w1_kernel, 64, 256) }
    }
#undef MOE_RBW
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (p.dw_router || p.dbias) {
    const size_t nq = (size_t)p.E * p.d / 4;
    const int gx = (int)std::max<size_t>((nq + 15) / 16, (size_t)p.E);
    route_bwd_reduce_kernel<<<dim3(gx, 2), 256, 0, s>>>(p);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
