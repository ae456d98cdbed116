// Grouped expert GEMM: for every expert e and every row r of its segment
// [offsets[e], offsets[e+1]) of the permuted activations,
//   C[r, n] = act( sum_k A[r, k] * B[e, n, k] ),   act = SiLU (first layer) or identity.
// [P4 §2.4] each expert is a two-layer FFN; the layer runs all experts' segments in one launch
// instead of a loop over experts. Both operands are K-contiguous (B is [out, in] per expert).
//
// Tiling: a workgroup of 4 waves computes a 128 x 128 tile of C; each wave a 64 x 64 quarter as
// 4 x 4 MFMA tiles of 16 x 16 (bf16: v_mfma_f32_16x16x32_bf16; fp32: v_mfma_f32_16x16x4_f32).
// K is staged through LDS 128 bytes per row at a time (64 bf16 or 32 fp32), with the next
// slice prefetched into registers while the current one is multiplied. The variable rows per
// expert are handled on the device: the m-tiles of all experts are numbered consecutively
// (expert by expert) from the offsets, and blockIdx.x picks one; blocks past the last tile exit.
// blockIdx.y is the output column tile.
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int LDS_ROW = 128 + 16;  // bytes per staged row: 128 data + 16 pad (bank spread)
}

template <bool BF16, bool SILU>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr int BM = GEMM_BM, BN = GEMM_BN;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int BK = 128 / ESZ;
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BN * LDS_ROW];
  __shared__ int s_off[MOE_MAX_EXPERTS_DEV + 1];
  __shared__ int s_tile[MOE_MAX_EXPERTS_DEV + 1];

  const int tid = threadIdx.x;
  const int E = p.E;
  if (tid == 0) {
    // clamp the segment bounds into [0, max_rows] and make them non-decreasing, so that no
    // offsets value can send a block outside the buffers
    int prev = 0, tiles = 0;
    for (int e = 0; e <= E; ++e) {
      int o = p.offsets[e];
      o = o < prev ? prev : (o > p.max_rows ? p.max_rows : o);
      s_off[e] = o;
      if (e > 0) {
        s_tile[e - 1] = tiles;
        tiles += (o - prev + BM - 1) / BM;
      }
      prev = o;
    }
    s_tile[E] = tiles;
  }
  __syncthreads();
  const int mt = blockIdx.x;
  if (mt >= s_tile[E]) return;
  int e = 0;
  while (s_tile[e + 1] <= mt) ++e;
  const int row0 = s_off[e] + (mt - s_tile[e]) * BM;
  const int row_end = s_off[e + 1];
  const int n0 = blockIdx.y * BN;
  const int N = p.N, K = p.K;
  const size_t rowA = (size_t)K * ESZ;  // bytes per row of A and of B
  const uint8_t* __restrict__ A = (const uint8_t*)p.A;
  const uint8_t* __restrict__ B = (const uint8_t*)p.B + (size_t)e * N * rowA;

  // global -> register staging: thread loads 4 16-byte chunks of A and 4 of B per K slice
  const int lr = tid >> 3;          // tile row (plus 32 * i)
  const int lc = tid & 7;           // 16-byte chunk within the 128-byte slice
  uint4 ra[4], rb[4];
  auto load_slice = [&](int kt) {
    const int kbyte = kt * 128 + lc * 16;
    const bool kin = kbyte < (int)rowA;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 32 * i;
      const int ga = row0 + r;
      const int gb = n0 + r;
      ra[i] = (kin && ga < row_end) ? *(const uint4*)(A + (size_t)ga * rowA + kbyte) : make_uint4(0, 0, 0, 0);
      rb[i] = (kin && gb < N) ? *(const uint4*)(B + (size_t)gb * rowA + kbyte) : make_uint4(0, 0, 0, 0);
    }
  };

  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int fr = lane & 15, fg = lane >> 4;
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((rowA + 127) / 128);
  load_slice(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(uint4*)(sA + (lr + 32 * i) * LDS_ROW + lc * 16) = ra[i];
      *(uint4*)(sB + (lr + 32 * i) * LDS_ROW + lc * 16) = rb[i];
    }
    __syncthreads();
    if (kt + 1 < nk) load_slice(kt + 1);
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          af[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sA + (wm * 64 + i * 16 + fr) * LDS_ROW + ks * 64 + fg * 16));
          bfr[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sB + (wn * 64 + i * 16 + fr) * LDS_ROW + ks * 64 + fg * 16));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        float af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          af[i] = *(const float*)(sA + (wm * 64 + i * 16 + fr) * LDS_ROW + (ks * 4 + fg) * 4);
          bfr[i] = *(const float*)(sB + (wn * 64 + i * 16 + fr) * LDS_ROW + (ks * 4 + fg) * 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds C rows 4*fg .. 4*fg+3 of column fr of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wm * 64 + i * 16 + 4 * fg + r;
        if (row < row_end && col < N) {
          float v = acc[i][j][r];
          if (SILU && p.C2) {   // the pre-activation, rounded once
            if constexpr (BF16)
              ((uint16_t*)p.C2)[(size_t)row * N + col] = (uint16_t)f32_to_bf16_bits(v);
            else
              ((float*)p.C2)[(size_t)row * N + col] = v;
          }
          if (SILU) v = v / (1.0f + expf(-v));
          if constexpr (BF16)
            ((uint16_t*)p.C)[(size_t)row * N + col] = (uint16_t)f32_to_bf16_bits(v);
          else
            ((float*)p.C)[(size_t)row * N + col] = v;
        }
      }
    }
  }
}

int gemm_max_mtiles(int max_rows, int E) { return (max_rows + GEMM_BM - 1) / GEMM_BM + E; }

// The 256 x 256 kernel loads up to three K stages ahead across its tiles, so it needs at least
// four stages (K >= 256) per tile; shorter reductions take the 128 x 128 kernel.
bool gemm_uses_big(bool bf16, int K, int max_rows, int E) {
  return bf16 && K % 64 == 0 && K >= 256 && max_rows >= 256 * E;
}

// The weight-streaming kernel: bf16, K a multiple of 64, at most 64 rows per expert on average
// (and not the 256 x 256 kernel's case).
bool gemm_uses_stream(bool bf16, int K, int max_rows, int E) {
  return !gemm_uses_big(bf16, K, max_rows, E) && bf16 && K % 64 == 0 && max_rows <= 64 * E;
}

hipError_t launch_gemm(const GemmParams& p, bool bf16, bool silu, hipStream_t s) {
  // bf16 with K a multiple of 64 (at least 128): on average at least 256 rows per expert, 256 x 256
  // tiles; at most 64, one pass over the expert weights. Weights stored [K, N] (p.b_kn) are read by
  // those two kernels only.
  if (gemm_uses_big(bf16, p.K, p.max_rows, p.E)) return launch_gemm_big(p, silu, s);
  if (gemm_uses_stream(bf16, p.K, p.max_rows, p.E)) return launch_gemm_stream(p, silu, s);
  if (p.b_kn) return hipErrorInvalidValue;
  dim3 grid(gemm_max_mtiles(p.max_rows, p.E), (p.N + GEMM_BN - 1) / GEMM_BN);
  if (bf16) {
    if (silu) gemm_kernel<true, true><<<grid, 256, 0, s>>>(p);
    else gemm_kernel<true, false><<<grid, 256, 0, s>>>(p);
  } else {
    if (silu) gemm_kernel<false, true><<<grid, 256, 0, s>>>(p);
    else gemm_kernel<false, false><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
