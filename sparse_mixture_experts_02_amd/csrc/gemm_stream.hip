// Grouped expert GEMM, weight-streaming variant (bf16) for short expert segments.
//
//   C[r, n] = act( sum_k A[r, k] * B[e, n, k] ),  r in expert e's segment of the permuted rows,
// with act = SiLU for the first FFN layer (P4 §2.4: every expert is a two-layer FFN).
//
// With few tokens per expert (decode-sized batches, or a tight capacity) every weight element is
// used by only a handful of rows, so the product is bound by reading the expert weights from HBM
// once. The kernel is shaped for that:
//  * One workgroup per (expert, block of SB_N output features); it streams that weight block
//    (SB_N rows of B, all of K) exactly once and applies it to the expert's rows, 64 at a time
//    (a segment longer than 64 rows walks its row chunks, re-reading the block from L2 or HBM).
//  * Workgroups are ordered expert-major and dealt so that all blocks of one expert run on the
//    same XCD: the expert's activation rows are then fetched into one L2 only.
//  * K advances 64 elements (128 bytes of every row) per stage through an SB_STAGES-deep LDS
//    ring filled by direct buffer -> LDS loads (whole 128-byte lines), so SB_STAGES - 1 stages of
//    weights are in flight per workgroup to cover HBM latency.
//  * 4 waves; wave w owns output features [w SB_N/4, (w+1) SB_N/4) for all 64 rows of the chunk,
//    as v_mfma_f32_16x16x32_bf16 blocks with the weight fragment as the first operand.
//  * Rows are addressed through buffer resources sized to the valid rows (of the segment chunk,
//    and of B), so loads past the end fetch nothing; they only feed outputs that are not stored.
// K must be a multiple of 64 and N of 8.
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int SB_M = 64;                       // rows per chunk
constexpr int SB_N = 64;                       // output features per workgroup
constexpr int SB_STAGES = 4;
constexpr int SB_ROWB = 128;                   // bytes of one row per stage (64 bf16)
constexpr int SB_A_BYTES = SB_M * SB_ROWB;     // 8 KiB
constexpr int SB_B_BYTES = SB_N * SB_ROWB;     // 8 KiB
constexpr int SB_STAGE_BYTES = SB_A_BYTES + SB_B_BYTES;
constexpr int SB_NB = SB_N / 64;               // 16-feature blocks per wave
constexpr int SB_LOADS = (SB_M + SB_N) / 32;   // direct loads per wave per stage (8 rows each)

typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int sb_off(int row, int chunk) {
  return row * SB_ROWB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ float sb_silu(float v) {
  const float e = __builtin_amdgcn_exp2f(-v * 1.44269504088896341f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ i32x4_t sb_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// Direct buffer -> LDS 16-byte load per lane (lane l writes LDS [lds_addr + 16 l, + 16)).
__device__ __forceinline__ void sb_load(i32x4_t rsrc, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory");
}

template <int N>
__device__ __forceinline__ void sb_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef short sb_v4i16 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane s reads 8 bytes of
// row r0 + s / 4 at column c0 + 4 (s % 4), and lane i receives column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ sb_v4i16 sb_read_tr(const uint8_t* q) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) sb_v4i16*)(__attribute__((address_space(3))) const uint8_t*)q);
}
}  // namespace

// BT: the weights are stored [E][K][N] (the backward's dH and dXp read W2 and W1 as they are).
// A stage of the block is then 64 k-rows x the workgroup's 64 features, 128 bytes of each row,
// loaded as the [N, K] block's 64 rows are; the 32-byte quarters of k-row r are XOR-swizzled by
// f(r) = ((r >> 1) & 1) | (((r >> 3) & 1) << 1), and wave w reads its 16 features as MFMA operands
// with two transposing reads per operand (8 consecutive k per lane), as the 256 x 256 kernel's
// [K, N] variant does. Features past N get an offset outside the resource (zeros).
template <bool SILU, bool BT>
__global__ __launch_bounds__(256, 2) void gemm_stream_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[SB_STAGES * SB_STAGE_BYTES];

  const int E = p.E, N = p.N;
  const int NTB = (N + SB_N - 1) / SB_N;
  const int total = E * NTB;
  // expert-major tile order, a contiguous range per XCD (workgroup ids are dealt round robin)
  const int q = total >> 3, rem = total & 7, xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int id = (xcd < rem) ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
  if (local >= ((xcd < rem) ? q + 1 : q)) return;
  const int e = id / NTB, n0 = (id - e * NTB) * SB_N;
  // segment bounds, clamped into [0, max_rows]
  int lo = p.offsets[e], hi = p.offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > p.max_rows ? p.max_rows : lo);
  hi = hi < lo ? lo : (hi > p.max_rows ? p.max_rows : hi);
  if (hi <= lo) return;
  const int cols = min(N - n0, SB_N);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fc = lane >> 4;
  const int rowbytes = p.K * 2, nk = p.K / 64;
  const uint8_t* __restrict__ A = (const uint8_t*)p.A;
  const uint8_t* __restrict__ Bw = (const uint8_t*)p.B + ((size_t)e * N + n0) * rowbytes;
  const uint32_t nb2 = (uint32_t)N * 2u;   // BT: bytes of a [K, N] row
  const uint8_t* __restrict__ Bt = (const uint8_t*)p.B + (size_t)e * (size_t)p.K * nb2 + (size_t)n0 * 2u;
  uint16_t* __restrict__ C = (uint16_t*)p.C;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  // Load j of a wave moves 8 rows x 128 B: loads [0, SB_M / 32) fill activation rows
  // 16 w + 8 j + lane / 8, the rest weight rows; lane l lands at byte 16 l of the load's 1 KiB and
  // fetches the chunk that the swizzle puts there.
  uint32_t voff[SB_LOADS];
#pragma unroll
  for (int j = 0; j < SB_LOADS; ++j) {
    const bool a = j < SB_M / 32;
    const int jj = a ? j : j - SB_M / 32;
    const int r = (a ? w * (SB_M / 4) : w * (SB_N / 4)) + jj * 8 + (lane >> 3);
    if (BT && !a) {   // k-row r of the stage, slot lane % 8 holds chunk (lane % 8) ^ 2 f(r)
      const int chunk = (lane & 7) ^ ((((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1);
      voff[j] = 8 * chunk < cols ? (uint32_t)r * nb2 + (uint32_t)chunk * 16u : 0x80000000u;
    } else {
      const int chunk = (lane & 7) ^ ((r >> 1) & 7);   // the slot this lane fills holds that chunk
      voff[j] = (uint32_t)r * (uint32_t)rowbytes + chunk * 16;
    }
  }
  // BT fragment reads: lane (fr, fc) of wave w reads k-rows 8 fc + fr / 4 (+ 4) of its k-step,
  // bytes 8 (fr % 4) of quarter w ^ f(row)
  const uint32_t bt_rd = (uint32_t)((8 * fc + (fr >> 2)) * 128 + 8 * (fr & 3) + 32 * ((fr >> 3) | ((fc & 1) << 1))) ^
                         (uint32_t)(32 * w);

  for (int m0 = lo; m0 < hi; m0 += SB_M) {
    const int rows = min(hi - m0, SB_M);
    // stage kt (clamped to the last one: a harmless reload) into ring slot kt mod SB_STAGES
    auto issue = [&](int kt) {
      const int st = min(kt, nk - 1);
      const uint32_t base = lds0 + (kt % SB_STAGES) * SB_STAGE_BYTES;
      const i32x4_t rsa = sb_rsrc(A + (size_t)m0 * rowbytes + st * SB_ROWB, (uint32_t)rows * rowbytes);
      const i32x4_t rsb = BT ? sb_rsrc(Bt + (size_t)st * 64u * nb2, 64u * nb2)
                             : sb_rsrc(Bw + st * SB_ROWB, (uint32_t)cols * rowbytes);
#pragma unroll
      for (int j = 0; j < SB_LOADS; ++j) {
        const bool a = j < SB_M / 32;
        const int jj = a ? j : j - SB_M / 32;
        const uint32_t row = (a ? w * (SB_M / 4) : w * (SB_N / 4)) + jj * 8;
        sb_load(a ? rsa : rsb, voff[j], base + (a ? 0 : SB_A_BYTES) + row * SB_ROWB);
      }
    };

    f32x4_t acc[4][SB_NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < SB_NB; ++b) acc[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < SB_STAGES - 1; ++s) issue(s);
    for (int s = 0; s < nk; ++s) {
      sb_wait<(SB_STAGES - 2) * SB_LOADS>();   // stage s has landed (for this wave)
      __syncthreads();                          // ... for every wave; slot (s - 1) is free
      issue(s + SB_STAGES - 1);
      const uint8_t* sa = smem + (s % SB_STAGES) * SB_STAGE_BYTES;
      const uint8_t* sb = sa + SB_A_BYTES;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t xa[4], wb[SB_NB];
#pragma unroll
        for (int b = 0; b < SB_NB; ++b) {
          if constexpr (BT) {
            const uint8_t* q = sb + ks * 32 * 128 + bt_rd;
            const sb_v4i16 lo = sb_read_tr(q), hi = sb_read_tr(q + 4 * 128);
            wb[b] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            wb[b] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sb + sb_off(w * (SB_N / 4) + b * 16 + fr, ks * 4 + fc)));
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xa[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sa + sb_off(i * 16 + fr, ks * 4 + fc)));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int b = 0; b < SB_NB; ++b)
            acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[b], xa[i], acc[i][b], 0, 0, 0);
      }
    }
    sb_wait<0>();
    __syncthreads();   // the ring is reused by the next chunk

    // lane holds features n0 + 16 (4 w / 4 ...) + 4 fc .. + 3 of row m0 + 16 i + fr
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 16 + fr;
      if (r >= rows) continue;
#pragma unroll
      for (int b = 0; b < SB_NB; ++b) {
        const int n = w * (SB_N / 4) + b * 16 + 4 * fc;
        if (n >= cols) continue;
        float v[4];
        if (SILU && p.C2) {   // the pre-activation, rounded once
          uint2 a;
          a.x = pack_bf16x2(acc[i][b][0], acc[i][b][1]);
          a.y = pack_bf16x2(acc[i][b][2], acc[i][b][3]);
          *(uint2*)((uint16_t*)p.C2 + (size_t)(m0 + r) * N + n0 + n) = a;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = SILU ? sb_silu(acc[i][b][u]) : acc[i][b][u];
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *(uint2*)(C + (size_t)(m0 + r) * N + n0 + n) = o;
      }
    }
  }
}

int gemm_stream_grid(int E, int N) { return E * ((N + SB_N - 1) / SB_N); }

hipError_t launch_gemm_stream(const GemmParams& p, bool silu, hipStream_t s) {
  const int grid = gemm_stream_grid(p.E, p.N);
  if (p.b_kn && silu) return hipErrorInvalidValue;   // [K, N] weights: the backward's plain products
  if (p.b_kn) gemm_stream_kernel<false, true><<<grid, 256, 0, s>>>(p);
  else if (silu) gemm_stream_kernel<true, false><<<grid, 256, 0, s>>>(p);
  else gemm_stream_kernel<false, false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
