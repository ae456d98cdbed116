// Grouped expert GEMM, large-segment variant (bf16): a 256 x 256 output tile per workgroup.
//
//   C[r, n] = act( sum_k A[r, k] * B[e, n, k] ),  r in expert e's segment of the permuted rows,
// with act = SiLU for the first FFN layer (P4 §2.4: every expert is a two-layer FFN).
//
// Layout of the work:
//  * 4 waves in a 2 x 2 arrangement, each owning a 128 x 128 quarter of the tile as 8 x 8
//    v_mfma_f32_16x16x32_bf16 blocks (256 fp32 accumulators per lane, kept in AGPRs). On this
//    chip the 16x16x32 form sustains a higher rate than 32x32x16.
//  * K advances 64 elements (128 bytes of every row, whole 128-byte lines) per stage. Two LDS
//    stages (2 x (A + B) x 256 rows x 128 B = 128 KiB) are filled by gfx950's direct global ->
//    LDS 16-byte loads, so no registers stage the data; stage s + 1 is requested when stage s
//    starts.
//  * A stage is two k-steps of 32. Operand fragments are read one k-step ahead, interleaved
//    with the MFMAs. The one barrier per stage sits in the middle of the second k-step: after it
//    stage s + 1 is complete in LDS and stage s's buffer is free, and the fragment reads of
//    stage s + 1 overlap the remaining MFMAs of stage s.
//  * LDS rows are 128 B with the eight 16-byte chunks XOR-swizzled by (row / 2) mod 8: 16 lanes
//    reading 16 consecutive rows at one chunk then touch all 64 banks once.
//  * The MFMA's first operand is the weight tile (its 16 rows are output features) and the
//    second the activation tile, so each lane ends with 4 consecutive output features of one
//    row: the epilogue (SiLU in fp32, one rounding to bf16) stores 8 bytes per lane.
//  * Tiles of all experts are numbered on the device from the segment offsets. Workgroup ids
//    are remapped so that each of the 8 XCDs (ids are dealt to XCDs round robin) works through
//    one contiguous range of tiles, ordered in groups of 4 m-tiles x all n-tiles, so that the
//    tiles running together on one XCD share rows of A and B in its L2.
// K must be a multiple of 64.
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int BIG_BM = 256, BIG_BN = 256;
constexpr int ROWB = 128;                     // staged bytes of one row per stage (64 bf16)
constexpr int TILE_BYTES = BIG_BM * ROWB;     // one operand, one stage: 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;   // A + B
constexpr int NSTAGE = 2;
constexpr int GROUP_M = 4;

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// SiLU(v) = v * sigmoid(v), fp32, with the hardware exp2 and reciprocal: the result is rounded
// to bf16 right after, far coarser than their error.
__device__ __forceinline__ float silu_fast(float v) {
  const float e = __builtin_amdgcn_exp2f(-v * 1.44269504088896341f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// acc += A * B on v_mfma_f32_16x16x32_bf16 with the accumulator bound to AGPRs. Written as inline
// asm so that all 256 accumulators of a lane stay in the AGPR file: left to itself the register
// allocator shuffles some of them through VGPRs inside the main loop. Same-shape MFMAs chained
// on one accumulator are interlocked by the hardware; the first read of the results after the
// loop is preceded by explicit wait states.
__device__ __forceinline__ void mfma_16x16x32(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// One direct global -> LDS 16-byte load per lane (gfx950 global_load_lds_dwordx4): lane l reads
// sbase + voff and writes LDS bytes [lds_addr + 16 l, lds_addr + 16 l + 16). M0 carries the LDS
// address and is restored afterwards. Issued as inline asm so that the compiler does not wait
// on it before unrelated LDS reads; the kernel counts these loads and waits (vmcnt) itself.
__device__ __forceinline__ void load_lds16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory");
}

__device__ __forceinline__ void wait_loads_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
}  // namespace

template <bool SILU>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int E = p.E, N = p.N;
  // Segment bounds, clamped into [0, max_rows] and made non-decreasing so that no offsets value
  // can send a block outside the buffers. Every lane walks the (uniform) offsets itself: the
  // LDS is entirely taken by the stage ring.
  auto bound = [&](int e, int prev) {
    const int o = p.offsets[e];
    return o < prev ? prev : (o > p.max_rows ? p.max_rows : o);
  };
  const int base0 = bound(0, 0);
  int MT = 0;
  {
    int prev = base0;
    for (int e = 1; e <= E; ++e) {
      const int o = bound(e, prev);
      MT += (o - prev + BIG_BM - 1) / BIG_BM;
      prev = o;
    }
  }
  const int NT = (N + BIG_BN - 1) / BIG_BN;
  const int total = MT * NT;
  const int wg = blockIdx.x;
  if (wg >= total) return;
  // XCD-aware remap: XCD x (= wg mod 8) takes a contiguous range of tile ids.
  const int q = total >> 3, rem = total & 7, xcd = wg & 7, local = wg >> 3;
  const int id = (xcd < rem) ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
  const int group = id / (GROUP_M * NT);
  const int first_m = group * GROUP_M;
  const int gm = min(GROUP_M, MT - first_m);
  const int in_group = id - group * GROUP_M * NT;
  const int mt = first_m + in_group % gm;
  const int nt = in_group / gm;
  int e = 0, row0 = 0, row_end = 0;
  {
    int prev = base0, tstart = 0;
    for (int ee = 0; ee < E; ++ee) {
      const int o = bound(ee + 1, prev);
      const int t = (o - prev + BIG_BM - 1) / BIG_BM;
      if (mt < tstart + t) {
        e = ee;
        row0 = prev + (mt - tstart) * BIG_BM;
        row_end = o;
        break;
      }
      tstart += t;
      prev = o;
    }
  }
  if (row_end <= row0) return;   // unreachable for mt < MT; keeps every address below in range
  const int n0 = nt * BIG_BN;
  const int rowbytes = p.K * 2;
  const uint8_t* __restrict__ A = (const uint8_t*)p.A;
  const uint8_t* __restrict__ B = (const uint8_t*)p.B + (size_t)e * N * rowbytes;

  // Direct loads: one instruction moves 16 rows x 64 B; lane l lands at byte 16 l of the
  // instruction's 1 KiB, i.e. row l / 4, slot l % 4, and loads the global chunk that the
  // swizzle puts in that slot. Wave w fills rows [64 w, 64 w + 64) of both tiles. Rows past the
  // segment (or past N) are clamped to a valid row: they only feed outputs the epilogue masks.
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t offA[8], offB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = w * 64 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (((i & 1) << 2) | (lane >> 4));
    const int ra = min(row0 + r, row_end - 1);
    const int rb = min(n0 + r, N - 1);
    offA[i] = (uint32_t)ra * (uint32_t)rowbytes + chunk * 16;
    offB[i] = (uint32_t)rb * (uint32_t)rowbytes + chunk * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int nk = rowbytes / ROWB;
  auto issue = [&](int kt) {
    const int st = min(kt, nk - 1);
    const uint8_t* akt = A + (size_t)st * ROWB;
    const uint8_t* bkt = B + (size_t)st * ROWB;
    const uint32_t sa = lds0 + (kt & 1) * STAGE_BYTES + w * 64 * ROWB;
    const uint32_t sb = sa + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      load_lds16(akt, offA[i], sa + i * 8 * ROWB);
      load_lds16(bkt, offB[i], sb + i * 8 * ROWB);
    }
  };

  const int wm = w >> 1, wn = w & 1;
  const int fr = lane & 15, fc = lane >> 4;   // fragment row within 16, 16-byte chunk
  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  bf16x8_t xa[2][8], wb[2][8];
  auto frag_x = [&](int buf, int stage, int ks, int i) {
    const uint8_t* sa = smem + (stage & 1) * STAGE_BYTES;
    xa[buf][i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sa + lds_off(wm * 128 + i * 16 + fr, ks * 4 + fc)));
  };
  auto frag_w = [&](int buf, int stage, int ks, int j) {
    const uint8_t* sb = smem + (stage & 1) * STAGE_BYTES + TILE_BYTES;
    wb[buf][j] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sb + lds_off(wn * 128 + j * 16 + fr, ks * 4 + fc)));
  };

  issue(0);
  wait_loads_all();
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) frag_x(0, 0, 0, i);
#pragma unroll
  for (int j = 0; j < 8; ++j) frag_w(0, 0, 0, j);

  for (int s = 0; s < nk; ++s) {
    issue(s + 1);   // past the end: a harmless reload into the idle buffer
    // k-step 0 of stage s from F0, reading k-step 1 of stage s into F1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma_16x16x32(acc[i][j], wb[0][j], xa[0][i]);
      frag_x(1, s, 1, i);
      frag_w(1, s, 1, i);
    }
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // first half of k-step 1
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma_16x16x32(acc[i][j], wb[1][j], xa[1][i]);
    __builtin_amdgcn_sched_barrier(0);
    // stage s + 1 has landed everywhere and nobody reads stage s's buffer any more
    wait_loads_all();
    __syncthreads();
    // second half of k-step 1, reading k-step 0 of stage s + 1 into F0
#pragma unroll
    for (int i = 4; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma_16x16x32(acc[i][j], wb[1][j], xa[1][i]);
      frag_x(0, s + 1, 0, 2 * (i - 4));
      frag_x(0, s + 1, 0, 2 * (i - 4) + 1);
      frag_w(0, s + 1, 0, 2 * (i - 4));
      frag_w(0, s + 1, 0, 2 * (i - 4) + 1);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_loads_all();
  // let the last MFMAs retire before their accumulators are read
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // epilogue: lane holds output features n = 4*(lane/16) + 0..3 of row m = lane % 16 of each
  // 16 x 16 block
  uint16_t* __restrict__ C = (uint16_t*)p.C;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = row0 + wm * 128 + i * 16 + fr;
    if (m >= row_end) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + wn * 128 + j * 16 + 4 * fc;
      if (n >= N) continue;
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = SILU ? silu_fast(acc[i][j][u]) : acc[i][j][u];
      uint2 o;
      o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *(uint2*)(C + (size_t)m * N + n) = o;
    }
    // one 16-row block at a time: keeps the epilogue from pulling every accumulator into VGPRs
    __builtin_amdgcn_sched_barrier(0);
  }
}

int gemm_big_grid(int max_rows, int E, int N) {
  return ((max_rows + BIG_BM - 1) / BIG_BM + E) * ((N + BIG_BN - 1) / BIG_BN);
}

hipError_t launch_gemm_big(const GemmParams& p, bool silu, hipStream_t s) {
  const int grid = gemm_big_grid(p.max_rows, p.E, p.N);
  if (silu) gemm_big_kernel<true><<<grid, 256, 0, s>>>(p);
  else gemm_big_kernel<false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
