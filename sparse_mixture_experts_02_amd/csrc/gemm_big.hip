// Grouped expert GEMM, large-segment variant (bf16): persistent workgroups, 256 x 256 tiles.
//
//   C[r, n] = act( sum_k A[r, k] * B[e, n, k] ),  r in expert e's segment of the permuted rows,
// with act = SiLU for the first FFN layer (P4 §2.4: every expert is a two-layer FFN).
//
// Layout of the work:
//  * One workgroup per CU (the grid is at most 256 workgroups), each walking a list of output
//    tiles. Tiles of all experts are numbered on the device from the segment offsets; each of the
//    8 XCDs (workgroup ids are dealt to XCDs round robin) works through one contiguous range of
//    tile ids, ordered in groups of 4 m-tiles x all n-tiles so that the tiles running together on
//    one XCD share rows of A and B in its L2.
//  * 8 waves in a 2 x 4 arrangement, each owning 128 rows x 64 output features of the tile as
//    8 x 4 v_mfma_f32_16x16x32_bf16 blocks (128 fp32 accumulators per lane, kept in AGPRs). Wave w
//    and wave w + 4 run on the same SIMD (waves 0-3 are dealt to the four SIMDs, 4-7 likewise;
//    checked on the GPU from the hardware wave id), and they are the two 128-row halves of the
//    tile.
//  * K advances 64 elements (128 bytes of every row) per stage. Two LDS stages (2 x (A + B) x
//    256 rows x 128 B = 128 KiB) are filled by direct buffer -> LDS 16-byte loads.
//  * Ping-pong: the two halves (groups) take turns at the matrix cores. While one group issues
//    its 64 MFMAs of a stage, with no other instruction between them, the other reads its next
//    stage's fragments from LDS and issues its share of the direct loads; a barrier ends each
//    phase and the roles swap. Group 1 runs one phase behind group 0 for the whole kernel. The
//    loads of a stage are split evenly between the groups' memory phases, each issued as soon as
//    the rows it overwrites have been read by both groups, two phases before they are read.
//    Measured on the expert-FFN shapes against an interleaved schedule (both waves of a SIMD
//    mixing loads, fragment reads and MFMAs, one barrier per stage): GEMM2 441 -> 409 us and
//    GEMM1 482 -> 465 us on the main layer. With the loads removed the same loop runs GEMM2 at
//    1.58 PFLOP/s, so the direct loads are what is left between it and the matrix cores.
//  * Stages are numbered across a workgroup's tiles; past a tile's last stages the loads fetch
//    the next tile's first stages, so the pipeline runs through the tile boundary. A tile's
//    epilogue (SiLU in fp32, one rounding to bf16) falls in each group's memory phase, beside the
//    other group's MFMAs. This needs at least four stages per tile (K >= 256).
//  * The loads address rows through buffer resources whose size is the tile's valid rows of A (or
//    of B): rows past a segment's end or past N fall outside the resource and are not fetched.
//    They only feed accumulators whose outputs are never stored.
//  * Epilogue: the MFMA leaves 4 consecutive output features of one row per lane; it is turned
//    into whole output rows through a small per-wave LDS area (see the epilogue) and stored with
//    16-byte buffer stores, 8 rows x 128 contiguous bytes per instruction, through a buffer
//    resource sized to the tile's valid rows (lanes past N get an out-of-range offset).
// K must be a multiple of 64, at least 256, and N of 8.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

namespace {
constexpr int BIG_BM = 256, BIG_BN = 256;
constexpr int ROWB = 128;                     // staged bytes of one row per stage (64 bf16)
constexpr int TILE_BYTES = BIG_BM * ROWB;     // one operand, one stage: 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;   // A + B
constexpr int GROUP_M = 4;
constexpr int MAX_WGS = 256;                  // one workgroup per CU
constexpr int EPI_BYTES = 16 * 128;            // per wave: 16 output rows x 64 bf16

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// SiLU(v) = v * sigmoid(v), fp32, with the hardware exp2 and reciprocal: the result is rounded
// to bf16 right after, far coarser than their error.
__device__ __forceinline__ float silu_fast(float v) {
  const float e = __builtin_amdgcn_exp2f(-v * 1.44269504088896341f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// acc += A * B on v_mfma_f32_16x16x32_bf16 with the accumulator bound to AGPRs (inline asm keeps
// all 256 accumulators of a lane in the AGPR file). Same-shape MFMAs chained on one accumulator
// are interlocked by the hardware; the first read of the results after the loop is preceded by
// explicit wait states.
__device__ __forceinline__ void mfma_16x16x32(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Raw buffer resource (stride 0) over `bytes` bytes from `base`: lanes whose offset is at or past
// `bytes` are out of range (loads fetch nothing, stores write nothing).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// One direct buffer -> LDS 16-byte load per lane: lane l reads rsrc + voff and writes LDS bytes
// [lds_addr + 16 l, lds_addr + 16 l + 16). M0 carries the LDS address and is restored afterwards.
// Inline asm, so the compiler neither waits on it nor reorders it against the other inline asm;
// the kernel counts these loads and waits (vmcnt) itself.
__device__ __forceinline__ void load_lds16(i32x4_t rsrc, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory");
}

// The same with a uniform byte offset in the instruction's scalar offset register (it does not
// take a vector register per distinct offset).
__device__ __forceinline__ void load_lds16s(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}

// One 16-byte buffer store per lane; lanes that must not write carry an out-of-range offset. The
// output is not read again by this kernel, so it is stored with the non-temporal hint and does not
// displace the operand rows that the XCD's L2 is serving to the other tiles. The compiler does not
// see inside the asm, so the wait states that a store of more than 64 bits needs before a VALU
// instruction may overwrite its data registers are part of it.
__device__ __forceinline__ void store16(i32x4_t rsrc, uint32_t voff, u32x4_t v) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen nt\n\ts_nop 1" ::"v"(v), "v"(voff), "s"(rsrc) : "memory");
}

// Waits until every vector-memory operation of the wave has completed (the direct-to-LDS loads
// are not assumed to complete in issue order, so no partial count is used).
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct Tile {
  int e, row0, rows, n0, cols;
};

// fp32 partial sums of one 256 x 256 tile in the accumulator layout: [wave 8][16 x 16 block
// i * 4 + j 32][lane 64] x 16 bytes
constexpr uint32_t PART_BYTES = BIG_BM * BIG_BN * 4;

// Split of the last, partial round of tiles (when there is more than one round): the R tiles
// left over after whole rounds of G workgroups are each cut into s K-ranges (s the largest power
// of two with s R <= G, at most 8), so that s R workgroups share the last round instead of R. The
// parts' fp32 sums cost a write and a read of 256 KiB each and a second kernel; measured on the
// expert-FFN shapes this repays itself for reductions of at least 64 stages (K >= 4096) and not
// for 32, so shorter reductions are not split. Returns s (1: no split).
__device__ __forceinline__ int tail_parts(int total, int G, int nk) {
  const int R = total % G;
  if (total <= G || R == 0 || nk < 64) return 1;
  int s = 1;
  while (s < 8 && 2 * s * R <= G) s *= 2;
  return s;
}

// Narrow tiles for the partial last round of reductions under 64 stages, where splitting K does
// not repay its partial sums: when at most 64 tiles are left over after whole rounds of the 256
// workgroups, each is cut along N into s = 4 or 8 slices of 256 / s output features (s R <= 256),
// which the workgroups compute at full K after their whole tiles, so that s R workgroups share the
// last round instead of R and nothing is added up afterwards. A slice loads all 256 rows of A for
// 1 / s of the tile's products, so halves of full tiles cost more than they save (measured on the
// main expert-FFN layer: 160 halves of full tiles took longer than 80 whole tiles). The leftover
// tiles are the last ids, which hold the experts' partial m-tiles with the fewest rows (see
// decode_tile); when they all have at most 128 rows, halves (s = 2, R up to 128) pay: the waves
// whose rows are all past the tile's end skip their products, and A's missing rows are not
// fetched. tiny: the tiles are in that order and the leftover ones have at most 128 rows.
// Returns s (1: no narrow tail).
__device__ __forceinline__ int narrow_parts(int total, int G, int nk, bool tiny) {
  const int R = total % G;
  if (nk >= 64 || G != MAX_WGS || R == 0) return 1;
  if (4 * R <= G) return 8 * R <= G ? 8 : 4;
  return tiny ? 2 : 1;
}

// The m-tiles are numbered expert by expert (each expert's from its first row), or, when that
// makes the partial last round of a reduction under 64 stages hold at most 128 tiles, all of them
// partial m-tiles of at most 128 rows (see narrow_parts), every expert's full 256-row m-tiles
// first (expert order) and then the experts' partial last m-tiles, most rows first (ties: lower
// expert first), so that the partial last round holds the emptiest ones: its narrow slices then
// fetch fewer rows of A (small_bf16's GEMM1, 8 tiles left over as 32-feature slices: the 86-row
// m-tile instead of a 247-row one, 40.7 -> 37.7 us). (Sorting in every case measured slower where
// many experts have partial m-tiles: a group of m-tiles from different experts shares no weight
// rows in L2.) The order of the partial m-tiles is formed once per workgroup by one wave (lane e
// ranks expert e's remainder) into porder[]. seg: the clamped segment bounds in LDS.
__device__ __forceinline__ void order_partials(const int* seg, int E, int* porder) {
  const int lane = threadIdx.x & 63;
  if (lane >= E) return;
  const int mine = (seg[lane + 1] - seg[lane]) % BIG_BM;
  if (mine == 0) return;
  int rank = 0;
  for (int e = 0; e < E; ++e) {
    const int r = (seg[e + 1] - seg[e]) % BIG_BM;
    rank += (r > mine || (r == mine && e < lane)) ? 1 : 0;
  }
  porder[rank] = lane;
}

// Whether the sorted order applies (see above); returns the MF to decode with (0: expert order).
// total: the tiles, MT the m-tiles, MF0 the full m-tiles, G the workgroups, nk the stages. For 64
// stages or more, the leftover tiles of a K-split tail (split: the kernel splits, and the product
// allows it, GemmParams::sort_split) in the same way: the waves of a part whose rows all lie past
// the tile's end skip their products.
__device__ __forceinline__ int sorted_mf(int total, int MT, int MF0, int NT, int G, int nk, bool split,
                                         const int* seg, const int* porder) {
  const int R = total % G;
  if (G != MAX_WGS || MF0 == MT || R == 0 || 2 * R > G) return 0;
  if (nk >= 64 && !split) return 0;
  // the partial m-tiles that do not fit in the leftover round end up in groups of m-tiles from
  // different experts inside the whole rounds (no weight rows shared in L2): at most one group
  if ((MT - MF0) * NT - R > GROUP_M * NT) return 0;
  // the leftover tiles lie in m-tiles from the first of the group holding tile total - R on
  const int first_m = ((total - R) / (GROUP_M * NT)) * GROUP_M;
  if (first_m < MF0) return 0;
  const int ee = porder[first_m - MF0];   // the partial m-tile with the most rows among them
  return (seg[ee + 1] - seg[ee]) % BIG_BM <= 128 ? MF0 : 0;
}

// Tile id -> (expert, rows, output features): ids run over groups of GROUP_M m-tiles x all NT
// n-tiles, the m-tiles in the order above (MF > 0 with sorted partials: MF full m-tiles in expert
// order, then the partial ones in porder; MF = 0: expert by expert). The fields are wave-uniform
// and kept in scalar registers.
__device__ __forceinline__ Tile decode_tile(int id, int MT, int MF, int NT, int N, int E, const int* seg,
                                            const int* porder) {
  const int group = id / (GROUP_M * NT);
  const int first_m = group * GROUP_M;
  const int gm = min(GROUP_M, MT - first_m);
  const int in_group = id - group * GROUP_M * NT;
  const int mt = first_m + in_group % gm;
  const int nt = in_group / gm;
  Tile t{0, 0, 0, nt * BIG_BN, min(N - nt * BIG_BN, BIG_BN)};
  if (MF > 0 && mt >= MF) {
    const int ee = porder[mt - MF];
    const int len = seg[ee + 1] - seg[ee];
    t.e = ee;
    t.row0 = seg[ee] + (len / BIG_BM) * BIG_BM;
    t.rows = len % BIG_BM;
  } else {
    // expert by expert (MF = 0), or among the full m-tiles (rounding the counts down)
    const int round = MF > 0 ? 0 : BIG_BM - 1;
    int tstart = 0;
    for (int ee = 0; ee < E; ++ee) {
      const int lo = seg[ee], hi = seg[ee + 1];
      const int n = (hi - lo + round) / BIG_BM;
      if (mt < tstart + n) {
        t.e = ee;
        t.row0 = lo + (mt - tstart) * BIG_BM;
        t.rows = min(hi - t.row0, BIG_BM);
        break;
      }
      tstart += n;
    }
  }
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  t.rows = __builtin_amdgcn_readfirstlane(t.rows);
  t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
  t.cols = __builtin_amdgcn_readfirstlane(t.cols);
  return t;
}

// One 16-byte store of fp32 partial sums straight from the accumulator registers; the block's
// offset goes in the scalar offset. Includes the wait states a store of more than 64 bits needs
// before its data registers may be overwritten (the compiler does not see inside the asm).
__device__ __forceinline__ void store_part(i32x4_t rsrc, uint32_t voff, uint32_t soff, const f32x4_t& v) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, %3 offen\n\ts_nop 1" ::"a"(v), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}
}  // namespace

// A narrow-tail slice (see narrow_parts): 256 rows x BN (128, 64 or 32) output features of tile t
// from feature n0 (bcols valid) at full K, by the 8 waves of the workgroup after its whole tiles,
// in the whole-tile kernel's LDS: a 3-stage ring (A: 256 rows, B: max(BN, 64) rows, 128 bytes of
// each per stage, swizzled as the whole tiles) filled by direct buffer -> LDS loads two stages
// ahead, one barrier per stage. Wave w owns rows [32 w, 32 w + 32) x all BN features as
// 2 x BN / 16 MFMA blocks with the weight fragment first; a wave whose rows all lie past the
// tile's end reads no fragments and issues no MFMAs (it still loads and passes the barriers).
// Epilogue per lane (4 consecutive features of one row): MODE 0 the accumulator, 1 its SiLU, 2
// also the pre-activation to C2 first; one rounding.
constexpr int NR_STAGES = 3;

template <int MODE, int BN>
__device__ __forceinline__ void narrow_slice(const GemmParams& p, uint8_t* smem, const Tile& t, int n0, int bcols) {
  constexpr int NJ = BN / 16;                   // 16-feature blocks per wave
  constexpr int BROWS = BN < 64 ? 64 : BN;      // B rows staged
  constexpr int NR_STAGE_BYTES = TILE_BYTES + BROWS * ROWB;   // 40 or 48 KiB
  constexpr int NR_LPS = 4 + BROWS / 64;        // load instructions per wave and stage
  static_assert(NR_STAGES * NR_STAGE_BYTES <= 2 * STAGE_BYTES + 8 * EPI_BYTES, "ring exceeds the LDS");
  const int N = p.N, rowbytes = p.K * 2, nk = p.K / 64;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, fc = lane >> 4;
  const uint8_t* __restrict__ A = (const uint8_t*)p.A + (size_t)t.row0 * rowbytes;
  const uint8_t* __restrict__ B = (const uint8_t*)p.B + ((size_t)t.e * N + n0) * rowbytes;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // wave w loads A rows 32 w + 8 i + lane / 8 (i < 4) and B rows 64 h + 8 w + lane / 8 (h <
  // BROWS / 64; B rows at or past bcols are outside the resource: zeros, nothing fetched); lane l
  // fills slot l % 8 of its row with the chunk the swizzle puts there (the swizzle of B row r
  // depends on r % 16 only, so one offset serves every h)
  uint32_t va[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = w * 32 + i * 8 + (lane >> 3);
    va[i] = (uint32_t)r * (uint32_t)rowbytes + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  const int rbw = w * 8 + (lane >> 3);
  const uint32_t vb = (uint32_t)rbw * (uint32_t)rowbytes + (((lane & 7) ^ ((rbw >> 1) & 7)) << 4);
  auto issue = [&](int st) {
    const int slot = st % NR_STAGES;
    st = min(st, nk - 1);   // past the end: a harmless reload, so every stage issues NR_LPS loads
    const i32x4_t ra = make_rsrc(A + st * ROWB, (uint32_t)t.rows * rowbytes);
    const i32x4_t rb = make_rsrc(B + st * ROWB, (uint32_t)bcols * rowbytes);
    const uint32_t base = lds0 + slot * NR_STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16(ra, va[i], base + (w * 32 + i * 8) * ROWB);
#pragma unroll
    for (int h = 0; h < BROWS / 64; ++h)
      load_lds16(rb, vb + (uint32_t)(64 * h) * (uint32_t)rowbytes, base + TILE_BYTES + (64 * h + w * 8) * ROWB);
  };
  const bool live = w * 32 < t.rows;   // wave-uniform
  f32x4_t acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0);
  issue(1);
  for (int s = 0; s < nk; ++s) {
    // this wave's loads of stage s have landed (those of stage s + 1 may still be in flight);
    // after the barrier every wave's have, and the slot of stage s + 2 was last read in stage s - 1
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NR_LPS) : "memory");
    __syncthreads();
    issue(s + 2);
    const uint8_t* sa = smem + (s % NR_STAGES) * NR_STAGE_BYTES;
    const uint8_t* sb = sa + TILE_BYTES;
    if (!live) continue;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t xa[2], wb[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        xa[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sa + lds_off(w * 32 + 16 * i + fr, ks * 4 + fc)));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        wb[j] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sb + lds_off(16 * j + fr, ks * 4 + fc)));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[j], xa[i], acc[i][j], 0, 0, 0);
    }
  }
  wait_vm_all();   // the clamped reloads of the last two iterations
  // lane holds features 4 fc .. + 3 of row fr of each 16 x 16 block
  uint16_t* __restrict__ C = (uint16_t*)p.C;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = w * 32 + 16 * i + fr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = 16 * j + 4 * fc;
      if (r >= t.rows || n >= bcols) continue;
      const size_t o = (size_t)(t.row0 + r) * N + n0 + n;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if constexpr (MODE == 2) {   // the pre-activation, rounded once
        *(uint2*)((uint16_t*)p.C2 + o) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
      if constexpr (MODE == 1 || MODE == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = silu_fast(v[u]);
      }
      *(uint2*)(C + o) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

// BT: the weights are stored [E][K][N] (the transposes of the [E][N][K] layout; the backward's dH
// and dXp read W2 and W1 as they are). A stage of B, 64 k-rows of the tile's 256 features, is then
// staged as four 64-feature blocks of 64 rows x 128 bytes (block wn is what waves wn and wn + 4
// read), the 32-byte quarters of row r XOR-swizzled by f(r) = ((r >> 1) & 1) | (((r >> 3) & 1) <<
// 1), and read with the transposing LDS read (ds_read_b64_tr_b16: in each group of 16 lanes, lane s
// reads 8 bytes of row r0 + s / 4 at column c0 + 4 (s % 4), and lane i receives column c0 + i of
// rows r0 .. r0 + 3), two reads per MFMA operand. The swizzle puts the 16 rows x 32 bytes of one
// such read on every bank octet exactly twice. No narrow tail (its ring stages B as [N][K]).
template <bool SILU, bool PRE, bool BT>
__global__ __launch_bounds__(512, 1) void gemm_big_kernel(GemmParams p) {
  static_assert(SILU || !PRE, "the pre-activation is kept by the SiLU GEMM only");
  static_assert(!BT || !SILU, "[K, N] weights are read by the backward's plain products only");
  // the two operand stages and the per-wave epilogue areas; the narrow tail reuses all of it as a
  // 3-stage ring (3 x 48 KiB)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES + 8 * EPI_BYTES];
  uint8_t* const epi = smem + 2 * STAGE_BYTES;

  __shared__ int seg[MOE_MAX_EXPERTS_DEV + 1];
  __shared__ int porder[MOE_MAX_EXPERTS_DEV];

  const int tid = threadIdx.x;
  const int E = p.E, N = p.N;
  // Segment bounds, clamped into [0, max_rows] and made non-decreasing so that no offsets value
  // can send a tile outside the buffers, and the order of the partial m-tiles. Kept in LDS: tiles
  // are decoded between the kernel's own counted memory operations, where a global load (and the
  // wait for it) would not belong.
  if (tid <= E) seg[tid] = p.offsets[tid];   // all loads in flight at once
  __syncthreads();
  if (tid == 0) {
    int prev = 0;
    for (int e = 0; e <= E; ++e) {
      const int o = seg[e];
      prev = o < prev ? prev : (o > p.max_rows ? p.max_rows : o);
      seg[e] = prev;
    }
  }
  __syncthreads();
  if constexpr (!PRE) {   // the pre-activation variant keeps the expert order (no registers to spare)
    if (tid < 64) order_partials(seg, E, porder);
    __syncthreads();
  }
  int MT = 0, MF0 = 0;
  for (int e = 0; e < E; ++e) {
    const int len = seg[e + 1] - seg[e];
    MF0 += len / BIG_BM;
    MT += (len + BIG_BM - 1) / BIG_BM;
  }
  const int NT = (N + BIG_BN - 1) / BIG_BN;
  const int total = MT * NT;
  const int rowbytes = p.K * 2;
  const int nk = rowbytes / ROWB;
  // Whole tiles: each XCD takes a contiguous range of tile ids, walked by its workgroups with a
  // stride of their count. With a split tail (partial-sum workspace given, G == 256) the whole
  // tiles are the first `full` (a multiple of G, so every workgroup gets the same number), and
  // then workgroup v (XCD-major: the parts of one tile share an XCD) computes part v % s of tail
  // tile v / s into partial slot v; a second kernel adds the parts and stores the tile. With a
  // narrow tail the whole tiles are the first `full` as well, and then workgroup v computes slice
  // v % s of tail tile v / s (narrow_slice).
  const int G = gridDim.x, xcd = blockIdx.x & 7;
  const int sparts = (p.sk_part != nullptr && G == MAX_WGS) ? tail_parts(total, G, nk) : 1;
  // (the sorted order pays through the narrow tail under 64 stages, which BT does not have)
  const int MF = (PRE || (BT && nk < 64)) ? 0 : sorted_mf(total, MT, MF0, NT, G, nk, p.sort_split && sparts > 1, seg, porder);
  auto decode = [&](int id) { return decode_tile(id, MT, MF, NT, N, E, seg, porder); };
  const int nparts = BT ? 1 : narrow_parts(total, G, nk, MF > 0);
  const int full = (sparts > 1 || nparts > 1) ? total - total % G : total;
  const int q = full >> 3, rem = full & 7;
  const int cnt = (xcd < rem) ? q + 1 : q;
  const int start = (xcd < rem) ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
  const int step = (G - xcd + 7) >> 3;
  int local = blockIdx.x >> 3;
  const int vsplit = xcd * (G >> 3) + local;
  const bool has_split = sparts > 1 && vsplit < (total - full) * sparts;
  const bool has_narrow = nparts > 1 && vsplit < (total - full) * nparts;
  if (local >= cnt && !has_split && !has_narrow) return;


  const uint8_t* __restrict__ A = (const uint8_t*)p.A;
  const uint8_t* __restrict__ B = (const uint8_t*)p.B;
  uint16_t* __restrict__ C = (uint16_t*)p.C;

  // Direct loads: one instruction moves 8 rows x 128 B; lane l lands at byte 16 l of the
  // instruction's 1 KiB, i.e. row l / 8, slot l % 8, and loads the global chunk that the swizzle
  // puts in that slot. Wave w fills rows [32 w, 32 w + 32) of both operand tiles; the offsets
  // (relative to the tile's first row) are the same for A and B.
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // BT loads: rows 8 i + l / 8 of a 64-feature block (instruction i < 8 covers rows 8 i .. 8 i + 7),
  // lane l filling slot l % 8 with the chunk the swizzle puts there, (l % 8) ^ 2 f(row); per-lane
  // offset for even and odd i (the row offset 16 (i / 2) rows goes in the scalar offset), out of
  // range for features past the tile's last one
  const uint32_t nb2 = (uint32_t)N * 2u;   // bytes of a [K, N] row
  auto bt_off = [&](const Tile& t, int blk, int h) -> uint32_t {
    const int chunk = (lane & 7) ^ ((((lane >> 4) & 1) << 1) | (h << 2));
    const int c = 64 * blk + 8 * chunk;
    return c < t.cols ? (uint32_t)(8 * h + (lane >> 3)) * nb2 + (uint32_t)c * 2u : 0x80000000u;
  };
  // instructions [i0, i0 + n) of block blk of stage st of tile t into LDS (dst: the block's base),
  // with the block's two lane offsets o0, o1 (bt_off)
  // (n is 4 or 8 and i0 even: the loop has a fixed trip count, offsets alternate o0, o1)
  auto load_bt_o = [&](const Tile& t, int st, uint32_t o0, uint32_t o1, int i0, auto n_c, uint32_t dst) {
    constexpr int n = decltype(n_c)::value;
    const i32x4_t r = make_rsrc(B + ((size_t)t.e * p.K + (size_t)st * 64) * nb2 + (size_t)t.n0 * 2u, 64u * nb2);
    const uint32_t soff0 = (uint32_t)(i0 >> 1) * 16u * nb2;
    const uint32_t d0 = dst + (uint32_t)i0 * 1024u;
#pragma unroll
    for (int k = 0; k < n; ++k)
      load_lds16s(r, (k & 1) ? o1 : o0, soff0 + (uint32_t)((k >> 1) * 16) * nb2, d0 + k * 1024);
  };
  auto load_bt = [&](const Tile& t, int st, int blk, int i0, auto n_c, uint32_t dst) {
    load_bt_o(t, st, bt_off(t, blk, 0), bt_off(t, blk, 1), i0, n_c, dst);
  };
  uint32_t bto0 = 0, bto1 = 0;   // the split tail's offsets (one tile: computed once)
  // Requests stage kt of a run of stages [k0, k1) of tile t (clamped to its last one: a harmless
  // reload) into buffer (kt - k0) & 1.
  auto issue = [&](const Tile& t, int kt, int k0 = 0, int k1 = 0x7fffffff) {
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = w * 32 + i * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ (((i & 1) << 2) | (lane >> 4));
      voff[i] = (uint32_t)r * (uint32_t)rowbytes + chunk * 16;
    }
    const int st = min(kt, min(k1, nk) - 1);
    const i32x4_t ra = make_rsrc(A + (size_t)t.row0 * rowbytes + st * ROWB, (uint32_t)t.rows * rowbytes);
    const i32x4_t rb = make_rsrc(B + ((size_t)t.e * N + t.n0) * rowbytes + st * ROWB, (uint32_t)t.cols * rowbytes);
    const uint32_t sa = lds0 + ((kt - k0) & 1) * STAGE_BYTES + w * 32 * ROWB;
    const uint32_t sb = sa + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load_lds16(ra, voff[i], sa + i * 8 * ROWB);
      if constexpr (!BT) load_lds16(rb, voff[i], sb + i * 8 * ROWB);
    }
    if constexpr (BT)   // wave w: rows [32 (w >> 2), + 32) of block w & 3
      load_bt_o(t, st, bto0, bto1, 4 * (w >> 2), std::integral_constant<int, 4>{}, lds0 + ((kt - k0) & 1) * STAGE_BYTES + TILE_BYTES + (w & 3) * 8192);
  };

  const int wm = w >> 2, wn = w & 3;   // 2 x 4 waves, each 128 rows x 64 output features
  const int fr = lane & 15, fc = lane >> 4;   // fragment row within 16, 16-byte chunk
  f32x4_t acc[8][4];
  bf16x8_t xa[2][8], wb[2][4];
  auto frag_x = [&](int buf, int stage, int ks, int i) {
    const uint8_t* sa = smem + (stage & 1) * STAGE_BYTES;
    xa[buf][i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sa + lds_off(wm * 128 + i * 16 + fr, ks * 4 + fc)));
  };

  auto rs_a = [&](const Tile& t, int st) {
    return make_rsrc(A + (size_t)t.row0 * rowbytes + st * ROWB, (uint32_t)t.rows * rowbytes);
  };
  auto rs_b = [&](const Tile& t, int st) {
    return make_rsrc(B + ((size_t)t.e * N + t.n0) * rowbytes + st * ROWB, (uint32_t)t.cols * rowbytes);
  };
  // transposing reads of BT fragment j (16 features) of k-step ks from a block at `blk`
  const uint32_t bt_rd = (uint32_t)((8 * fc + (fr >> 2)) * 128 + 8 * (fr & 3) + 32 * ((fr >> 3) | ((fc & 1) << 1)));
  auto bt_frag = [&](const uint8_t* blk, int ks, int j) -> bf16x8_t {
    uint32_t o = bt_rd ^ (uint32_t)(32 * j);
    asm volatile("" : "+v"(o));   // formed at each read rather than four addresses held in registers
    const uint8_t* q = blk + ks * 32 * 128 + o;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(__attribute__((address_space(3))) const uint8_t*)q);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(__attribute__((address_space(3))) const uint8_t*)(q + 4 * 128));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto frag_w = [&](int buf, int stage, int ks, int j) {
    const uint8_t* sb = smem + (stage & 1) * STAGE_BYTES + TILE_BYTES;
    if constexpr (BT) wb[buf][j] = bt_frag(sb + wn * 8192, ks, j);
    else wb[buf][j] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(sb + lds_off(wn * 64 + j * 16 + fr, ks * 4 + fc)));
  };

  // Epilogue of tile t from the accumulators (after the wait states that let the last MFMAs
  // retire): SiLU (when S), one rounding, and row-contiguous stores to dst through a per-wave
  // LDS area.
  // MODE 0: the accumulator; 1: SiLU of it
  auto store_pass = [&](const Tile& t, auto mode_c, uint16_t* dst) {
    constexpr int MODE = decltype(mode_c)::value;
    // per-lane epilogue offsets, recomputed for every tile rather than held across the main loop
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int efr = lane_o & 15, efc = lane_o >> 4;

    // Epilogue, one 16-row block at a time through a per-wave LDS area. Lane (fr, fc) holds
    // features 4 fc .. 4 fc + 3 of row fr of every 16 x 16 block; swapping the odd 16-lane rows of
    // block 2 jp with the even rows of block 2 jp + 1 leaves 8 consecutive features per lane (lane
    // row fc gets columns 8 (fc / 2) + 16 (fc % 2) .. + 7 of the 32-column pair), written to LDS as
    // one 16-byte chunk of the wave's 128-byte row. Read back, each lane holds 16 bytes of one row
    // and a store instruction covers 8 rows x 128 contiguous bytes: whole lines, where the MFMA
    // layout would store 16 rows x 64 bytes (a third of the throughput per CU). The 8 chunks of an
    // LDS row are XOR-swizzled by the row.
    const i32x4_t rc = make_rsrc(dst + (size_t)t.row0 * N, (uint32_t)t.rows * N * 2);
    uint8_t* const ep = epi + w * EPI_BYTES;
    const int rrow = lane_o >> 3, rchunk = lane_o & 7;   // read-back: row within 8, chunk
  #pragma unroll
    for (int i = 0; i < 8; ++i) {
  #pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        uint32_t P[2], Q[2];
  #pragma unroll
        for (int h = 0; h < 2; ++h) {
          float a0 = acc[i][2 * jp][2 * h], a1 = acc[i][2 * jp][2 * h + 1];
          float b0 = acc[i][2 * jp + 1][2 * h], b1 = acc[i][2 * jp + 1][2 * h + 1];
          if constexpr (MODE == 1) {
            a0 = silu_fast(a0);
            a1 = silu_fast(a1);
            b0 = silu_fast(b0);
            b1 = silu_fast(b1);
          }
          const auto r = __builtin_amdgcn_permlane16_swap(pack_bf16x2(a0, a1), pack_bf16x2(b0, b1), false, false);
          P[h] = r[0];
          Q[h] = r[1];
        }
        const int chunk = jp * 4 + ((efc >> 1) | ((efc & 1) << 1));
        *(uint4*)(ep + efr * 128 + ((chunk ^ (efr & 7)) << 4)) = uint4{P[0], P[1], Q[0], Q[1]};
      }
  #pragma unroll
      for (int qd = 0; qd < 2; ++qd) {
        const int row = qd * 8 + rrow;
        const uint4 v = *(const uint4*)(ep + row * 128 + ((rchunk ^ (row & 7)) << 4));
        const int m = wm * 128 + i * 16 + row;
        const int n = wn * 64 + rchunk * 8;
        const uint32_t off = (n < t.cols) ? (uint32_t)(m * N + t.n0 + n) * 2u : 0x80000000u;
        store16(rc, off, u32x4_t{v.x, v.y, v.z, v.w});
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // PRE (with SILU, p.C2 set): also the pre-activation, same tile, before the SiLU pass.
  auto store_tile = [&](const Tile& t) {
    if constexpr (SILU) {
      if constexpr (PRE) store_pass(t, std::integral_constant<int, 0>{}, (uint16_t*)p.C2);
      store_pass(t, std::integral_constant<int, 1>{}, C);
    } else {
      store_pass(t, std::integral_constant<int, 0>{}, C);
    }
  };

  if (local < cnt) {
  // Ping-pong. The two waves on each SIMD (waves w and w + 4: the two 128-row halves of the tile,
  // groups 0 and 1) take turns. In phase X of stage g group 0 runs its 64 MFMAs of stage g while
  // group 1 reads its stage-g fragments from LDS; in phase Y they swap. A barrier ends each phase,
  // so in its MFMA phase a wave issues nothing but MFMAs and every SIMD's matrix core is fed by
  // one wave while the other works on memory. The direct loads are split evenly between the
  // groups' memory phases, each as soon as the rows it overwrites have been read by both groups:
  // group 0 loads the A rows of stage g + 2 in phase Y(g); wave wn of group 1 loads B rows
  // [64 wn, 64 wn + 64) (the block it and its partner read) of stage g + 2 in phase X(g), right
  // after its own stage-g reads. Each group waits for its loads at the end of its next MFMA
  // phase, about two phases after issuing them and before the barrier after which they are read.
  // A tile's epilogue falls in the group's memory phase (group 0: phase Y of the last stage;
  // group 1: phase X of the next tile's first stage), beside the other group's MFMAs.
  // Needs at least four stages per tile.
  const int gr = wm;
  // group 0: A rows of stage st of tile t into buffer buf; group 1: B rows. Wave wn loads rows
  // [64 wn, 64 wn + 64) of its operand, 8 rows per instruction: lane l fills row 8 i + l / 8 (of
  // the wave's 64) at slot l % 8 with the chunk the swizzle puts there. The plain variants hold
  // the two per-lane offsets (even and odd i) across the loop. The variant that also writes the
  // pre-activation has no vector register to spare for them: there they are recomputed from the
  // lane id at each call (in volatile asm, so not hoisted and held), and the row offset of i goes
  // in the scalar offset (held, they spilled to scratch, and the reloads stalled every stage).
  uint32_t vo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = wn * 64 + h * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((h << 2) | (lane >> 4));
    vo[h] = (uint32_t)r * (uint32_t)rowbytes + chunk * 16;
  }
  auto load_half = [&](const Tile& t, int st, int buf) {
    if constexpr (BT) {
      if (gr == 1) {   // block wn of B, all 64 rows
        load_bt(t, st, wn, 0, std::integral_constant<int, 8>{}, lds0 + buf * STAGE_BYTES + TILE_BYTES + wn * 8192);
        return;
      }
    }
    const i32x4_t r = gr == 0 ? rs_a(t, st) : rs_b(t, st);
    const uint32_t sa = lds0 + buf * STAGE_BYTES + gr * TILE_BYTES + wn * 64 * ROWB;
    if constexpr (PRE) {
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int c0 = (ln & 7) ^ (ln >> 4);
      const uint32_t vo0 = (uint32_t)(wn * 64 + (ln >> 3)) * (uint32_t)rowbytes + (uint32_t)(c0 << 4);
      const uint32_t vo1 = vo0 + 8u * (uint32_t)rowbytes + (uint32_t)(((c0 ^ 4) - c0) * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        load_lds16s(r, (i & 1) ? vo1 : vo0, (uint32_t)((i >> 1) * 16) * (uint32_t)rowbytes, sa + i * 8 * ROWB);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        load_lds16(r, vo[i & 1] + (uint32_t)((i >> 1) * 16) * (uint32_t)rowbytes, sa + i * 8 * ROWB);
    }
  };
  // Fragment reads of stage g: row r of a 16-row block sits at byte r * 128 of its block, its 16-byte
  // chunk c at ((c ^ ((r >> 1) & 7)) << 4); within one wave the swizzle depends on the lane only
  // (block rows are multiples of 16), so each k-step's reads are one per-lane base plus constants.
  // The base passes through an empty asm so that the compiler keeps one address register per
  // k-step instead of precomputing every read's address.
  // In the variant that also writes the pre-activation the per-lane base is formed from the lane
  // id at each call (volatile asm, so it is neither hoisted nor held): held, the two k-step bases
  // spilled, and each stage's reload waited for every outstanding load (vmcnt(0)), operand
  // prefetches included.
  const uint32_t fsw = (uint32_t)(fr * ROWB) + (uint32_t)((fc ^ ((fr >> 1) & 7)) << 4);
  auto read_frags = [&](int g) {
    const uint8_t* sbuf = smem + (g & 1) * STAGE_BYTES;
    uint32_t fsb = fsw;
    if constexpr (PRE) {
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int lr = ln & 15, lc = ln >> 4;
      fsb = (uint32_t)(lr * ROWB) + (uint32_t)((lc ^ ((lr >> 1) & 7)) << 4);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t oa = fsb ^ (uint32_t)(ks << 6);   // chunk ks * 4 + fc
      asm volatile("" : "+v"(oa));
      const uint8_t* pa = sbuf + wm * 128 * ROWB + oa;
      const uint8_t* pb = sbuf + TILE_BYTES + wn * 64 * ROWB + oa;
#pragma unroll
      for (int i = 0; i < 8; ++i) xa[ks][i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(pa + i * 16 * ROWB));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (BT) wb[ks][j] = bt_frag(sbuf + TILE_BYTES + wn * 8192, ks, j);
        else wb[ks][j] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(pb + j * 16 * ROWB));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  auto compute = [&]() {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma_16x16x32(acc[i][j], wb[ks][j], xa[ks][i]);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  // let the last MFMAs retire before their accumulators are read (the most recently written
  // accumulators pass through the wait so that no read of them is scheduled before it)
  auto retire = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]),
                   "+a"(acc[6][0]), "+a"(acc[6][1]), "+a"(acc[6][2]), "+a"(acc[6][3])
                 :
                 : "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Every wave runs the same loop, one stage per iteration: its MFMAs of stage g, a barrier, its
  // memory work (group 0: the A loads of stage g + 2; after a tile's last stage the epilogue; the
  // fragments of stage g + 1; group 1: then the B loads of stage g + 3 into the buffer just read),
  // a barrier. Group 1 passes one barrier before its first MFMAs, which puts it one phase behind
  // group 0 for the whole kernel (group 0 passes one more at the end, so both pass the same
  // number).
  Tile cur = decode(start + local);
  {   // stages 0 and 1 of the first tile, every wave its 32 rows of both operands
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = w * 32 + i * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ (((i & 1) << 2) | (lane >> 4));
      voff[i] = (uint32_t)r * (uint32_t)rowbytes + chunk * 16;
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const i32x4_t ra = rs_a(cur, st), rb = rs_b(cur, st);
      const uint32_t sa = lds0 + st * STAGE_BYTES + w * 32 * ROWB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        load_lds16(ra, voff[i], sa + i * 8 * ROWB);
        if constexpr (!BT) load_lds16(rb, voff[i], sa + TILE_BYTES + i * 8 * ROWB);
      }
      if constexpr (BT)   // wave w: rows [32 (w >> 2), + 32) of block w & 3
        load_bt(cur, st, w & 3, 4 * (w >> 2), std::integral_constant<int, 4>{}, lds0 + st * STAGE_BYTES + TILE_BYTES + (w & 3) * 8192);
    }
  }
  wait_vm_all();
  __syncthreads();
  zero_acc();
  read_frags(0);
  if (gr == 1) {
    load_half(cur, 2, 0);   // B rows of stage 2, over the stage-0 rows this wave has just read
    phase_end();
  }
  int g0 = 0;
  while (true) {
    const int nlocal = local + step;
    const bool more = nlocal < cnt;
    const Tile nxt = more ? decode(start + nlocal) : cur;
    for (int s = 0; s < nk; ++s) {
      const int g = g0 + s;
      compute();
      wait_vm_all();   // this wave's loads issued in its previous memory phase
      phase_end();
      if (gr == 0) {   // A rows of stage g + 2 into stage g's buffer
        const int st = s + 2;
        if (st < nk || more) load_half(st < nk ? cur : nxt, st < nk ? st : st - nk, g & 1);
      }
      if (s == nk - 1) {
        retire();
        store_tile(cur);
        zero_acc();
      }
      // (past the last tile this reads a stale buffer, unused)
      read_frags(g + 1);
      if (gr == 1) {   // B rows of stage g + 3 into the buffer of stage g + 1, just read
        const int st = s + 3;
        if (st < nk || more) load_half(st < nk ? cur : nxt, st < nk ? st : st - nk, (g + 1) & 1);
      }
      phase_end();
    }
    if (!more) break;
    g0 += nk;
    cur = nxt;
    local = nlocal;
  }
  if (gr == 0) phase_end();
  wait_vm_all();
  }

  if (has_split) {
    // part `part` of tail tile `tile`: stages [k0, k1), sums to partial slot vsplit
    const int part = vsplit % sparts;
    const Tile t = decode(full + vsplit / sparts);
    const int k0 = part * nk / sparts, k1 = (part + 1) * nk / sparts;
    if constexpr (BT) {
      bto0 = bt_off(t, w & 3, 0);
      bto1 = bt_off(t, w & 3, 1);
    }
    __syncthreads();   // the whole-tile loop may still be reading the LDS buffers
    issue(t, k0, k0, k1);
    issue(t, k0 + 1, k0, k1);
    wait_vm_all();
    __syncthreads();
    // a wave whose 128 rows all lie past the tile's end reads no fragments and issues no MFMAs
    // (it still loads its share and passes the barriers); its partial sums stay zero. Not in the
    // pre-activation variant, whose tiles keep the expert order (and whose main loop has no
    // registers to spare for the branches)
    const bool live = PRE || wm * 128 < t.rows;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (BT) {
      // one fragment slot, the reads of a stage before its MFMAs (the interleaved schedule below
      // holds two slots, which with the transposing reads does not fit in the registers); the
      // partner wave on the SIMD overlaps them
      for (int s = 0; s < k1 - k0; ++s) {
        if (s >= 1 && k0 + s + 1 < k1) issue(t, k0 + s + 1, k0, k1);
        if (live) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < 8; ++i) frag_x(0, s, ks, i);
#pragma unroll
            for (int j = 0; j < 4; ++j) frag_w(0, s, ks, j);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) mfma_16x16x32(acc[i][j], wb[0][j], xa[0][i]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_all();
        __syncthreads();
      }
    } else {
    if (live) {
#pragma unroll
      for (int i = 0; i < 8; ++i) frag_x(0, 0, 0, i);
#pragma unroll
      for (int j = 0; j < 4; ++j) frag_w(0, 0, 0, j);
    }
    for (int s = 0; s < k1 - k0; ++s) {
      if (s >= 1 && k0 + s + 1 < k1) issue(t, k0 + s + 1, k0, k1);
      if (live) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) mfma_16x16x32(acc[i][j], wb[0][j], xa[0][i]);
          if (i < 4) frag_w(1, s, 1, i);
          frag_x(1, s, 1, i);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) mfma_16x16x32(acc[i][j], wb[1][j], xa[1][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_all();
      __syncthreads();
      if (live) {
#pragma unroll
        for (int i = 4; i < 8; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) mfma_16x16x32(acc[i][j], wb[1][j], xa[1][i]);
          frag_x(0, s + 1, 0, 2 * (i - 4));
          frag_x(0, s + 1, 0, 2 * (i - 4) + 1);
          frag_w(0, s + 1, 0, i - 4);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]),
                   "+a"(acc[6][0]), "+a"(acc[6][1]), "+a"(acc[6][2]), "+a"(acc[6][3])
                 :
                 : "memory");
    __builtin_amdgcn_sched_barrier(0);
    const i32x4_t rp = make_rsrc((uint8_t*)p.sk_part + (size_t)vsplit * PART_BYTES, PART_BYTES);
    const uint32_t poff = (uint32_t)((w * 32 * 64 + lane) * 16);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) store_part(rp, poff, (i * 4 + j) * 64 * 16, acc[i][j]);
    wait_vm_all();
  }

  if constexpr (!BT) if (has_narrow) {
    // slice vsplit % s of leftover tile vsplit / s (XCD-major numbering: the slices of a tile share
    // an XCD and its L2 copy of the tile's rows of A)
    __syncthreads();   // every wave is done with the whole-tile buffers and epilogue areas
    const Tile t = decode(full + vsplit / nparts);
    const int bn = BIG_BN / nparts, sl = vsplit % nparts;
    const int bcols = min(t.cols - sl * bn, bn);
    if (bcols > 0) {   // slices past N of a narrower last n-tile have nothing to do
      constexpr int MODE = SILU ? (PRE ? 2 : 1) : 0;
      if (!PRE && nparts == 2) narrow_slice<MODE, 128>(p, smem, t, t.n0 + sl * bn, bcols);
      else if (nparts == 4) narrow_slice<MODE, 64>(p, smem, t, t.n0 + sl * bn, bcols);
      else narrow_slice<MODE, 32>(p, smem, t, t.n0 + sl * bn, bcols);
    }
  }
}


// Adds the s partial sums of each split tail tile (in part order), applies the activation and
// stores the tile. Item (r, w8, h): tail tile r, a quarter h of the 2048 16-byte chunks of wave
// w8 of the GEMM's tile layout (each of 4 consecutive features of one row); the grid walks the
// items.
template <bool SILU>
__global__ __launch_bounds__(256) void gemm_tail_kernel(GemmParams p, int G) {
  __shared__ int seg[MOE_MAX_EXPERTS_DEV + 1];
  __shared__ int porder[MOE_MAX_EXPERTS_DEV];
  const int E = p.E, N = p.N, tid = threadIdx.x;
  if (tid <= E) seg[tid] = p.offsets[tid];   // all loads in flight at once
  __syncthreads();
  if (tid == 0) {
    int prev = 0;
    for (int e = 0; e <= E; ++e) {
      const int o = seg[e];
      prev = o < prev ? prev : (o > p.max_rows ? p.max_rows : o);
      seg[e] = prev;
    }
  }
  __syncthreads();
  if (tid < 64) order_partials(seg, E, porder);
  __syncthreads();
  int MT = 0, MF0 = 0;
  for (int e = 0; e < E; ++e) {
    const int len = seg[e + 1] - seg[e];
    MF0 += len / BIG_BM;
    MT += (len + BIG_BM - 1) / BIG_BM;
  }
  const int NT = (N + BIG_BN - 1) / BIG_BN;
  const int total = MT * NT, nk = p.K / 64;
  const int sparts = tail_parts(total, G, nk);
  if (sparts < 2) return;
  const int full = total - total % G;
  // the GEMM's order (the pre-activation variant, SILU with C2, keeps the expert order)
  const int MF = (SILU && p.C2) ? 0 : sorted_mf(total, MT, MF0, NT, G, nk, p.sort_split != 0, seg, porder);
  for (int item = blockIdx.x; item < (total - full) * 32; item += gridDim.x) {
  const int r = item >> 5, w8 = (item >> 2) & 7, h = item & 3;
  const Tile tt = decode_tile(full + r, MT, MF, NT, N, E, seg, porder);   // as in the GEMM
  const int n0 = tt.n0, cols = tt.cols, row0 = tt.row0, rows = tt.rows;
  const float4* __restrict__ part = (const float4*)p.sk_part;
  uint16_t* __restrict__ C = (uint16_t*)p.C;
  const int wm = w8 >> 2, wn = w8 & 3;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int chunk = h * 512 + c * 256 + tid;           // within the wave's 2048 chunks
    const int blk = chunk >> 6, lane = chunk & 63;
    const int m = wm * 128 + (blk >> 2) * 16 + (lane & 15);
    const int n = wn * 64 + (blk & 3) * 16 + 4 * (lane >> 4);
    const size_t o = (size_t)w8 * 2048 + chunk;          // 16-byte units within a slot
    if (m >= rows || n >= cols) continue;                 // never stored: not summed either
    float4 s = part[(size_t)(r * sparts) * (PART_BYTES / 16) + o];
    for (int j = 1; j < sparts; ++j) {
      const float4 t = part[(size_t)(r * sparts + j) * (PART_BYTES / 16) + o];
      s.x += t.x;
      s.y += t.y;
      s.z += t.z;
      s.w += t.w;
    }
    float v[4] = {s.x, s.y, s.z, s.w};
    if (SILU && p.C2) {   // the pre-activation, rounded once
      uint2 a;
      a.x = pack_bf16x2(v[0], v[1]);
      a.y = pack_bf16x2(v[2], v[3]);
      *(uint2*)((uint16_t*)p.C2 + (size_t)(row0 + m) * N + n0 + n) = a;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = SILU ? silu_fast(v[u]) : v[u];
    uint2 out;
    out.x = pack_bf16x2(v[0], v[1]);
    out.y = pack_bf16x2(v[2], v[3]);
    *(uint2*)(C + (size_t)(row0 + m) * N + n0 + n) = out;
  }
  }
}

size_t gemm_big_part_bytes() { return (size_t)MAX_WGS * PART_BYTES; }

int gemm_big_grid(int max_rows, int E, int N) {
  const long tiles = (long)((max_rows + BIG_BM - 1) / BIG_BM + E) * ((N + BIG_BN - 1) / BIG_BN);
  return (int)(tiles < MAX_WGS ? tiles : MAX_WGS);
}

hipError_t launch_gemm_big(const GemmParams& p, bool silu, hipStream_t s) {
  if (p.K < 256) return hipErrorInvalidValue;   // the pipeline needs four K stages per tile
  // reductions under 64 stages always get all 256 workgroups, so that a narrow tail has them
  const int grid = p.K / 64 < 64 ? MAX_WGS : gemm_big_grid(p.max_rows, p.E, p.N);
  if (p.b_kn && silu) return hipErrorInvalidValue;
  if (silu && p.C2) gemm_big_kernel<true, true, false><<<grid, 512, 0, s>>>(p);
  else if (silu) gemm_big_kernel<true, false, false><<<grid, 512, 0, s>>>(p);
  else if (p.b_kn) gemm_big_kernel<false, false, true><<<grid, 512, 0, s>>>(p);
  else gemm_big_kernel<false, false, false><<<grid, 512, 0, s>>>(p);
  if (p.sk_part && grid == MAX_WGS && p.K / 64 >= 64) {   // tail_parts splits nothing below 64 stages
    // the kernel works out how many tail tiles there are (none: it returns at once)
    if (silu) gemm_tail_kernel<true><<<4 * MAX_WGS, 256, 0, s>>>(p, grid);
    else gemm_tail_kernel<false><<<4 * MAX_WGS, 256, 0, s>>>(p, grid);
  }
  return hipGetLastError();
}

}  // namespace moe
