// 4-bit expert weights for the weight-streaming regime: the quantiser and a grouped GEMM that
// reads int4 codes and bf16 scales.
//
// [P4 §5.2] quantise the expert weights to 4 bits. Format (symmetric, group-wise along K, groups
// of 64): per (row, group) a bf16 scale s = bf16(fp32(amax / 7)); codes q = clamp(rint(fp32(w /
// s)), -8, 7) (0 where s = 0), two's complement nibbles, two per byte (low nibble = even column).
// The layer uses w' = bf16(q s): q s has at most 12 significant bits, so the fp32 product is exact
// and the conversion rounds once. Layout, tiled for the GEMM's loads (rows a multiple of 16, K of
// 128): the codes of rows 16 t .. + 15 and columns 128 s .. + 127 form 1 KiB block t K/128 + s, in
// which the 16 bytes at 16 (16 g + r) hold row 16 t + r, columns 128 s + 32 g .. + 31 -- exactly
// what lane 16 g + r of a wave loads for one stage, so each load instruction reads 1 KiB
// contiguously. The scales follow from the next 256-byte boundary (zero bytes in between), 32 per
// block: row r's two groups at 2 r, 2 r + 1.
//
// gemm_q4_kernel: C[r, n] = act( sum_k A[r, k] * w'[e, n, k] ) over expert segments of at most a
// few dozen rows, where the weights are the HBM traffic (4.25 bits per weight instead of 16). One
// workgroup of 8 waves per (expert, 128 output features), two waves per SIMD:
//  * the weight block never passes through LDS: in each 128-column stage, lane (f, g) of wave w
//    loads, for its feature 16 w + f, the 16 bytes of codes of columns [32 g, 32 g +
//    32) and the scale of their group, two stages ahead in registers, and dequantises them
//    straight into MFMA operands (the four 32-wide MFMA steps of the stage take columns
//    32 g + 8 s .. + 7 from lane group g, so the loads are contiguous and the activation fragments
//    follow the same column assignment);
//  * the activation rows of the stage (64 rows x 128 columns, 16 KiB) are loaded into registers
//    two stages ahead and staged through a double LDS buffer one stage ahead;
//  * v_mfma_f32_16x16x32_bf16 with the weight fragment first (16-row blocks past the chunk's
//    rows are skipped), fp32 accumulation, the epilogue of the bf16 weight-streaming kernel (SiLU
//    in fp32, one rounding).
// K must be a multiple of 128 WPD (whole groups of WPD stages; the library asks for 512) and N of
// 128 (whole 128-feature blocks of whole tiles).
#include "moe_internal.h"

#include <type_traits>

namespace moe {

namespace {
constexpr int Q4_GROUP = 64;
constexpr int QM = 64;            // activation rows per chunk
constexpr int QW = 8;             // waves per workgroup
constexpr int QN = 128;           // output features per workgroup (16 per wave)
constexpr int QNB = QN / (16 * QW);   // 16-feature blocks per wave
constexpr int QK = 128;           // columns per stage (two scale groups: one per two lane groups)
constexpr int QAL = QM * QK / 8 / (64 * QW);   // 16-byte activation loads per thread per stage
constexpr int QPD = 2;            // stages of activations in flight per lane
// stages of weight codes and scales in flight per lane (4 spill at 128 VGPRs and measured slower;
// with the activations one stage ahead instead, so that they fit, no faster than 2)
constexpr int WPD = 2;

__device__ __forceinline__ float q4_silu(float v) {
  const float e = __builtin_amdgcn_exp2f(-v * 1.44269504088896341f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// 8 signed nibbles (nibble i = k offset i) times the scale s, as one bf16x8 MFMA operand. Each
// nibble's sign bit is flipped so that the nibbles read as u = q + 8 in [0, 15]; the even and odd
// nibbles are spread into bytes and converted by the byte-to-float conversions; then
// fma(u, s, -8 s) = q s exactly (u s and 8 s are exact in fp32, and so is their difference,
// which has at most 12 significant bits), and the bf16 conversion rounds once.
__device__ __forceinline__ bf16x8_t q4_dequant(uint32_t word, float s) {
  const uint32_t u = word ^ 0x88888888u;
  uint32_t ev = u & 0x0F0F0F0Fu, od = (u >> 4) & 0x0F0F0F0Fu;
  // opaque to the optimiser, which would otherwise fold the masks into one bit-field extract per
  // nibble and lose the per-byte conversions
  asm("" : "+v"(ev));
  asm("" : "+v"(od));
  const float ms = -8.0f * s;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __builtin_fmaf((float)((ev >> (8 * i)) & 0xFFu), s, ms);
    const float b = __builtin_fmaf((float)((od >> (8 * i)) & 0xFFu), s, ms);
    o[i] = pack_bf16x2(a, b);
  }
  return __builtin_bit_cast(bf16x8_t, uint4{o[0], o[1], o[2], o[3]});
}
}  // namespace

size_t q4_scale_offset(size_t rows, int K) { return (rows * (size_t)K / 2 + 255) / 256 * 256; }

size_t q4_bytes(size_t rows, int K) { return q4_scale_offset(rows, K) + rows * (size_t)(K / Q4_GROUP) * 2; }

// One thread per (row, group of 64): the group's scale and its 32 bytes of codes (two 16-byte
// lane pieces of a tile). The padding before the scales (fewer than 256 bytes) is written by the
// first workgroup's threads.
__global__ __launch_bounds__(256) void quantize_q4_kernel(const uint16_t* __restrict__ w, size_t rows, int K,
                                                          uint8_t* __restrict__ out, size_t scale_off) {
  const int G = K / Q4_GROUP;
  const int KS = K / 128;   // stages (tiles along K)
  const size_t n = rows * (size_t)G;
  const size_t code_end = rows * (size_t)K / 2;
  if (blockIdx.x == 0 && code_end + threadIdx.x < scale_off) out[code_end + threadIdx.x] = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t row = i / G;
    const int gi = (int)(i - row * G);
    const uint16_t* src = w + row * (size_t)K + (size_t)gi * Q4_GROUP;
    float v[Q4_GROUP];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < Q4_GROUP / 8; ++c) {
      const uint4 u = *(const uint4*)(src + 8 * c);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * c + 2 * q] = bf16_bits_to_f32(wd[q] & 0xFFFFu);
        v[8 * c + 2 * q + 1] = bf16_bits_to_f32(wd[q] >> 16);
      }
    }
#pragma unroll
    for (int c = 0; c < Q4_GROUP; ++c) amax = fmaxf(amax, fabsf(v[c]));
    const uint32_t sbits = f32_to_bf16_bits(__fdiv_rn(amax, 7.0f));
    const float s = bf16_bits_to_f32(sbits);
    uint32_t packed[Q4_GROUP / 8];
#pragma unroll
    for (int c = 0; c < Q4_GROUP / 8; ++c) {
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        int code = 0;
        if (s > 0.0f) {
          const float r = rintf(__fdiv_rn(v[8 * c + q], s));
          code = (int)fminf(fmaxf(r, -8.0f), 7.0f);
        }
        word |= ((uint32_t)code & 0xFu) << (4 * q);
      }
      packed[c] = word;
    }
    // group gi = stage gi / 2, half h = gi % 2: lane groups 2 h and 2 h + 1 of tile (row / 16, stage)
    const size_t tile = (row >> 4) * (size_t)KS + (size_t)(gi >> 1);
    const int r16 = (int)(row & 15), h = gi & 1;
    uint4* dst0 = (uint4*)(out + tile * 1024 + (size_t)(16 * (2 * h) + r16) * 16);
    uint4* dst1 = (uint4*)(out + tile * 1024 + (size_t)(16 * (2 * h + 1) + r16) * 16);
    *dst0 = uint4{packed[0], packed[1], packed[2], packed[3]};
    *dst1 = uint4{packed[4], packed[5], packed[6], packed[7]};
    ((uint16_t*)(out + scale_off))[tile * 32 + (size_t)(2 * r16 + h)] = (uint16_t)sbits;
  }
}

hipError_t launch_quantize_q4(const void* w, size_t rows, int K, void* out, hipStream_t s) {
  const size_t n = rows * (size_t)(K / Q4_GROUP);
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  quantize_q4_kernel<<<(unsigned)blocks, 256, 0, s>>>((const uint16_t*)w, rows, K, (uint8_t*)out,
                                                      q4_scale_offset(rows, K));
  return hipGetLastError();
}

template <bool SILU>
__global__ __launch_bounds__(64 * QW) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemm_q4_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][QM * QK];

  const int E = p.E, N = p.N, K = p.K;
  const int NTB = (N + QN - 1) / QN;
  const int total = E * NTB;
  // expert-major block order, a contiguous range per XCD (workgroup ids are dealt round robin)
  const int q = total >> 3, rem = total & 7, xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int id = (xcd < rem) ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
  if (local >= ((xcd < rem) ? q + 1 : q)) return;
  const int e = id / NTB, n0 = (id - e * NTB) * QN;
  int lo = p.offsets[e], hi = p.offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > p.max_rows ? p.max_rows : lo);
  hi = hi < lo ? lo : (hi > p.max_rows ? p.max_rows : hi);
  if (hi <= lo) return;
  const int cols = min(N - n0, QN);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int nk = K / QK;
  const uint16_t* __restrict__ A = (const uint16_t*)p.A;
  uint16_t* __restrict__ C = (uint16_t*)p.C;
  // this wave's 16 weight rows form tile row (e N + n0 + 16 w) / 16 of the packed layout; per stage
  // the wave reads that tile's 1 KiB (16 bytes per lane: feature 16 w + fr, columns 32 fg .. + 31
  // of the stage) and the scale of the lane's 64-column group
  const uint8_t* bcode[QNB];
  const uint16_t* bscale[QNB];
#pragma unroll
  for (int b = 0; b < QNB; ++b) {
    const size_t trow = ((size_t)e * N + (size_t)(n0 + w * (QN / QW) + b * 16)) >> 4;   // N % 16 == 0
    bcode[b] = (const uint8_t*)p.B + trow * (size_t)(K / 128) * 1024 + (size_t)lane * 16;
    bscale[b] = (const uint16_t*)((const uint8_t*)p.B + p.q4_scale_off) + trow * (size_t)(K / 128) * 32 + 2 * fr +
                (fg >> 1);
  }

  // one chunk of at most QM rows with NRB 16-row blocks (NRB = ceil(rows / 16)), so that no
  // per-block branch sits inside the stage loop
  auto chunk = [&](int m0, int rows, auto nrb_c) {
    constexpr int NRB = decltype(nrb_c)::value;
    // activation loads per thread and stage that cover the chunk's NRB 16-row blocks (the rows
    // past them are never read by the MFMAs, so they are neither loaded nor staged)
    constexpr int QALN = (NRB * 16 * (QK / 8) + 64 * QW - 1) / (64 * QW);
    static_assert(QALN <= QAL, "the activation stage holds QM rows");
    // activation stage: up to 64 rows x 16 chunks of 8 columns; thread t moves chunks t + 64 QW i
    // (i < QALN). Rows past the chunk read its last row instead (they only feed outputs that are
    // not stored), and stages past the end read the last stage: no load sits behind a branch, so
    // the compiler's load counting stays exact and the prefetch is not drained. The prefetched
    // values are kept in flat arrays indexed by constants only (so they stay in registers).
    auto lda = [&](int st, int i) -> uint4 {
      st = min(st, nk - 1);
      const int c = tid + 64 * QW * i, r = min(c >> 4, rows - 1), ch = c & 15;
      return *(const uint4*)(A + (size_t)(m0 + r) * K + st * QK + ch * 8);
    };
    auto sta = [&](int buf, int i, uint4 v) {
      const int c = tid + 64 * QW * i, r = c >> 4, ch = c & 15;
      *(uint4*)(&sA[buf][r * QK + ((ch ^ (r & 7)) << 3)]) = v;
    };
    auto ldq = [&](int st, int b) -> uint4 { return *(const uint4*)(bcode[b] + (size_t)min(st, nk - 1) * 1024); };
    auto lds = [&](int st, int b) -> uint16_t { return bscale[b][min(st, nk - 1) * 32]; };
    // weight codes of stage t sit in slot t % WPD, loaded at stage t - WPD; activations of stage t
    // in slot t % QPD, loaded at stage t - QPD, go to LDS buffer t & 1 at the end of stage t - 1
    // and are read in stage t
    uint4 bq[WPD * QNB];
    uint16_t bs[WPD * QNB];
    uint4 ra[QPD * QAL];
#pragma unroll
    for (int u = 0; u < WPD; ++u)
#pragma unroll
      for (int b = 0; b < QNB; ++b) {
        bq[u * QNB + b] = ldq(u, b);
        bs[u * QNB + b] = lds(u, b);
      }
#pragma unroll
    for (int u = 0; u < QPD; ++u)
#pragma unroll
      for (int i = 0; i < QALN; ++i) ra[u * QAL + i] = lda(u, i);
    f32x4_t acc[NRB][QNB];
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int b = 0; b < QNB; ++b) acc[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < QALN; ++i) sta(0, i, ra[i]);
    __syncthreads();
    static_assert(WPD % QPD == 0, "the unrolled loop covers whole periods of both rings");
    for (int s0 = 0; s0 < nk; s0 += WPD) {
#pragma unroll
      for (int uw = 0; uw < WPD; ++uw) {
        const int s = s0 + uw;   // s % WPD == uw (nk is a multiple of WPD)
        const int u = uw % QPD;  // s % QPD
#pragma unroll
        for (int i = 0; i < QALN; ++i) ra[u * QAL + i] = lda(s + QPD, i);
        const uint16_t* a = sA[s & 1];
#pragma unroll
        for (int ks = 0; ks < QK / 32; ++ks) {
#pragma unroll
          for (int b = 0; b < QNB; ++b) {
            const uint4 cw = bq[uw * QNB + b];
            const uint32_t word = ks == 0 ? cw.x : ks == 1 ? cw.y : ks == 2 ? cw.z : cw.w;
            const bf16x8_t Bf = q4_dequant(word, bf16_bits_to_f32(bs[uw * QNB + b]));
#pragma unroll
            for (int i = 0; i < NRB; ++i) {
              const int r = i * 16 + fr, ch = 4 * fg + ks;   // columns 32 fg + 8 ks .. + 7 of the stage
              const bf16x8_t X = __builtin_bit_cast(bf16x8_t, *(const uint4*)(a + r * QK + ((ch ^ (r & 7)) << 3)));
              acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Bf, X, acc[i][b], 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int b = 0; b < QNB; ++b) {
          bq[uw * QNB + b] = ldq(s + WPD, b);
          bs[uw * QNB + b] = lds(s + WPD, b);
        }
        // the next stage's activations into the other buffer (after the last stage: a harmless
        // copy of the last stage into the buffer nobody reads any more)
        const int un = (u + 1) % QPD;
#pragma unroll
        for (int i = 0; i < QALN; ++i) sta((s + 1) & 1, i, ra[un * QAL + i]);
        __syncthreads();
      }
    }

    // lane holds features n0 + 16 w + 4 fg .. + 3 of row m0 + 16 i + fr
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      const int r = i * 16 + fr;
      if (r >= rows) continue;
#pragma unroll
      for (int b = 0; b < QNB; ++b) {
        const int n = w * (QN / QW) + b * 16 + 4 * fg;
        if (n >= cols) continue;
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = SILU ? q4_silu(acc[i][b][t]) : acc[i][b][t];
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *(uint2*)(C + (size_t)(m0 + r) * N + n0 + n) = o;
      }
    }
  };
  for (int m0 = lo; m0 < hi; m0 += QM) {
    const int rows = min(hi - m0, QM);
    const int nrb = __builtin_amdgcn_readfirstlane((rows + 15) / 16);
    if (nrb == 1) chunk(m0, rows, std::integral_constant<int, 1>{});
    else if (nrb == 2) chunk(m0, rows, std::integral_constant<int, 2>{});
    else if (nrb == 3) chunk(m0, rows, std::integral_constant<int, 3>{});
    else chunk(m0, rows, std::integral_constant<int, 4>{});
  }
}

hipError_t launch_gemm_q4(const GemmParams& p, bool silu, hipStream_t s) {
  const int grid = p.E * ((p.N + QN - 1) / QN);
  if (silu) gemm_q4_kernel<true><<<grid, 64 * QW, 0, s>>>(p);
  else gemm_q4_kernel<false><<<grid, 64 * QW, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
