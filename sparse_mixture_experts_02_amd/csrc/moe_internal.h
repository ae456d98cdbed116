// Internal declarations shared by the kernel files and the host API of libmoe.
// Not part of the public ABI (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------------------ tile constants

// Device-side copies of the public limits (include/moe.h).
constexpr int MOE_MAX_EXPERTS_DEV = 64;
constexpr int MOE_MAX_TOP_K_DEV = 8;

// Generic router: one wave per tile of ROUTE_TILE tokens (two 16-row MFMA tiles); the grid is
// capped so the per-wave probability partial sums stay small.
constexpr int ROUTE_TILE = 32;
constexpr int ROUTE_MAX_WAVES = 2048;

// Dispatch: tokens per histogram block of moe_dispatch's own histogram kernel (moe_forward uses
// the router's token groups, 16, 32 or 64 tokens), the most tokens a block may have, and the
// largest histogram (blocks x experts) that every dispatch workgroup sums itself (beyond it a
// one-workgroup scan kernel forms the block prefixes first).
constexpr int DISPATCH_BLOCK_TOKENS = 64;
constexpr int DISPATCH_MAX_BT = 64;
constexpr int DISPATCH_FUSED_MAX = 16384;

// Grouped GEMM tile (rows of the permuted activations x output columns).
constexpr int GEMM_BM = 128;
constexpr int GEMM_BN = 128;

// ------------------------------------------------------------------------------ device helpers

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// g * SiLU'(x) in fp32, SiLU'(x) = s (1 + x (1 - s)) with s = sigmoid(x) from the hardware exp2
// and reciprocal (their error is far below the bf16 rounding that follows); the FMA is explicit,
// so the rounding does not depend on how the compiler contracts the expression.
__device__ __forceinline__ float dsilu_mul(float g, float x) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
  return g * (s * __builtin_fmaf(x, 1.0f - s, 1.0f));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest, ties to even: one
// v_cvt_pk_bf16_f32 on gfx950 (checked bit-exact against f32_to_bf16_bits on 4M values
// including ties).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// ------------------------------------------------------------------------------ kernel params

struct RouteParams {
  int T, d, E, k;
  float tau;
  int renormalize;
  int straight_through;     // gate weight 1 for every selected expert
  const void* x;            // [T, d] act
  const float* w_router;    // [E, d] fp32, 16-byte aligned
  const float* bias;        // [E] or null
  const float* gumbel;      // [T, E] or null: Gumbel noise (selection key) or additive logit noise
  int noise_in_logits;      // 1: the noise is added to the logits
  const uint8_t* token_mask;   // [T] or null: 0 = padding token (not routed)
  const float* logits_in;   // [T, E] or null (skip the product)
  float* logits_out;        // [T, E] or null
  float* probs_out;         // [T, E] or null
  int32_t* ids;             // [T, k]
  float* weights;           // [T, k]
  double* psum;             // [route_num_parts][E + 2] per-workgroup statistics, or null
  int32_t* blk_hist;        // [route_blocks][E] selections per expert of each token group, or null
};

struct HistParams {
  int TK, E, k, bt;         // TK = T * k assignments; bt tokens per block
  const int32_t* ids;       // [TK]
  int32_t* blk_hist;        // [nb][E]
};

struct ScanParams {
  int nb, E, capacity, TK;
  const int32_t* blk_hist;  // [nb][E]
  int32_t* blk_base;        // [nb][E]
  int32_t* counts_pre;      // [E]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* n_dropped;       // [1]
};

struct AuxParams {
  int T, E, k, nparts;
  float coef;
  float tau;
  const double* psum;       // [nparts][E + 2]: probability sums, entropy sum, real-token count
  const int32_t* counts_pre;
  float* aux;               // [3]
};

// The dispatch proper: one workgroup per block of bt tokens ranks its slots and gathers its rows.
// With blk_base null it also sums the block histograms itself (block prefix and totals), and
// block 0 writes counts_pre, counts, offsets, n_dropped (and, with aux.aux set, the aux losses and
// shared_offsets); otherwise blk_base and offsets come from the scan kernel.
struct DispatchParams {
  int T, k, E, row_bytes, capacity;
  int bt, nb;               // tokens per block, blocks
  const int32_t* ids;       // [T, k]
  const int32_t* blk_hist;  // [nb][E]
  const int32_t* blk_base;  // [nb][E] pre-cut rank of each block's first slot per expert, or null
  int32_t* counts_pre;      // [E]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* n_dropped;       // [1]
  const uint8_t* x;
  int32_t* row_of;
  uint8_t* dropped;
  int32_t* perm_token;
  uint8_t* xp;
  AuxParams aux;            // aux.aux null: no aux losses
  int32_t* shared_offsets;  // [2] set to {0, T}, or null
};

struct GemmParams {
  int E, N, K;              // output columns N, reduction length K (per expert)
  int max_rows;             // rows of A/C allocated (T * k)
  const void* A;            // [rows, K] act
  const void* B;            // [E, N, K] weights
  void* C;                  // [rows, N] act
  const int32_t* offsets;   // [E+1]
  // Partial-sum workspace of the 256 x 256 kernel's split tail (gemm_big_part_bytes), or null:
  // whole tiles only.
  void* sk_part;
  // 4-bit weights: B is the packed buffer (codes, then bf16 scales from this byte offset)
  size_t q4_scale_off;
  // SiLU GEMMs: when not null, also receives the pre-activation (the accumulator rounded once to
  // act, before the SiLU), [rows, N] like C
  void* C2;
  // 256 x 256 kernel: a K-split tail may hold the emptiest tiles (sorted tile order). Set for the
  // products whose bits need not equal a first-layer product of the pre-activation variant (which
  // keeps the expert order): the second layer and the backward's dH and dXp.
  int sort_split;
  // 256 x 256 kernel, products without activation: B is stored [E, K, N] (the weights of the other
  // layer as they are) instead of [E, N, K]
  int b_kn;
};

struct CombineParams {
  int T, d, k;
  int max_rows;             // rows of y (T * k); a row index outside [0, max_rows) counts as dropped
  const void* y;
  const void* y_shared;     // [T, d] act added with weight 1 after the routed slots, or null
  const int32_t* row_of;
  const float* weights;     // [T, k], or null: every kept row with weight 1
  void* out;
};

struct CombineBwdParams {
  int T, d, k;
  int max_rows;
  const void* d_out;        // [T, d] act
  const void* y;            // [T*k, d] act (forward expert outputs)
  const int32_t* row_of;    // [T, k]
  const float* weights;     // [T, k]
  void* dy;                 // [T*k, d] act: dY[row] = w * dOut[t]
  float* dweights;          // [T, k]: <dOut[t], Y[row]>, 0 for slots without a row
};

struct ScanAuxParams {
  ScanParams s;
  AuxParams a;              // a.counts_pre is not read: the scan's own pre-cut counts are used
  int32_t* shared_offsets;  // [2] set to {0, T} (the shared expert's one segment), or null
};

struct ProbSumParams {
  int T, E;
  float tau;
  const float* probs;       // [T, E] or null
  const float* logits;      // [T, E] (used when probs is null)
  const uint8_t* token_mask;   // [T] or null
  double* psum;             // [gridDim][E + 2]
};

// ------------------------------------------------------------------------------ launchers
// Each returns the launch status (hipGetLastError after the launch).

int route_expert_tiles(int E);
int route_num_parts(int T, int E, bool bf16, bool logits_in);   // rows of psum a launch writes
int route_max_parts(int T, int E);
hipError_t launch_route(const RouteParams& p, bool bf16, hipStream_t s);

// token groups of the router's histogram (blocks of moe_forward's dispatch) and their count
int route_block_tokens(int T, int E, bool bf16, bool logits_in);
int dispatch_blocks(int T, int bt);
bool dispatch_fused(int nb, int E);
hipError_t launch_hist(const HistParams& p, hipStream_t s);
hipError_t launch_scan(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_aux(const ScanAuxParams& p, hipStream_t s);
hipError_t launch_dispatch(const DispatchParams& p, hipStream_t s);

int gemm_max_mtiles(int max_rows, int E);
hipError_t launch_gemm(const GemmParams& p, bool bf16, bool silu, hipStream_t s);
int gemm_big_grid(int max_rows, int E, int N);
size_t gemm_big_part_bytes();
// whether launch_gemm takes the 256 x 256 kernel for these operands
bool gemm_uses_big(bool bf16, int K, int max_rows, int E);
bool gemm_uses_stream(bool bf16, int K, int max_rows, int E);
hipError_t launch_gemm_big(const GemmParams& p, bool silu, hipStream_t s);
int gemm_stream_grid(int E, int N);
hipError_t launch_gemm_stream(const GemmParams& p, bool silu, hipStream_t s);

// 4-bit weights (packed codes + scales of a [rows, K] weight)
size_t q4_scale_offset(size_t rows, int K);
size_t q4_bytes(size_t rows, int K);
hipError_t launch_quantize_q4(const void* w, size_t rows, int K, void* out, hipStream_t s);
hipError_t launch_gemm_q4(const GemmParams& p, bool silu, hipStream_t s);

hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s);

// backward pass
struct GradWParams {
  int E, M, N;              // output per expert [M, N]
  int max_rows;             // rows of P and Q (T * k)
  const void* P;            // [rows, M] act
  const void* Q;            // [rows, N] act
  const int32_t* offsets;   // [E+1] expert segments of the rows
  float* G;                 // [E, M, N] fp32
  int splits;               // set by launch_grad_w: 1, or 2 (each tile's rows in two halves, added into G)
};
hipError_t launch_grad_w(const GradWParams& p, bool bf16, hipStream_t s);
struct RouteBwdParams {
  int T, d, E, k;
  float tau, coef, d_aux;
  int renormalize;
  const void* x;            // [T, d] act
  const float* w_router;    // [E, d]
  const float* logits;      // [T, E] (the forward's logits, noise included in the additive mode)
  const int32_t* ids;       // [T, k]
  const float* weights;     // [T, k]
  const float* dweights;    // [T, k]
  const int32_t* counts_pre;   // [E]
  const uint8_t* token_mask;   // [T] or null
  float* dlogits;           // [T, E] out
  void* dx;                 // [T, d] act, accumulated into, or null
  float* dw_router;         // [E, d] or null
  float* dbias;             // [E] or null
  float* part;              // [chunks, E, d] fp32 workspace of the router weight gradient
  int chunks, chunk_tokens; // set by launch_route_bwd
  // moe_backward (route_bwd_fuses_gather): when dxp is not null, dx is written, not read: each
  // token's dx is the sum of its kept slots' rows of dxp [max_rows, d] (row_of, slot order), then
  // its row of dxs [T, d] when not null, then the router term, in fp32 with one rounding to act
  const void* dxp;
  const int32_t* row_of;    // [T, k]
  int max_rows;
  const void* dxs;
};
// Whether launch_route_bwd can also form dx from the gather (bf16, top-1 or top-2, E <= 16)
bool route_bwd_fuses_gather(bool bf16, int E, int k);
size_t route_bwd_part_bytes(int T, int d, int E);
hipError_t launch_route_bwd(const RouteBwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_combine_bwd(const CombineBwdParams& p, bool bf16, hipStream_t s);
// out[b, c, r] = in[b, r, c] for a batch of [R, C] matrices (elements of `elem` bytes, 2 or 4)
hipError_t launch_transpose(const void* in, void* out, int B, int R, int C, int elem, hipStream_t s);
// dA = dH * SiLU'(A), elementwise over n values (act dtype)
// nrows: device pointer to the number of rows to process (at most max_rows), e.g. offsets + E
hipError_t launch_silu_bwd(const void* dh, const void* a, void* da, const int32_t* nrows, int max_rows, int cols,
                           bool bf16, hipStream_t s);

int probsum_num_blocks(int T);
hipError_t launch_probsum(const ProbSumParams& p, hipStream_t s);
hipError_t launch_aux_final(const AuxParams& p, hipStream_t s);

}  // namespace moe
