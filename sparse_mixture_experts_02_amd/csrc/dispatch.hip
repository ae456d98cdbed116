// Dispatch kernels: per-block expert histograms, the scan of the block histograms with the
// capacity cut, and the dispatch proper: stable ranks, the row map and the row gather x -> Xp.
//
// [P4 §2.4] sort the [T, k] expert index by expert id, count the tokens of each expert, split
// them into per-expert segments and collect each expert's tokens with a table lookup.
// [P3 §3.1, §3.4] cap the tokens one expert processes (capacity); the overflow is dropped.
// Assignments are ranked in flattened (token, slot) order, so each expert keeps its first C
// assignments in token order and its segment lists tokens in increasing order.
//
// Blocks are runs of bt consecutive tokens. blk_hist[b][e] counts the slots of block b that chose
// expert e: in moe_forward the router writes it for its own token groups; moe_dispatch runs
// hist_kernel. The pre-cut rank of a slot is (slots of its expert in earlier blocks) + (slots of
// its expert earlier in its block); the dispatch workgroup of a block forms the first term from
// the histograms and the second from the block's ids with wave ballots.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

// ------------------------------------------------------------------------------ histogram
// One workgroup per block of bt tokens: counts per expert with LDS integer atomics (the counts do
// not depend on their order). ids outside [0, E) (a padding token's -1) are not counted.
__global__ __launch_bounds__(256) void hist_kernel(HistParams p) {
  __shared__ int cnt[MOE_MAX_EXPERTS_DEV];
  const int tid = threadIdx.x;
  if (tid < p.E) cnt[tid] = 0;
  __syncthreads();
  const int n = p.bt * p.k;
  const size_t i0 = (size_t)blockIdx.x * n;
  for (int i = tid; i < n; i += 256) {
    const size_t gi = i0 + i;
    if (gi < (size_t)p.TK) {
      const int e = p.ids[gi];
      if (e >= 0 && e < p.E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid < p.E) p.blk_hist[(size_t)blockIdx.x * p.E + tid] = cnt[tid];
}

// ------------------------------------------------------------------------------ scan
// One block. For each expert: exclusive scan of the block histograms (the pre-cut rank of
// each block's first assignment), the pre-cut total, the kept count min(total, C); then the
// exclusive scan of kept counts gives the segment offsets.
// `pre` (LDS, E entries) receives the pre-cut counts.
__device__ __forceinline__ void scan_block(const ScanParams& p, int* pre) {
  __shared__ int kept[MOE_MAX_EXPERTS_DEV];
  const int tid = threadIdx.x;
  const int E = p.E;
  // Threads are split into E groups of G lanes; group e scans column e. Each lane sums a
  // contiguous run of blocks, the lanes' totals are scanned in lane order, then each lane
  // writes its run's exclusive prefixes.
  __shared__ int part[256];
  const int G = 256 / E >= 1 ? 256 / E : 1;
  const int e = tid / G;
  const int g = tid % G;
  const bool active = e < E;
  const int per = (p.nb + G - 1) / G;
  const int b0 = g * per;
  const int b1 = min(p.nb, b0 + per);
  int local = 0;
  auto hist = [&](int b) { return p.blk_hist[(size_t)b * E + e]; };
  if (active)
    for (int b = b0; b < b1; ++b) local += hist(b);
  part[tid] = local;
  __syncthreads();
  if (active) {
    int before = 0;
    for (int q = 0; q < g; ++q) before += part[e * G + q];
    int run = before;
    for (int b = b0; b < b1; ++b) {
      p.blk_base[(size_t)b * E + e] = run;
      run += hist(b);
    }
    if (g == G - 1) {
      pre[e] = run;
      kept[e] = (p.capacity < 0 || run < p.capacity) ? run : p.capacity;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    int total_pre = 0;
    for (int q = 0; q < E; ++q) {
      p.offsets[q] = off;
      p.counts_pre[q] = pre[q];
      p.counts[q] = kept[q];
      off += kept[q];
      total_pre += pre[q];
    }
    p.offsets[E] = off;
    *p.n_dropped = total_pre - off;
  }
}

__global__ __launch_bounds__(256) void scan_kernel(ScanParams p) {
  __shared__ int pre[MOE_MAX_EXPERTS_DEV];
  scan_block(p, pre);
}

// ------------------------------------------------------------------------------ aux losses
// [P4 §3.2, P3 §3.2] One block: P_i = (sum of the partial sums) / T, then both losses in double, stored as fp32.
// The partial rows of expert e are split over the lanes (e, sub), sub = 0 .. nsub-1; each lane
// keeps 4 independent running sums (so its loads overlap) and all sums are combined in a fixed
// order, so the result does not depend on timing.
template <int NT>
__device__ __forceinline__ void aux_block(const AuxParams& p, const int* counts_pre) {
  __shared__ double part[NT];
  __shared__ double S[MOE_MAX_EXPERTS_DEV + 2];
  const int tid = threadIdx.x;
  const int E = p.E;
  const int C = E + 2;   // columns of a statistics row: E probability sums, entropy, count
  int CPAD = 1;
  while (CPAD < C) CPAD <<= 1;
  const int c = tid % CPAD;
  const int sub = tid / CPAD;
  const int nsub = NT / CPAD;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  if (c < C) {
    int q = sub;
    for (; q + 3 * nsub < p.nparts; q += 4 * nsub) {
      a0 += p.psum[(size_t)q * C + c];
      a1 += p.psum[(size_t)(q + nsub) * C + c];
      a2 += p.psum[(size_t)(q + 2 * nsub) * C + c];
      a3 += p.psum[(size_t)(q + 3 * nsub) * C + c];
    }
    for (; q < p.nparts; q += nsub) a0 += p.psum[(size_t)q * C + c];
  }
  part[tid] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (tid < C) {
    double s = 0.0;
    for (int q = 0; q < nsub; ++q) s += part[q * CPAD + tid];
    S[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    const double n = S[E + 1];   // real tokens (an exact integer)
    double sw = 0.0, sb = 0.0, ent = 0.0;
    if (n > 0.0) {
      const double nk = n * (double)p.k;
      const double uni = (double)p.k / (double)E;
      for (int q = 0; q < E; ++q) {
        const double cq = (double)counts_pre[q];
        sw += (cq / nk) * (S[q] / n);
        const double dv = cq / n - uni;
        sb += dv * dv;
      }
      sw *= (double)p.coef * (double)E;
      sb *= (double)p.coef;
      ent = S[E] / n;
    }
    p.aux[0] = (float)sw;
    p.aux[1] = (float)sb;
    p.aux[2] = (float)ent;
  }
}

__global__ __launch_bounds__(256) void aux_final_kernel(AuxParams p) { aux_block<256>(p, p.counts_pre); }

hipError_t launch_aux_final(const AuxParams& p, hipStream_t s) {
  aux_final_kernel<<<1, 256, 0, s>>>(p);
  return hipGetLastError();
}


// ------------------------------------------------------------------------------ scan + aux
// The scan, then (in the same block, from the pre-cut counts it just formed) both aux losses:
// one launch fewer in the forward pass.
__global__ __launch_bounds__(256) void scan_aux_kernel(ScanAuxParams p) {
  __shared__ int pre[MOE_MAX_EXPERTS_DEV];
  scan_block(p.s, pre);
  __syncthreads();
  aux_block<256>(p.a, pre);
  if (p.shared_offsets && threadIdx.x < 2) p.shared_offsets[threadIdx.x] = threadIdx.x == 0 ? 0 : p.a.T;
}

// ------------------------------------------------------------------------------ dispatch
// One workgroup of 16 waves per block of bt = 16 TB tokens (TB = 1, 2, 4).
//  1. The block's ids into LDS. Without blk_base: the per-expert sums of the histograms over the
//     earlier blocks (this block's base ranks) and over all blocks (the pre-cut counts), every
//     workgroup on its own (the histograms are small and read from L2), then the kept counts
//     min(count, C) and their exclusive scan (the segment offsets). One more workgroup (index nb)
//     stores counts_pre, counts, offsets and n_dropped and finishes the aux losses, beside the
//     others.
//  2. Wave w takes tokens w + 16 i, i < TB: for each slot j the rank inside the block is the number
//     of earlier slots of the block with the same expert (ballots over the ids in LDS), the pre-cut
//     rank adds the block's base; kept iff rank < C; row = offset + rank. Lanes j < k write the row
//     map. Then the wave copies its tokens' rows of x to their kept rows of Xp, the loads of all TB
//     tokens in flight before their stores.
template <bool FUSED, int TB>
__global__ __launch_bounds__(1024) void dispatch_kernel(DispatchParams p) {
  __shared__ int s_ids[DISPATCH_MAX_BT * MOE_MAX_TOP_K_DEV];
  __shared__ int s_base[MOE_MAX_EXPERTS_DEV];
  __shared__ int s_off[MOE_MAX_EXPERTS_DEV + 1];
  __shared__ int s_tot[MOE_MAX_EXPERTS_DEV];
  __shared__ int red[2][1024];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = p.E, k = p.k, b = blockIdx.x;
  const bool stats = b == p.nb;   // the extra workgroup: counts, offsets, aux losses
  const int t0 = b * p.bt;
  const int nt = stats ? 0 : min(p.bt, p.T - t0);
  for (int i = tid; i < nt * k; i += 1024) s_ids[i] = p.ids[(size_t)t0 * k + i];
  if constexpr (FUSED) {
    // thread (g, e): blocks g, g + G, ... of expert column e (consecutive threads read
    // consecutive ints), four loads in flight
    const int G = 1024 / E;
    const int e = tid % E, g = tid / E;
    int pre = 0, tot = 0;
    if (g < G) {
      int q = g;
      for (; q + 3 * G < p.nb; q += 4 * G) {
        const int v0 = p.blk_hist[(size_t)q * E + e];
        const int v1 = p.blk_hist[(size_t)(q + G) * E + e];
        const int v2 = p.blk_hist[(size_t)(q + 2 * G) * E + e];
        const int v3 = p.blk_hist[(size_t)(q + 3 * G) * E + e];
        tot += (v0 + v1) + (v2 + v3);
        pre += (q < b ? v0 : 0) + (q + G < b ? v1 : 0) + (q + 2 * G < b ? v2 : 0) + (q + 3 * G < b ? v3 : 0);
      }
      for (; q < p.nb; q += G) {
        const int v = p.blk_hist[(size_t)q * E + e];
        tot += v;
        pre += q < b ? v : 0;
      }
    }
    red[0][tid] = pre;
    red[1][tid] = tot;
    __syncthreads();
    for (int ee = w; ee < E; ee += 16) {   // wave w: expert columns w, w + 16, ...
      int a = 0, c = 0;
      for (int gg = lane; gg < G; gg += 64) {
        a += red[0][gg * E + ee];
        c += red[1][gg * E + ee];
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        a += __shfl_xor(a, m);
        c += __shfl_xor(c, m);
      }
      if (lane == 0) {
        s_base[ee] = a;
        s_tot[ee] = c;
      }
    }
    __syncthreads();
    if (w == 0) {   // kept counts and their exclusive scan over the experts (E <= 64: one wave)
      const int cnt = lane < E ? s_tot[lane] : 0;
      const int kept = (p.capacity < 0 || cnt < p.capacity) ? cnt : p.capacity;
      int inc = kept;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int v = __shfl_up(inc, m);
        if (lane >= m) inc += v;
      }
      if (lane < E) s_off[lane] = inc - kept;
      if (stats) {
        int drop = cnt - kept;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) drop += __shfl_xor(drop, m);
        if (lane < E) {
          p.counts_pre[lane] = cnt;
          p.counts[lane] = kept;
          p.offsets[lane] = inc - kept;
        }
        if (lane == E - 1) p.offsets[E] = inc;
        if (lane == 0) *p.n_dropped = drop;
        if (p.shared_offsets && lane < 2) p.shared_offsets[lane] = lane == 0 ? 0 : p.T;
      }
    }
    if (stats) {
      if (p.aux.aux) {
        __syncthreads();
        aux_block<1024>(p.aux, s_tot);
      }
      return;   // uniform within the workgroup
    }
  } else {
    if (tid < E) {
      s_base[tid] = p.blk_base[(size_t)b * E + tid];
      s_off[tid] = p.offsets[tid];
    }
  }
  __syncthreads();

  // per-token steps, expanded at compile time for tokens i = 0 .. TB - 1 (constant indices keep the
  // arrays below in registers)
  auto each_token = [&](auto f) {
    f(std::integral_constant<int, 0>{});
    if constexpr (TB > 1) f(std::integral_constant<int, 1>{});
    if constexpr (TB > 2) {
      f(std::integral_constant<int, 2>{});
      f(std::integral_constant<int, 3>{});
    }
  };
  int myrow[TB];   // token i's slot-j row in lane j (-1: dropped or no row)
  each_token([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int tt = w + 16 * i;
    int my_row = -1, my_drop = 0;
    if (tt < nt) {   // uniform within the wave
      for (int j = 0; j < k; ++j) {
        const int pos = tt * k + j;
        const int e = s_ids[pos];
        const bool valid = e >= 0 && e < E;
        int local = 0;
        for (int q0 = 0; q0 < pos; q0 += 64) {
          const int q = q0 + lane;
          local += __popcll(__ballot(q < pos && s_ids[q] == e));
        }
        const int rank = (valid ? s_base[e] : 0) + local;
        const bool keep = valid && (p.capacity < 0 || rank < p.capacity);
        if (lane == j) {
          my_row = keep ? s_off[e] + rank : -1;
          my_drop = valid && !keep;
        }
      }
      if (lane < k) {
        const size_t idx = (size_t)(t0 + tt) * k + lane;
        p.row_of[idx] = my_row;
        p.dropped[idx] = (uint8_t)my_drop;
        if (my_row >= 0) p.perm_token[my_row] = t0 + tt;
      }
    }
    myrow[i] = my_row;
  });
  // (a native vector type: an array of HIP's uint4 structs is not kept in registers)
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int nvec = p.row_bytes / 16;
  for (int c0 = 0; c0 < nvec; c0 += 256) {
    u32x4 v[TB][4];
    each_token([&](auto ic) {   // clamped token and column: every load is issued unconditionally
      constexpr int i = decltype(ic)::value;
      const u32x4* __restrict__ src = (const u32x4*)(p.x + (size_t)(t0 + min(w + 16 * i, nt - 1)) * p.row_bytes);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[i][u] = src[min(c0 + u * 64 + lane, nvec - 1)];
    });
    // every load has landed before the first store: without this the compiler, unable to count
    // the conditional stores, waits for all earlier stores before each group of them
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt not waited
    each_token([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (w + 16 * i >= nt) return;   // uniform within the wave
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOP_K_DEV; ++j) {   // unrolled: v stays in registers
        if (j >= k) break;
        const int r = __builtin_amdgcn_readlane(myrow[i], j);
        if (r < 0) continue;
        u32x4* __restrict__ dst = (u32x4*)(p.xp + (size_t)r * p.row_bytes);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < nvec) dst[c] = v[i][u];
        }
      }
    });
  }
}

int dispatch_blocks(int T, int bt) { return (T + bt - 1) / bt; }

bool dispatch_fused(int nb, int E) { return (long)nb * E <= DISPATCH_FUSED_MAX; }

hipError_t launch_hist(const HistParams& p, hipStream_t s) {
  hist_kernel<<<dispatch_blocks(p.TK / p.k, p.bt), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanParams& p, hipStream_t s) {
  scan_kernel<<<1, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_scan_aux(const ScanAuxParams& p, hipStream_t s) {
  scan_aux_kernel<<<1, 256, 0, s>>>(p);
  return hipGetLastError();
}

template <int TB>
static void launch_dispatch_tb(const DispatchParams& p, hipStream_t s) {
  // fused: one more workgroup for the counts, offsets and aux losses
  if (p.blk_base) dispatch_kernel<false, TB><<<p.nb, 1024, 0, s>>>(p);
  else dispatch_kernel<true, TB><<<p.nb + 1, 1024, 0, s>>>(p);
}

hipError_t launch_dispatch(const DispatchParams& p, hipStream_t s) {
  switch (p.bt) {   // the router's token groups (16, 32, 64) or moe_dispatch's blocks (64)
    case 16: launch_dispatch_tb<1>(p, s); break;
    case 32: launch_dispatch_tb<2>(p, s); break;
    case 64: launch_dispatch_tb<4>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
