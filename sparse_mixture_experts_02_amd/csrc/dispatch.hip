// Dispatch kernels: per-expert histogram with stable in-block ranks, the cross-block scan with
// the capacity cut, and the scatter of row indices fused with the row gather x -> Xp.
//
// [P4 §2.4] sort the [T, k] expert index by expert id, count the tokens of each expert, split
// them into per-expert segments and collect each expert's tokens with a table lookup.
// [P3 §3.1, §3.4] cap the tokens one expert processes (capacity); the overflow is dropped.
// Assignments are ranked in flattened (token, slot) order, so each expert keeps its first C
// assignments in token order and its segment lists tokens in increasing order.
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------------------------ histogram
// Block b ranks assignments [b*CHUNK, (b+1)*CHUNK) in order. Within a wave, the lanes that hold
// the same expert are found with ballots (one ballot per distinct expert in the wave); the
// rank of a lane is the number of such lanes below it. Wave counts are combined in LDS in wave
// order, then chunk rounds in order, so rank_local is the stable rank inside the block.
__device__ __forceinline__ void hist_block(const HistParams& p) {
  __shared__ int wave_cnt[4][MOE_MAX_EXPERTS_DEV];
  __shared__ int wave_base[4][MOE_MAX_EXPERTS_DEV];
  __shared__ int running[MOE_MAX_EXPERTS_DEV];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int E = p.E;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  if (tid < E) running[tid] = 0;
  const int base = blockIdx.x * DISPATCH_CHUNK;
  for (int round = 0; round < DISPATCH_CHUNK / 256; ++round) {
    for (int i = tid; i < 4 * MOE_MAX_EXPERTS_DEV; i += 256) (&wave_cnt[0][0])[i] = 0;
    __syncthreads();
    const int i = base + round * 256 + tid;
    int e = (i < p.TK) ? p.ids[i] : -1;
    const bool ok = e >= 0 && e < E;   // out-of-range ids are left unranked (never written)
    if (!ok) e = -1;
    uint64_t todo = __ballot(ok);
    int my_rank = 0;
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int le = __shfl(e, leader);
      const uint64_t peers = __ballot(ok && e == le);
      if (ok && e == le) {
        my_rank = __popcll(peers & lt_mask);
        if (lane == leader) wave_cnt[w][e] = __popcll(peers);
      }
      todo &= ~peers;
    }
    __syncthreads();
    if (tid < E) {
      int run = running[tid];
      for (int ww = 0; ww < 4; ++ww) {
        wave_base[ww][tid] = run;
        run += wave_cnt[ww][tid];
      }
      running[tid] = run;
    }
    __syncthreads();
    if (ok) p.rank_local[i] = wave_base[w][e] + my_rank;
    __syncthreads();
  }
  __syncthreads();
  if (tid < E) p.blk_hist[(size_t)blockIdx.x * E + tid] = running[tid];
}

__global__ __launch_bounds__(256) void hist_kernel(HistParams p) { hist_block(p); }

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
__device__ __forceinline__ void aux_block(const AuxParams& p, const int* counts_pre) {
  __shared__ double part[256];
  __shared__ double S[MOE_MAX_EXPERTS_DEV + 2];
  const int tid = threadIdx.x;
  const int E = p.E;
  const int C = E + 2;   // columns of a statistics row: E probability sums, entropy, count
  int CPAD = 1;
  while (CPAD < C) CPAD <<= 1;
  const int c = tid % CPAD;
  const int sub = tid / CPAD;
  const int nsub = 256 / CPAD;
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

__global__ __launch_bounds__(256) void aux_final_kernel(AuxParams p) { aux_block(p, p.counts_pre); }

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
  aux_block(p.a, pre);
  if (p.shared_offsets && threadIdx.x < 2) p.shared_offsets[threadIdx.x] = threadIdx.x == 0 ? 0 : p.a.T;
}

// ------------------------------------------------------------------------------ gather
// One wave per token. Lanes j < k resolve slot j: global pre-cut rank = block base + local
// rank; kept iff rank < C; row = offsets[e] + rank. The wave then reads the token's row of x
// once (16 B per lane per step) and writes it to each kept row of Xp.
__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int k = p.k;
  int row = -1;
  if (lane < k) {
    const int i = t * k + lane;
    const int e = p.ids[i];
    bool keep = false;
    int rank = 0;
    if (e >= 0 && e < p.E) {   // an id outside [0, E) (a padding token's -1) has no row
      rank = p.blk_base[(size_t)(i / DISPATCH_CHUNK) * p.E + e] + p.rank_local[i];
      keep = p.capacity < 0 || rank < p.capacity;
    }
    row = keep ? p.offsets[e] + rank : -1;
    p.row_of[i] = row;
    p.dropped[i] = (e >= 0 && e < p.E && !keep) ? 1 : 0;   // a -1 slot (padding) is not dropped
    if (keep) p.perm_token[row] = t;
  }
  int rows[MOE_MAX_TOP_K_DEV];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K_DEV; ++j) rows[j] = (j < k) ? __shfl(row, j) : -1;
  const int nvec = p.row_bytes / 16;
  const uint4* __restrict__ src = (const uint4*)(p.x + (size_t)t * p.row_bytes);
  for (int c = lane; c < nvec; c += 64) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOP_K_DEV; ++j)
      if (rows[j] >= 0) ((uint4*)(p.xp + (size_t)rows[j] * p.row_bytes))[c] = v;
  }
}

int dispatch_num_blocks(int TK) { return (TK + DISPATCH_CHUNK - 1) / DISPATCH_CHUNK; }

hipError_t launch_hist(const HistParams& p, hipStream_t s) {
  hist_kernel<<<dispatch_num_blocks(p.TK), 256, 0, s>>>(p);
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

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
  gather_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
