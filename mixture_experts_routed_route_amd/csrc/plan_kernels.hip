// Plan kernels of the routed MoE layer on gfx950: route (top-k + weights +
// per-chunk expert histogram), the capacity scan, and the stable permute
// into an expert-sorted pair list.
//
// The router keeps each token's k best experts and renormalises their
// softmax weights over those k (mini-AGI PR #3, minagi/pool.py,
// `requested(scores)`). An expert keeps at most `limit` pairs, first come in
// token order; the kept pairs are grouped by expert (the `keep` filter and
// the argsort/bincount of minagi/pool.py in mini-AGI PR #3 and #4). Here the
// grouping is a chunked histogram, a column scan and an in-chunk stable rank:
// deterministic, with no atomics in any ordering decision.
#include "moe_internal.h"

namespace moe {

// Order-preserving map of a float onto uint32: larger float -> larger key.
// +0 and -0 map to one key; NaN maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) == 0u) b = 0u;
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

// Number of lanes whose predicate holds, over the wave.
__device__ __forceinline__ int wave_count(bool pred) {
  return __popcll(__ballot(pred));
}

// One wavefront per token; PER = ceil(E / 64) logits per lane (expert
// lane + 64 p). The k-th largest order key tau is built bit by bit from the
// top (a candidate stays if at least k keys reach it): 32 steps of
// compare + ballot + popcount, no data exchange between lanes. Keys above
// tau are chosen, then keys equal to tau in expert order until k are
// chosen, so equal logits resolve to the lower expert index. A chosen
// expert's position j is the number of chosen experts ranked above it.
// Weights: exp(l_j - l_0) / sum_i exp(l_i - l_0) in double, rounded to f32.
// Block = 16 waves x TPW tokens; the block's histogram row
// hist[block, 0..E-1] counts its tokens' choices per expert, and
// hist[block, E] their NaN logits.
template <int PER, int TPW>
__global__ __launch_bounds__(1024) void route_hist_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ hist) {
  extern __shared__ int32_t sh_hist[];   // E + 1
  constexpr int kTokPerWave = TPW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) sh_hist[e] = 0;
  __syncthreads();

  const int tbase = chunk * 16 * TPW + wave * kTokPerWave;
  // every logit this wave needs, loaded up front
  float lv[kTokPerWave][PER];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int t = tbase + i;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = lane + 64 * p;
      lv[i][p] = (t < T && e < E) ? logits[(size_t)t * E + e] : 0.f;
    }
  }
  // keys of the wave's tokens (a token past T has no valid expert: it
  // chooses nothing and writes nothing)
  uint32_t key[kTokPerWave][PER];
  bool valid[kTokPerWave][PER];
  int nan_count = 0;
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i)
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      valid[i][p] = tbase + i < T && lane + 64 * p < E;
      key[i][p] = order_key(lv[i][p]);
      nan_count += (valid[i][p] && lv[i][p] != lv[i][p]) ? 1 : 0;
    }
  // tau: the k-th largest key of each token, the tokens side by side
  uint32_t tau[kTokPerWave];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) tau[i] = 0u;
  for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
      const uint32_t test = tau[i] | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int p = 0; p < PER; ++p) cnt += wave_count(valid[i][p] && key[i][p] >= test);
      if (cnt >= k) tau[i] = test;
    }
  }
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int t = tbase + i;
    int above = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) above += wave_count(valid[i][p] && key[i][p] > tau[i]);
    // ties at tau: the first (k - above) in expert order
    int ties_before = 0;
    bool sel[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const bool eqp = valid[i][p] && key[i][p] == tau[i];
      const uint64_t eq = __ballot(eqp);
      const int r = ties_before + __popcll(eq & lanes_below);
      sel[p] = valid[i][p] && (key[i][p] > tau[i] || (eqp && r < k - above));
      ties_before += __popcll(eq);
    }
    // positions: chosen experts ranked above each chosen one; the largest
    // chosen key is l_0's
    int pos[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) pos[p] = 0;
    uint32_t top = 0u;
#pragma unroll
    for (int pp = 0; pp < PER; ++pp) {
      uint64_t m = __ballot(sel[pp]);
      while (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const uint32_t ko = (uint32_t)__builtin_amdgcn_readlane((int)key[i][pp], l);
        const int eo = l + 64 * pp;
        top = ko > top ? ko : top;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
          const int e = lane + 64 * p;
          pos[p] += (sel[p] && (ko > key[i][p] || (ko == key[i][p] && eo < e))) ? 1 : 0;
        }
      }
    }
    const double l0 = (double)key_value(top);
    double ex[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) ex[p] = sel[p] ? exp((double)lv[i][p] - l0) : 0.0;
    // the sum in expert order, the same in every lane
    double sum = 0.0;
#pragma unroll
    for (int pp = 0; pp < PER; ++pp) {
      uint64_t m = __ballot(sel[pp]);
      while (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const uint64_t bits = (uint64_t)__double_as_longlong(ex[pp]);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), l);
        sum += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
      }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      if (sel[p]) {
        const int e = lane + 64 * p;
        ids[(size_t)t * k + pos[p]] = e;
        w[(size_t)t * k + pos[p]] = (float)(ex[p] / sum);
        atomicAdd(&sh_hist[e], 1);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nan_count += __shfl_xor(nan_count, off);
  if (lane == 0 && nan_count) atomicAdd(&sh_hist[E], nan_count);
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x)
    hist[(size_t)chunk * (E + 1) + e] = sh_hist[e];
}

hipError_t launch_route_hist(const float* logits, int T, int E, int k,
                             int32_t* ids, float* w, int32_t* hist, int tpw,
                             hipStream_t s) {
  if (tpw != 1 && tpw != 4) return hipErrorInvalidValue;
  const int NR = (T + 16 * tpw - 1) / (16 * tpw);
  const size_t sh = (size_t)(E + 1) * sizeof(int32_t);
  const int per = (E + 63) / 64;
#define MOE_ROUTE(P)                                                             \
  do {                                                                           \
    if (tpw == 1)                                                                \
      hipLaunchKernelGGL((route_hist_kernel<P, 1>), dim3(NR), dim3(1024), sh, s, \
                         logits, T, E, k, ids, w, hist);                         \
    else                                                                         \
      hipLaunchKernelGGL((route_hist_kernel<P, 4>), dim3(NR), dim3(1024), sh, s, \
                         logits, T, E, k, ids, w, hist);                         \
  } while (0)
  if (per <= 1) MOE_ROUTE(1);
  else if (per <= 2) MOE_ROUTE(2);
  else if (per <= 4) MOE_ROUTE(4);
  else if (per <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}

// ---- block helpers (1024 threads) ----------------------------------------

// Exclusive scan of v over the block in thread order; returns the prefix and
// writes the block total to *total. 16 waves of 64.
__device__ __forceinline__ int block_scan_excl(int v, int* total,
                                               int* sh_waves /*[16]*/) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh_waves[wave] = incl;
  __syncthreads();
  int wave_pre = 0, tot = 0;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) {
    const int t = sh_waves[i];
    if (i < wave) wave_pre += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wave_pre + incl - v;
}

// One block of 1024 threads. The chunk columns of the E + 1 histogram
// columns are cut into P parts (P = 1024 / (E + 1), at most 16), so thread
// (part, column) scans one part of one column, twice: first the part sums,
// then in-place exclusive bases. Afterwards: kept counts min(total, limit),
// offsets by exclusive scan over experts (the shared expert, if any, last
// with T rows), and the plan counters.
__global__ __launch_bounds__(1024) void scan_kernel(
    int32_t* __restrict__ hist, int NC, int T, int E, int k, int n_shared,
    int64_t limit, int32_t* __restrict__ total, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int64_t* __restrict__ stats) {
  __shared__ int part_sum[1024];
  __shared__ int tot[kMaxExperts + 1];
  __shared__ int sh_waves[16];
  __shared__ int red[4];
  const int EH = E + 1;
  const int P = max(1, min(16, (int)blockDim.x / EH));
  const int W = (int)blockDim.x / P;          // columns per pass
  const int part = threadIdx.x / W;
  const int col = threadIdx.x - part * W;
  const int cp = (NC + P - 1) / P;
  const int c0 = min(NC, part * cp);
  const int c1 = min(NC, c0 + cp);
  for (int g = 0; g < EH; g += W) {
    const int e = g + col;
    const bool mine = part < P && e < EH;
    int s = 0;
    if (mine) {
#pragma unroll 8
      for (int c = c0; c < c1; ++c) s += hist[(size_t)c * EH + e];
    }
    if (part < P) part_sum[part * W + col] = s;
    __syncthreads();
    if (mine) {
      int run = 0;
      for (int p = 0; p < part; ++p) run += part_sum[p * W + col];
#pragma unroll 8
      for (int c = c0; c < c1; ++c) {
        const size_t ix = (size_t)c * EH + e;
        const int v = hist[ix];
        hist[ix] = run;
        run += v;
      }
      if (part == P - 1) tot[e] = run;
    }
    __syncthreads();
  }
  if (threadIdx.x < 4) red[threadIdx.x] = 0;
  __syncthreads();
  // kept counts, drop statistics
  int kept_local = 0, touched_local = 0, max_local = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    total[e] = tot[e];
    const int c = (limit < 0 || (int64_t)tot[e] < limit) ? tot[e] : (int)limit;
    counts[e] = c;
    kept_local += c;
    touched_local += c > 0 ? 1 : 0;
    max_local = max(max_local, c);
  }
  if (kept_local) atomicAdd(&red[0], kept_local);
  if (touched_local) atomicAdd(&red[1], touched_local);
  if (max_local) atomicMax(&red[2], max_local);
  if (n_shared && threadIdx.x == 0) counts[E] = T;
  __syncthreads();
  // offsets over E + n_shared experts, in blocks of 1024 with a carry
  const int n = E + n_shared;
  int carry = 0;
  for (int b = 0; b < n; b += blockDim.x) {
    const int e = b + threadIdx.x;
    int c = 0;
    if (e < E) {
      c = (limit < 0 || (int64_t)tot[e] < limit) ? tot[e] : (int)limit;
    } else if (e < n) {
      c = T;
    }
    int blk_total = 0;
    const int pre = block_scan_excl(c, &blk_total, sh_waves);
    if (e < n) offsets[e] = carry + pre;
    carry += blk_total;
  }
  if (threadIdx.x == 0) {
    offsets[n] = carry;
    const int64_t pairs = (int64_t)T * k;
    stats[0] = pairs - red[0];       // dropped
    stats[1] = red[0];               // kept
    stats[2] = tot[E];               // NaN logits
    stats[3] = red[1];               // touched experts
    stats[4] = red[2];               // max rows
    stats[5] = 0;
    stats[6] = 0;
    stats[7] = 0;
  }
}

hipError_t launch_scan(int32_t* hist, int NC, int T, int E, int k,
                       int n_shared, int64_t limit, int32_t* total,
                       int32_t* counts, int32_t* offsets, int64_t* stats,
                       hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, hist, NC, T, E,
                     k, n_shared, limit, total, counts, offsets, stats);
  return hipGetLastError();
}

// One block per 64-token chunk. mask[e] has bit i set when the chunk's token
// i chose expert e; a pair's rank among the chunk's earlier tokens for the
// same expert is the popcount of the mask below its bit, so
// slot = base[chunk's first histogram row, e] + rank counts every earlier
// token in the prompt (the scanned row holds the counts of all tokens before
// it; a chunk spans rows_per_chunk rows).
__global__ __launch_bounds__(256) void permute_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w,
    const int32_t* __restrict__ base, int rows_per_chunk,
    const int32_t* __restrict__ offsets,
    int T, int E, int k, int n_shared, int64_t limit,
    int32_t* __restrict__ slot, int32_t* __restrict__ tok2pair,
    int32_t* __restrict__ pair_token, float* __restrict__ pair_w) {
  extern __shared__ unsigned long long mask[];   // E
  const int chunk = blockIdx.x;
  const int t0 = chunk * kChunk;
  const int nt = min(kChunk, T - t0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
  __syncthreads();
  const int np = nt * k;
  const size_t g0 = (size_t)t0 * k;
  for (int p = threadIdx.x; p < np; p += blockDim.x) {
    const int tl = p / k;
    const int e = ids[g0 + p];
    atomicOr(&mask[e], 1ull << tl);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < np; p += blockDim.x) {
    const int tl = p / k;
    const size_t gp = g0 + p;
    const int e = ids[gp];
    const unsigned long long below = (1ull << tl) - 1ull;
    const int rank = __popcll(mask[e] & below);
    const int sl = base[(size_t)chunk * rows_per_chunk * (E + 1) + e] + rank;
    slot[gp] = sl;
    const bool keep = limit < 0 || (int64_t)sl < limit;
    const int pos = keep ? offsets[e] + sl : -1;
    tok2pair[gp] = pos;
    if (keep) {
      pair_token[pos] = t0 + tl;
      pair_w[pos] = w[gp];
    }
  }
  if (n_shared) {
    const int sbase = offsets[E];
    for (int tl = threadIdx.x; tl < nt; tl += blockDim.x) {
      pair_token[sbase + t0 + tl] = t0 + tl;
      pair_w[sbase + t0 + tl] = 1.0f;
    }
  }
}

hipError_t launch_permute(const int32_t* ids, const float* w,
                          const int32_t* base, int rows_per_chunk,
                          const int32_t* offsets, int T, int E, int k,
                          int n_shared, int64_t limit, int32_t* slot,
                          int32_t* tok2pair, int32_t* pair_token,
                          float* pair_w, hipStream_t s) {
  const int NC = (T + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(permute_kernel, dim3(NC), dim3(256),
                     (size_t)E * sizeof(unsigned long long), s, ids, w, base,
                     rows_per_chunk, offsets, T, E, k, n_shared, limit, slot,
                     tok2pair, pair_token, pair_w);
  return hipGetLastError();
}

}  // namespace moe
