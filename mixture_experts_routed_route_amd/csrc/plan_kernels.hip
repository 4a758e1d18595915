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

// One step of a wave-wide max of 64-bit values through DPP (a lane reads
// another lane's registers in the VALU, no LDS round trip): lanes of the
// rows in ROWMASK take the larger of their value and the one CTRL routes to
// them; the others keep theirs.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWMASK, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWMASK, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

// Max of v over the 64 lanes, returned in every lane (a scalar): lane pairs
// xor 1 and xor 2 within quads, then the half-row and row mirrors (each lane
// then holds its 16-lane row's max), then row 0 into row 1 and row 2 into
// row 3 (row_bcast:15), and row 1 into rows 2 and 3 (row_bcast:31): lane 63
// holds the max of all four rows.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_max_step<0x4E, 0xF>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_max_step<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);   // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
  v = dpp_max_step<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Number of lanes whose predicate holds, over the wave.
__device__ __forceinline__ int wave_count(bool pred) {
  return __popcll(__ballot(pred));
}

// One wavefront per token; PER = ceil(E / 64) logits per lane (expert
// lane + 64 p). Selection: k rounds of a wave-wide arg-max over the order
// keys, ties to the lower expert index, so round j yields the expert of
// rank j (its position in the token's top-k list) and round 0 the largest
// logit l_0. Lane j % 64 keeps round j's expert and key in slot j / 64.
// Weights: exp(l_j - l_0) / sum_i exp(l_i - l_0) in double (the sum in rank
// order), rounded to f32.
// The TPW tokens from tbase of one wave: their top-k ids and weights into
// ids / w, one count per chosen expert into sh_hist (LDS); returns the
// wave's NaN logits (the same value in every lane).
template <int PER, int TPW>
__device__ __forceinline__ int route_wave_tokens(
    const float* __restrict__ logits, int T, int E, int k, int tbase,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* sh_hist) {
  const int lane = threadIdx.x & 63;
  int nan_count = 0;
  // every token's logits are loaded before the first is ranked: one memory
  // round trip per wave, not one per token
  float lg[TPW][PER];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = lane + 64 * p;
      lg[i][p] = (tbase + i < T && e < E) ? logits[(size_t)(tbase + i) * E + e] : 0.f;
    }
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = tbase + i;
    if (t >= T) break;   // wave-uniform
    uint32_t key[PER];
    bool valid[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = lane + 64 * p;
      valid[p] = e < E;
      const float l = lg[i][p];
      key[p] = order_key(l);
      nan_count += (valid[p] && l != l) ? 1 : 0;
    }
    bool sel[PER];
    uint32_t my_key[PER];
    int my_e[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) { sel[p] = false; my_key[p] = 0u; my_e[p] = 0; }
    uint32_t top = 0u;
    for (int jr = 0; jr < k; ++jr) {
      // candidate: key << 32 | (2^32 - 1 - e); 0 means none
      uint64_t best = 0ull;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const uint64_t v = ((uint64_t)key[p] << 32) |
                           (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * p));
        if (valid[p] && !sel[p] && v > best) best = v;
      }
      best = wave_max_u64(best);
      const int ew = (int)(0xFFFFFFFFu - (uint32_t)best);   // wave-uniform
      const uint32_t kw = (uint32_t)(best >> 32);
      if (jr == 0) top = kw;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        if (lane + 64 * p == ew) sel[p] = true;
        if ((jr >> 6) == p && lane == (jr & 63)) { my_key[p] = kw; my_e[p] = ew; }
      }
    }
    const double l0 = (double)key_value(top);
    double ex[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p)
      ex[p] = (64 * p + lane < k) ? exp((double)key_value(my_key[p]) - l0) : 0.0;
    // the sum in rank order, the same in every lane
    double sum = 0.0;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const uint64_t bits = (uint64_t)__double_as_longlong(ex[p]);
      for (int l = 0; l < 64 && 64 * p + l < k; ++l) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), l);
        sum += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
      }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int jr = 64 * p + lane;
      if (jr < k) {
        ids[(size_t)t * k + jr] = my_e[p];
        w[(size_t)t * k + jr] = (float)(ex[p] / sum);
        atomicAdd(&sh_hist[my_e[p]], 1);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nan_count += __shfl_xor(nan_count, off);
  return nan_count;
}

// Max of v over the 16 lanes of each DPP row (lanes 16 g .. 16 g + 15),
// in every lane of the row.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_max_step<0x4E, 0xF>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_max_step<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);   // row_mirror
  return v;
}

// The same selection and weights for four tokens at once: token tbase + g
// takes the 16 lanes of row g (lanes 16 g .. 16 g + 15), P16 = ceil(E / 16)
// logits per lane (expert lane % 16 + 16 p), so one round of the arg-max is
// a 16-lane reduction inside a DPP row and the four tokens' rounds share
// every instruction. Needs E <= 16 P16 <= 256 and k <= 16 (lane 16 g + j
// keeps round j). Same results as route_wave_tokens.
template <int P16>
__device__ __forceinline__ int route_group_tokens(
    const float* __restrict__ logits, int T, int E, int k, int tbase,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* sh_hist) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int t = tbase + (lane >> 4);
  const bool tv = t < T;   // uniform in the row
  uint32_t key[P16];
  bool valid[P16], sel[P16];
  int nan_count = 0;
#pragma unroll
  for (int p = 0; p < P16; ++p) {
    const int e = l16 + 16 * p;
    valid[p] = tv && e < E;
    const float l = valid[p] ? logits[(size_t)t * E + e] : 0.f;
    key[p] = order_key(l);
    sel[p] = false;
    nan_count += wave_count(valid[p] && l != l);
  }
  uint32_t my_key = 0u, top = 0u;
  int my_e = 0;
  for (int jr = 0; jr < k; ++jr) {
    uint64_t best = 0ull;
#pragma unroll
    for (int p = 0; p < P16; ++p) {
      const uint64_t v = ((uint64_t)key[p] << 32) |
                         (uint64_t)(0xFFFFFFFFu - (uint32_t)(l16 + 16 * p));
      if (valid[p] && !sel[p] && v > best) best = v;
    }
    best = row_max_u64(best);
    const int ew = (int)(0xFFFFFFFFu - (uint32_t)best);   // uniform in the row
    const uint32_t kw = (uint32_t)(best >> 32);
    if (jr == 0) top = kw;
#pragma unroll
    for (int p = 0; p < P16; ++p)
      if (l16 + 16 * p == ew) sel[p] = true;
    if (l16 == jr) { my_key = kw; my_e = ew; }
  }
  const double l0 = (double)key_value(top);
  const double ex = l16 < k ? exp((double)key_value(my_key) - l0) : 0.0;
  // the sum in rank order, the same in every lane of the row
  double sum = 0.0;
  const int row0 = lane & 48;
  for (int j = 0; j < k; ++j) sum += __shfl(ex, row0 + j);
  if (tv && l16 < k) {
    ids[(size_t)t * k + l16] = my_e;
    w[(size_t)t * k + l16] = (float)(ex / sum);
    atomicAdd(&sh_hist[my_e], 1);
  }
  return nan_count;
}

// Histogram rows of 64 tokens from the grouped router: 16 waves x 4 tokens.
template <int P16>
__global__ __launch_bounds__(1024) void route_hist_group_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ hist) {
  extern __shared__ int32_t sh_hist[];   // E + 1
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) sh_hist[e] = 0;
  __syncthreads();
  const int nan_count = route_group_tokens<P16>(logits, T, E, k, chunk * 64 + wave * 4,
                                                ids, w, sh_hist);
  if (lane == 0 && nan_count) atomicAdd(&sh_hist[E], nan_count);
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x)
    hist[(size_t)chunk * (E + 1) + e] = sh_hist[e];
}

// Block = 16 waves x TPW tokens; the block's histogram row
// hist[block, 0..E-1] counts its tokens' choices per expert, and
// hist[block, E] their NaN logits.
template <int PER, int TPW>
__global__ __launch_bounds__(1024) void route_hist_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ hist) {
  extern __shared__ int32_t sh_hist[];   // E + 1
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) sh_hist[e] = 0;
  __syncthreads();
  const int tbase = chunk * 16 * TPW + wave * TPW;
  const int nan_count = route_wave_tokens<PER, TPW>(logits, T, E, k, tbase, ids, w, sh_hist);
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
  if (tpw == 4 && route_grouped(E, k)) {
    const int p16 = (E + 15) / 16;
#define MOE_ROUTE_G(P)                                                              \
    hipLaunchKernelGGL((route_hist_group_kernel<P>), dim3(NR), dim3(1024), sh, s,   \
                       logits, T, E, k, ids, w, hist)
    if (p16 <= 1) MOE_ROUTE_G(1);
    else if (p16 <= 2) MOE_ROUTE_G(2);
    else if (p16 <= 4) MOE_ROUTE_G(4);
    else if (p16 <= 8) MOE_ROUTE_G(8);
    else MOE_ROUTE_G(16);
#undef MOE_ROUTE_G
    return hipGetLastError();
  }
  const int per = (E + 63) / 64;
#define MOE_ROUTE(P, TPW)                                                          \
  hipLaunchKernelGGL((route_hist_kernel<P, TPW>), dim3(NR), dim3(1024), sh, s,     \
                     logits, T, E, k, ids, w, hist)
  if (tpw == 4 && per > 4) return hipErrorInvalidValue;
  if (per <= 1) { if (tpw == 1) MOE_ROUTE(1, 1); else MOE_ROUTE(1, 4); }
  else if (per <= 2) { if (tpw == 1) MOE_ROUTE(2, 1); else MOE_ROUTE(2, 4); }
  else if (per <= 4) { if (tpw == 1) MOE_ROUTE(4, 1); else MOE_ROUTE(4, 4); }
  else if (per <= 8) MOE_ROUTE(8, 1);
  else MOE_ROUTE(16, 1);
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

// The whole plan of a prompt of at most 64 tokens (one permute chunk) in
// one block: route into LDS, then the counts, offsets and statistics of the
// scan kernel for a single histogram row (every base is zero), then the
// permute of that chunk. Same arithmetic and order as the three kernels;
// one launch instead of three for decode-shaped and short prompts.
template <int PER>
__global__ __launch_bounds__(1024) void plan_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int n_shared,
    int64_t limit, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ total, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int64_t* __restrict__ stats,
    int32_t* __restrict__ slot, int32_t* __restrict__ tok2pair,
    int32_t* __restrict__ pair_token, float* __restrict__ pair_w,
    DecodeGroups dg) {
  __shared__ int32_t sh_hist[kMaxExperts + 1];
  __shared__ int32_t sh_grp[kMaxExperts + 2];   // decode: expert of group g
  __shared__ int32_t sh_pt[kPlanSmallPairs + kDecodeT];   // decode: pair tokens
  __shared__ int32_t sh_off[kMaxExperts + 2];
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int32_t sh_ids[kPlanSmallPairs];
  __shared__ float sh_w[kPlanSmallPairs];
  __shared__ int sh_waves[16];
  __shared__ int red[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e <= E; e += blockDim.x) sh_hist[e] = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
  if (threadIdx.x < 4) red[threadIdx.x] = 0;
  __syncthreads();
  // route: PER > 0: a wave ranks one token at a time on all 64 lanes, one
  // token per wave up to 16 tokens, else 4 per wave; PER < 0 (more than 16
  // tokens): four tokens per wave at once, 16 lanes and -PER logits a lane
  int nan_count;
  if constexpr (PER > 0) {
    if (T <= 16)
      nan_count = route_wave_tokens<PER, 1>(logits, T, E, k, wave, sh_ids, sh_w, sh_hist);
    else
      nan_count = route_wave_tokens<PER, 4>(logits, T, E, k, wave * 4, sh_ids, sh_w, sh_hist);
  } else {
    nan_count = route_group_tokens<-PER>(logits, T, E, k, wave * 4, sh_ids, sh_w, sh_hist);
  }
  if (lane == 0 && nan_count) atomicAdd(&sh_hist[E], nan_count);
  __syncthreads();
  const int np = T * k;
  for (int p = threadIdx.x; p < np; p += blockDim.x) {
    ids[p] = sh_ids[p];
    w[p] = sh_w[p];
  }
  // counts, offsets and statistics
  int kept_local = 0, touched_local = 0, max_local = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int tot = sh_hist[e];
    total[e] = tot;
    const int c = (limit < 0 || (int64_t)tot < limit) ? tot : (int)limit;
    counts[e] = c;
    kept_local += c;
    touched_local += c > 0 ? 1 : 0;
    max_local = max(max_local, c);
  }
  if (kept_local) atomicAdd(&red[0], kept_local);
  if (touched_local) atomicAdd(&red[1], touched_local);
  if (max_local) atomicMax(&red[2], max_local);
  if (n_shared && threadIdx.x == 0) counts[E] = T;
  const int n = E + n_shared;
  int carry = 0, gcarry = 0;
  for (int b = 0; b < n; b += blockDim.x) {
    const int e = b + threadIdx.x;
    int c = 0;
    if (e < E) {
      const int tot = sh_hist[e];
      c = (limit < 0 || (int64_t)tot < limit) ? tot : (int)limit;
    } else if (e < n) {
      c = T;
    }
    int blk_total = 0;
    const int pre = block_scan_excl(c, &blk_total, sh_waves);
    if (e < n) {
      offsets[e] = carry + pre;
      sh_off[e] = carry + pre;
    }
    carry += blk_total;
    if (dg.list) {
      // decode groups: one per touched expert, numbered in expert order
      int g_total = 0;
      const int gpre = block_scan_excl(c > 0 ? 1 : 0, &g_total, sh_waves);
      if (e < n) {
        const int g = gcarry + gpre;
        if (c > 0) {
          sh_grp[g] = e;
          dg.list[4 * g] = e;
          dg.list[4 * g + 1] = 0;
          dg.list[4 * g + 2] = c;
          dg.list[4 * g + 3] = carry - blk_total + pre;
        }
      }
      gcarry += g_total;
    }
  }
  const int dg_groups = gcarry;
  if (threadIdx.x == 0) {
    offsets[n] = carry;
    sh_off[n] = carry;
    if (dg.list) dg.meta[kMetaSk1] = gcarry;
  }
  if (dg.list)
    for (int i = threadIdx.x; i < kMetaCount; i += blockDim.x)
      if (i != kMetaSk1) dg.meta[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    stats[0] = (int64_t)T * k - red[0];   // dropped
    stats[1] = red[0];                    // kept
    stats[2] = sh_hist[E];                // NaN logits
    stats[3] = red[1];                    // touched experts
    stats[4] = red[2];                    // max rows
    stats[5] = 0;
    stats[6] = 0;
    stats[7] = 0;
  }
  // permute of the single chunk: slot = rank among earlier tokens
  for (int p = threadIdx.x; p < np; p += blockDim.x)
    atomicOr(&mask[sh_ids[p]], 1ull << (p / k));
  __syncthreads();
  for (int p = threadIdx.x; p < np; p += blockDim.x) {
    const int tl = p / k;
    const int e = sh_ids[p];
    const unsigned long long below = (1ull << tl) - 1ull;
    const int sl = __popcll(mask[e] & below);
    slot[p] = sl;
    const bool keep = limit < 0 || (int64_t)sl < limit;
    const int pos = keep ? sh_off[e] + sl : -1;
    tok2pair[p] = pos;
    if (keep) {
      pair_token[pos] = tl;
      pair_w[pos] = sh_w[p];
      if (dg.list) sh_pt[pos] = tl;
    }
  }
  if (n_shared) {
    const int sbase = sh_off[E];
    for (int tl = threadIdx.x; tl < T; tl += blockDim.x) {
      pair_token[sbase + tl] = tl;
      pair_w[sbase + tl] = 1.0f;
      if (dg.list) sh_pt[sbase + tl] = tl;
    }
  }
  if (dg.list) {
    // each group's x rows, kStreamTokRows entries, rows past the group's
    // last clamped to it; 64 threads a group, contiguous stores
    __syncthreads();
    const int ng = dg_groups;
    for (int i = threadIdx.x; i < ng * kStreamTokRows; i += blockDim.x) {
      const int g = i / kStreamTokRows, r = i - g * kStreamTokRows;
      const int e = sh_grp[g];
      const int c = sh_off[e + 1] - sh_off[e];
      dg.tok[i] = sh_pt[sh_off[e] + min(r, c - 1)];
    }
  }
}

hipError_t launch_plan_small(const float* logits, int T, int E, int k,
                             int n_shared, int64_t limit, int32_t* ids,
                             float* w, int32_t* total, int32_t* counts,
                             int32_t* offsets, int64_t* stats, int32_t* slot,
                             int32_t* tok2pair, int32_t* pair_token,
                             float* pair_w, const DecodeGroups* dgp,
                             hipStream_t s) {
  if (T < 1 || T > kChunk || (int64_t)T * k > kPlanSmallPairs || E > kPlanSmallE)
    return hipErrorInvalidValue;
  DecodeGroups dg{nullptr, nullptr, nullptr};
  if (dgp) {
    if (T > kDecodeT) return hipErrorInvalidValue;
    dg = *dgp;
  }
  const int per = (E + 63) / 64;
#define MOE_PLAN_SMALL(P)                                                        \
  hipLaunchKernelGGL((plan_small_kernel<P>), dim3(1), dim3(1024), 0, s, logits, T, \
                     E, k, n_shared, limit, ids, w, total, counts, offsets,     \
                     stats, slot, tok2pair, pair_token, pair_w, dg)
  if (T > 16 && route_grouped(E, k)) {
    const int p16 = (E + 15) / 16;
    if (p16 <= 1) MOE_PLAN_SMALL(-1);
    else if (p16 <= 2) MOE_PLAN_SMALL(-2);
    else if (p16 <= 4) MOE_PLAN_SMALL(-4);
    else if (p16 <= 8) MOE_PLAN_SMALL(-8);
    else MOE_PLAN_SMALL(-16);
  } else if (per <= 1) MOE_PLAN_SMALL(1);
  else if (per <= 2) MOE_PLAN_SMALL(2);
  else MOE_PLAN_SMALL(4);
#undef MOE_PLAN_SMALL
  return hipGetLastError();
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
