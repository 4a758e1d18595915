// Forward kernels of the routed MoE layer on gfx950.
//
// Per expert: gathered rows of x times W_gate and W_up, clamped SwiGLU, times
// W_down; the combine scales each pair's output by its routing weight
// (mini-AGI PR #4, minagi/pool.py, `experts()`; the clamp from Strata PR
// #4366, "Approach").
// Three routes, chosen per expert from its row count on the device:
//   full    LDS-staged MFMA tile (v_mfma_f32_32x32x16) for experts with many
//           rows; the fused SwiGLU runs in the gate/up tile's epilogue;
//   fat     4-bit experts with many rows: weights dequantised once to fp16
//           (Strata PR #4366: decode once instead of once per 64-row chunk),
//           then the full tile;
//   split-K a K-parallel tile for experts holding few pairs (TensorFold PR
//           #1607): weights stream once from HBM straight into
//           v_mfma_f32_16x16x32 operands, four waves split K and reduce in LDS
//           in a fixed order; 4-bit weights are dequantised in registers.
// The combine gathers each token's pair rows, weighted, in fixed order, with
// no atomics.
#include <algorithm>
#include <type_traits>

#include "device_common.h"

namespace moe {

// ---- element types ----------------------------------------------------------

struct F16T {
  using S = _Float16;
  using V8 = half8;
  static constexpr int kBytes = 2;
};
struct BF16T {
  using S = __bf16;
  using V8 = bf16x8;
  static constexpr int kBytes = 2;
};
struct F32T {
  using S = float;
  static constexpr int kBytes = 4;
};

// ---- classify -------------------------------------------------------------

__device__ __forceinline__ int warp_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive scan over the block (thread order) with the block total.
__device__ __forceinline__ int block_excl(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = warp_incl_scan(v);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
    if (i < wave) pre += sh[i];
    tot += sh[i];
  }
  __syncthreads();
  *total = tot;
  return pre + incl - v;
}

// One block of 1024 threads. Route per expert from its kept rows n:
//   mode 0 (f32): split-K; mode 1 (bf16/f16): split-K iff n <= S, else full;
//   mode 2 (q4): fat iff fat_rows > 0 and n >= fat_rows, else split-K.
// Mode 1 with full_fill > 0: if the full experts' tiles times the column
// blocks per tile would not occupy full_fill work-groups (one round of the
// persistent full tile), the full tile would leave most compute units idle
// while each busy one walks the whole K; the split-K tile spreads the same
// weights over every unit instead, so full experts of at most kFullBM rows
// move to split-K.
// Full/fat experts are ordered largest first (ties: lower index) and cut into
// kFullBM-row tiles. Split-K experts are cut into groups of <= 64 rows;
// groups of at most 16 rows go to the first list, the others to the second;
// for the stream tile each group's x rows go to a table beside its list.
__global__ __launch_bounds__(1024) void classify_kernel(ClassifyArgs a) {
  constexpr int kPadE = (kMaxExperts + 1 + 3) / 4 * 4;
  __shared__ int cnt[kPadE];
  __shared__ int rte[kPadE];
  __shared__ __attribute__((aligned(16))) int fkey[kPadE];   // rows if full, else -1
  __shared__ int order[kPadE];
  __shared__ int sh[16];
  __shared__ int nfull_sh;
  __shared__ int ntiles_sh;
  const int n = a.n_exp;
  const int n4 = (n + 3) / 4 * 4;
  if (threadIdx.x == 0) { nfull_sh = 0; ntiles_sh = 0; }
  for (int e = threadIdx.x; e < n4; e += blockDim.x) {
    const int c = e < n ? a.counts[e] : 0;
    int r = kRouteNone;
    if (c > 0) {
      if (a.mode == 0) r = kRouteSplitK;
      else if (a.mode == 1) r = ((double)c <= a.S) ? kRouteSplitK : kRouteFull;
      else r = (a.fat_rows > 0 && c >= a.fat_rows) ? kRouteFat : kRouteSplitK;
    }
    cnt[e] = c;
    rte[e] = r;
    fkey[e] = r >= kRouteFull ? c : -1;
  }
  __syncthreads();
  if (a.mode == 1 && a.full_fill > 0) {
    int t = 0;
    for (int e = threadIdx.x; e < n; e += blockDim.x)
      if (rte[e] == kRouteFull) t += (cnt[e] + kFullBM - 1) / kFullBM;
    if (t) atomicAdd(&ntiles_sh, t);
    __syncthreads();
    if ((int64_t)ntiles_sh * a.full_nnb < (int64_t)a.full_fill) {
      for (int e = threadIdx.x; e < n; e += blockDim.x)
        if (rte[e] == kRouteFull && cnt[e] <= kFullBM) {
          rte[e] = kRouteSplitK;
          fkey[e] = -1;
        }
    }
    __syncthreads();
  }
  // rank among full/fat experts: more rows first, then the lower index
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    if (rte[e] < kRouteFull) continue;
    int rank = 0;
    const int c = cnt[e];
    for (int f = 0; f < n4; f += 4) {
      const int4 v = *reinterpret_cast<const int4*>(&fkey[f]);
      rank += (v.x > c || (v.x == c && f + 0 < e)) ? 1 : 0;
      rank += (v.y > c || (v.y == c && f + 1 < e)) ? 1 : 0;
      rank += (v.z > c || (v.z == c && f + 2 < e)) ? 1 : 0;
      rank += (v.w > c || (v.w == c && f + 3 < e)) ? 1 : 0;
    }
    order[rank] = e;
    atomicAdd(&nfull_sh, 1);
  }
  __syncthreads();
  const int nfull = nfull_sh;
  // full tiles in largest-first order
  int carry = 0;
  for (int b = 0; b < nfull; b += blockDim.x) {
    const int r = b + threadIdx.x;
    const int e = r < nfull ? order[r] : 0;
    const int nt = r < nfull ? (cnt[e] + kFullBM - 1) / kFullBM : 0;
    int tot = 0;
    const int pre = carry + block_excl(nt, &tot, sh);
    for (int i = 0; i < nt; ++i) {
      a.full_tiles[2 * (pre + i)] = e;
      a.full_tiles[2 * (pre + i) + 1] = i * kFullBM;
    }
    carry += tot;
  }
  const int n_tiles = carry;
  // split-K groups and fat slots in expert order
  int c1 = 0, c4 = 0, cf = 0;
  for (int b = 0; b < n; b += blockDim.x) {
    const int e = b + threadIdx.x;
    int g1 = 0, g4 = 0, fat = 0, c = 0;
    if (e < n) {
      c = cnt[e];
      if (rte[e] == kRouteSplitK) {
        const int ng = (c + kSkRows - 1) / kSkRows;
        const int last = c - (ng - 1) * kSkRows;
        g4 = (ng - 1) + (last > 16 ? 1 : 0);
        g1 = last <= 16 ? 1 : 0;
      }
      fat = rte[e] == kRouteFat ? 1 : 0;
    }
    int t1 = 0, t4 = 0, tf = 0;
    const int p1 = c1 + block_excl(g1, &t1, sh);
    const int p4 = c4 + block_excl(g4, &t4, sh);
    const int pf = cf + block_excl(fat, &tf, sh);
    if (e < n) {
      if (rte[e] == kRouteSplitK) {
        const int ng = (c + kSkRows - 1) / kSkRows;
        for (int g = 0; g < ng; ++g) {
          const int row0 = g * kSkRows;
          const int rows = min(kSkRows, c - row0);
          const int pstart = a.offsets[e] + row0;
          const bool one = rows <= 16;
          const int slot = one ? p1 : p4 + g;
          int32_t* dst = (one ? a.sk1 : a.sk4) + 4 * slot;
          dst[0] = e;
          dst[1] = row0;
          dst[2] = rows;
          dst[3] = pstart;
        }
      }
      a.fat_slot[e] = fat ? pf : -1;
      if (fat) a.fat_list[pf] = e;
    }
    c1 += t1;
    c4 += t4;
    cf += tf;
  }
  if (a.sk1_tok || a.sk4_tok) {
    // The groups' x rows for the stream tile, and for the wide 4-bit tile
    // (sk4 only), a group's rows clamped to its last, one row per thread
    // over all groups: one round trip for the group entries written above,
    // one for the pair list.
    __syncthreads();   // the group entries are visible to the whole block
    const int r1 = a.sk1_tok ? c1 * 16 : 0;
    const int r4 = a.sk4_tok ? c4 * kStreamTokRows : 0;
    for (int i = threadIdx.x; i < r1 + r4; i += blockDim.x) {
      const bool one = i < r1;
      const int j = one ? i : i - r1;
      const int slot = one ? j >> 4 : j / kStreamTokRows;
      const int t = one ? j & 15 : j - slot * kStreamTokRows;
      const int32_t* g = (one ? a.sk1 : a.sk4) + 4 * slot;
      const int rows = g[2], pstart = g[3];
      (one ? a.sk1_tok : a.sk4_tok)[(size_t)kStreamTokRows * slot + t] =
          a.pair_token[pstart + min(t, rows - 1)];
    }
  }
  if (threadIdx.x == 0) {
    a.meta[kMetaFullTiles] = n_tiles;
    a.meta[kMetaSk1] = c1;
    a.meta[kMetaSk4] = c4;
    a.meta[kMetaFat] = cf;
  }
  for (int i = kMetaQueueGateUp + threadIdx.x; i < kMetaCount; i += blockDim.x)
    a.meta[i] = 0;
}

hipError_t launch_classify(const ClassifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(classify_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

// ---- dequantise once --------------------------------------------------------

// Fat experts: slot s of a staging buffer holds expert fat_list[s]'s
// [rows, K] matrix as fp16, k-block-major: [K / 32][rows][32], so that the
// full tile reads one stage's rows as a single contiguous slab. blockIdx.y
// picks one of up to three matrices (W_gate, W_up, W_down). A block takes
// tiles of 64 rows x KB blocks of 32 values (KB = 8 when K is a multiple of
// 256, so every row's nibbles come as one whole 128-byte line; else 4): it
// decodes into LDS in the output order and writes the tile's KB 4 KB runs
// 1 KB per store instruction.
struct DequantSet {
  const uint8_t* q[3];
  const char* sc[3];      // scales (FMT 0) or (scale, bias) words
  _Float16* out[3];
  int rows[3], K[3];
};

template <int KB, int FMT>
__device__ __forceinline__ void dequant_fat_tiles(const DequantSet& d, int m,
                                                  const int32_t* fat_list,
                                                  int nfat, char* tile) {
  constexpr int TPR = 4;                          // threads per row
  constexpr int BPT = KB / TPR;                   // 32-value blocks per thread
  const uint8_t* __restrict__ q = d.q[m];
  const char* __restrict__ sc = d.sc[m];
  _Float16* __restrict__ out = d.out[m];
  const int rows = d.rows[m], K = d.K[m];
  const int kbs = K / 32;                         // 32-value blocks per row
  const int ngr = K / Q4F<FMT>::kGroup;           // parameters per row
  const int rt = rows / 64, ktn = kbs / KB;       // tiles per slot: rt x ktn
  const int per_slot = rt * ktn;
  const int total = nfat * per_slot;
  const int tid = threadIdx.x;
  const int r = tid >> 2, qq = tid & 3;           // decode: row, quarter of the tile's blocks
  // a tile's nibbles and parameters, loaded one tile ahead: the next tile's
  // loads are in flight while this one is decoded and stored
  uint4 qa[BPT], qn[BPT];
  uint32_t pa[BPT], pn[BPT];
  auto load = [&](int w, uint4* qv, uint32_t* pv) {
    const int slot = w / per_slot;
    const int rem = w - slot * per_slot;
    const int kq = rem / rt;
    const int kb0 = kq * KB;
    const int row0 = (rem - kq * rt) * 64;
    const size_t er = (size_t)fat_list[slot] * rows + row0 + r;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int kb = kb0 + qq * BPT + b;
      qv[b] = *reinterpret_cast<const uint4*>(q + er * (size_t)(K / 2) + kb * 16);
      if constexpr (FMT == 0)
        pv[b] = *reinterpret_cast<const uint16_t*>(sc + (er * (size_t)kbs + kb) * 2);
      else
        pv[b] = *reinterpret_cast<const uint32_t*>(
            sc + (er * (size_t)ngr + kb * 32 / Q4F<FMT>::kGroup) * 4);
    }
  };
  if (blockIdx.x < total) load(blockIdx.x, qn, pn);
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int slot = w / per_slot;
    const int rem = w - slot * per_slot;
    const int kq = rem / rt;
    const int kb0 = kq * KB;
    const int row0 = (rem - kq * rt) * 64;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      qa[b] = qn[b];
      pa[b] = pn[b];
    }
    if (w + (int)gridDim.x < total) load(w + gridDim.x, qn, pn);
    __syncthreads();   // the previous tile's stores have read the LDS tile
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      half8 ha[4];
      dequant32_f<FMT>(qa[b], pa[b], ha);
      char* ta = tile + ((qq * BPT + b) * 64 + r) * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(ta + ((i ^ qq) * 16)) = __builtin_bit_cast(uint4, ha[i]);
    }
    __syncthreads();
    // KB x 256 16-byte pieces; block kb's 64 rows are 4 KB contiguous. In
    // LDS, 16-byte piece c of a row of block kb sits at c ^ (kb / BPT): the
    // four threads of a row decode blocks BPT apart, and their stores of
    // the same piece would otherwise hit one bank group; the reads take
    // whole rows.
    char* os = reinterpret_cast<char*>(out + (size_t)slot * rows * K);
#pragma unroll
    for (int it = 0; it < KB; ++it) {
      const int rr = tid >> 2, pc = tid & 3;
      const uint4 v = *reinterpret_cast<const uint4*>(
          tile + ((it * 64 + rr) * 4 + (pc ^ ((it / BPT) & 3))) * 16);
      *reinterpret_cast<uint4*>(os + ((size_t)(kb0 + it) * rows + row0) * 64 + tid * 16) = v;
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void dequant_fat_kernel(
    DequantSet d, const int32_t* __restrict__ fat_list,
    const int32_t* __restrict__ meta) {
  __shared__ __attribute__((aligned(16))) char tile[8 * 64 * 64];   // [kb][row][32 fp16]
  const int m = blockIdx.y;
  const int nfat = meta[kMetaFat];
  if (d.K[m] % 256 == 0)
    dequant_fat_tiles<8, FMT>(d, m, fat_list, nfat, tile);
  else
    dequant_fat_tiles<4, FMT>(d, m, fat_list, nfat, tile);
}

// One unit = 8 consecutive values of a row: 4 bytes of nibbles in, 16 bytes
// of fp16 out, so a wave's loads cover 256 contiguous bytes and its stores
// 1 KB. The four lanes of a 32-value block share its scale.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_rows_kernel(
    const uint8_t* __restrict__ q, const char* __restrict__ sc,
    _Float16* __restrict__ out, int64_t rows, int K) {
  const int upr = K / 8;
  const int ngr = K / Q4F<FMT>::kGroup;
  const size_t total = (size_t)rows * upr;
  for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < total;
       u += (size_t)gridDim.x * blockDim.x) {
    const size_t row = u / upr;
    const int c8 = (int)(u - row * upr);
    const uint32_t word = reinterpret_cast<const uint32_t*>(q + row * (size_t)(K / 2))[c8];
    if constexpr (FMT == 0) {
      const uint16_t sb = reinterpret_cast<const uint16_t*>(sc)[row * (size_t)(K / 32) + (c8 >> 2)];
      reinterpret_cast<uint4*>(out + row * (size_t)K)[c8] =
          __builtin_bit_cast(uint4, dequant_word(word, __builtin_bit_cast(_Float16, sb)));
    } else {
      const uint32_t p = reinterpret_cast<const uint32_t*>(sc)[
          row * (size_t)ngr + c8 * 8 / Q4F<FMT>::kGroup];
      reinterpret_cast<uint4*>(out + row * (size_t)K)[c8] =
          __builtin_bit_cast(uint4, dequant_word_affine(word, p));
    }
  }
}

hipError_t launch_dequant_fat(const void* const q[3], const void* const sc[3],
                              void* const out[3], const int rows[3],
                              const int K[3], int n, const int32_t* fat_list,
                              const int32_t* meta, int grid, int fmt,
                              hipStream_t s) {
  if (n < 1 || n > 3) return hipErrorInvalidValue;
  DequantSet d{};
  for (int i = 0; i < n; ++i) {
    d.q[i] = (const uint8_t*)q[i];
    d.sc[i] = (const char*)sc[i];
    d.out[i] = (_Float16*)out[i];
    d.rows[i] = rows[i];
    d.K[i] = K[i];
  }
  if (fmt == 0)
    hipLaunchKernelGGL(dequant_fat_kernel<0>, dim3(grid, n), dim3(256), 0, s, d, fat_list, meta);
  else if (fmt == 1)
    hipLaunchKernelGGL(dequant_fat_kernel<1>, dim3(grid, n), dim3(256), 0, s, d, fat_list, meta);
  else if (fmt == 2)
    hipLaunchKernelGGL(dequant_fat_kernel<2>, dim3(grid, n), dim3(256), 0, s, d, fat_list, meta);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const void* q, const void* sc, void* out,
                               int64_t rows, int K, int fmt, hipStream_t s) {
  const size_t units = (size_t)rows * (K / 8);
  const int grid = (int)std::min<size_t>((units + 255) / 256, 65536);
  if (grid == 0) return hipSuccess;
#define MOE_DQR(F_)                                                              \
  hipLaunchKernelGGL(dequant_rows_kernel<F_>, dim3(grid), dim3(256), 0, s,       \
                     (const uint8_t*)q, (const char*)sc, (_Float16*)out, rows, K)
  if (fmt == 0) MOE_DQR(0);
  else if (fmt == 1) MOE_DQR(1);
  else if (fmt == 2) MOE_DQR(2);
  else return hipErrorInvalidValue;
#undef MOE_DQR
  return hipGetLastError();
}

// ---- split-K tile -----------------------------------------------------------------
//
// Block = 4 waves on one item (split-K group of <= 16 RB rows, 64 output
// columns); wave w takes a contiguous quarter of K. Lane (n = l % 16,
// q = l / 16) streams, per super-step of KSS values of K, a contiguous
// 32 (16-bit) or 16 (f32) values of its weight row and of its A row, and
// MFMA i uses slice i of them, so every MFMA's K values are matched between
// A and B. Gate/up columns: blocks cb = 0..3 are W_gate f0..f0+15, W_up
// f0..f0+15, W_gate f0+16.., W_up f0+16.. for f0 = 32 nb, so g and u of one
// feature land in matching accumulators of one lane.

// 16-bit activations and weights (bf16/f16).
template <class TT, int RB, int MODE, int LO>
__device__ __forceinline__ void splitk_body16(const GemmArgs& a, int item,
                                              int NNB, float* red) {
  using S = typename TT::S;
  using V8 = typename TT::V8;
  constexpr int KSS = 128;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int g = item / NNB;
  const int nb = item - g * NNB;
  const int e = a.list[4 * g];
  const int row0 = a.list[4 * g + 1];
  const int nrows = a.list[4 * g + 2];
  const int off = a.offsets[e];
  const char* ap[RB];
  const char* ap2[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = row0 + min(rb * 16 + n, nrows - 1);
    if (MODE == 0)
      ap[rb] = (const char*)a.A + (size_t)a.pair_token[off + rr] * a.a_ld * 2;
    else
      ap[rb] = (const char*)a.A + (size_t)(off + rr) * a.a_ld * 2;
    ap2[rb] = LO ? (const char*)a.A2 + (size_t)(off + rr) * a.a_ld * 2 : nullptr;
  }
  const char* bp[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int row;
    const void* base;
    if (MODE == 0) {
      row = nb * 32 + (cb >> 1) * 16 + n;
      base = (cb & 1) ? a.B1 : a.B0;
    } else {
      row = nb * 64 + cb * 16 + n;
      base = a.B0;
    }
    bp[cb] = (const char*)base + ((size_t)e * N + row) * (size_t)K * 2;
  }
  floatx4 acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nss = K / KSS;
  const int s0 = wave * nss / 4, s1 = (wave + 1) * nss / 4;
  for (int s = s0; s < s1; ++s) {
    const int k0 = s * KSS + q * 32;
    V8 av[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) av[rb][i] = as_v8<V8>(ldg16(ap[rb] + (size_t)k0 * 2 + i * 16));
    V8 bv[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[cb][i] = as_v8<V8>(ldg16(bp[cb] + (size_t)k0 * 2 + i * 16));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma16(av[rb][i], bv[cb][i], acc[rb][cb]);
    if (LO) {
      // low plane of H: (hi + lo) W accumulated in f32
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) av[rb][i] = as_v8<V8>(ldg16(ap2[rb] + (size_t)k0 * 2 + i * 16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma16(av[rb][i], bv[cb][i], acc[rb][cb]);
    }
  }

  // fixed-order reduction over the four K quarters: ((w0 + w1) + w2) + w3
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* p = red + ((rb * 4 + cb) * 4 + r) * 64 + lane;
            *p = (w == 0) ? acc[rb][cb][r] : *p + acc[rb][cb][r];
          }
    }
    __syncthreads();
  }
  if (wave == 3) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[rb][cb][r] = red[((rb * 4 + cb) * 4 + r) * 64 + lane] + acc[rb][cb][r];
    // 16x16 accumulator element r of lane l is row 4 (l / 16) + r, column l % 16
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * 16 + q * 4 + r;
        if (row >= nrows) continue;
        const size_t prow = (size_t)(off + row0 + row);
        if (MODE == 0) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const int f = nb * 32 + pr * 16 + n;
            const float h = swiglu(acc[rb][2 * pr][r], acc[rb][2 * pr + 1][r], a.clamp);
            const S hv = (S)h;
            reinterpret_cast<S*>(a.out)[prow * a.out_ld + f] = hv;
            if (a.out2) reinterpret_cast<S*>(a.out2)[prow * a.out_ld + f] = (S)(h - (float)hv);
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int d = nb * 64 + cb * 16 + n;
            store_y1<typename YPairOf<S>::T>(a.out, prow * a.out_ld + d, acc[rb][cb][r]);
          }
        }
      }
  }
  __syncthreads();
}

// fp16 activations, 4-bit weights. As splitk_body16, but a lane reads 32
// bytes of nibbles per weight row and super-step (256 K values), so the four
// lanes of a row take one whole 128-byte line at a time: with 16-byte pieces
// and 128-value super-steps, the two halves of a line came in different
// super-steps, and rows of power-of-two strides lost the line from L2 in
// between often enough to read most lines twice. A K not a multiple of 256
// ends with one 128-value step.
template <int RB, int KH>
struct RawQ4 {
  uint4 av[RB][4 * KH];   // A values k0 .. k0 + 32 KH of the lane's rows
  uint4 w[4][KH];         // 32 KH nibbles of each column block's row
  Q4P p[4];               // their block parameters
};

template <int RB, int MODE, int FMT>
__device__ __forceinline__ void splitk_body_q4(const GemmArgs& a, int item,
                                               int NNB, float* red) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int K = a.K;
  const int N = a.N;
  const int g = item / NNB;
  const int nb = item - g * NNB;
  const int e = a.list[4 * g];
  const int row0 = a.list[4 * g + 1];
  const int nrows = a.list[4 * g + 2];
  const int off = a.offsets[e];
  const char* ap[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = row0 + min(rb * 16 + n, nrows - 1);
    const int arow = MODE == 0 ? a.pair_token[off + rr] : off + rr;
    ap[rb] = (const char*)a.A + (size_t)arow * a.a_ld * 2;
  }
  const uint8_t* bp[4];
  const char* bsp[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int row;
    const void* base;
    const void* sbase;
    if (MODE == 0) {
      row = nb * 32 + (cb >> 1) * 16 + n;
      base = (cb & 1) ? a.B1 : a.B0;
      sbase = (cb & 1) ? a.B1s : a.B0s;
    } else {
      row = nb * 64 + cb * 16 + n;
      base = a.B0;
      sbase = a.B0s;
    }
    const size_t wrow = (size_t)e * N + row;
    bp[cb] = (const uint8_t*)base + wrow * (size_t)(K / 2);
    bsp[cb] = (const char*)sbase +
              wrow * (size_t)(K / Q4F<FMT>::kGroup) * Q4F<FMT>::kPB;
  }
  floatx4 acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one super-step of 128 KH values of K from kbase; lane q takes the
  // 32 KH values from kbase + 32 KH q
  auto step = [&](auto kh, int kbase) {
    constexpr int KH = decltype(kh)::value;
    RawQ4<RB, KH> r;
    const int k0 = kbase + q * 32 * KH;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4 * KH; ++i) r.av[rb][i] = ldg16(ap[rb] + (size_t)k0 * 2 + i * 16);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int h = 0; h < KH; ++h) r.w[cb][h] = ldg16(bp[cb] + k0 / 2 + h * 16);
      r.p[cb] = load_q4p<FMT, KH>(bsp[cb], k0);
    }
    // every load of the step is issued before the first use: left to
    // itself, the scheduler sinks loads into the decode to save registers
    // and then waits on each of them in turn
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int h = 0; h < KH; ++h) {
        half8 hv[4];
        dequant32_f<FMT>(r.w[cb][h], q4p_block<FMT>(r.p[cb], h), hv);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][cb] = mfma16(as_v8<half8>(r.av[rb][4 * h + i]), hv[i], acc[rb][cb]);
      }
  };
  const int nss = K / 256;
  const int s0 = wave * nss / 4, s1 = (wave + 1) * nss / 4;
  for (int s = s0; s < s1; ++s) step(std::integral_constant<int, 2>{}, s * 256);
  if ((K & 255) && wave == 3) step(std::integral_constant<int, 1>{}, nss * 256);

  // fixed-order reduction over the four K quarters: ((w0 + w1) + w2) + w3
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* p = red + ((rb * 4 + cb) * 4 + r) * 64 + lane;
            *p = (w == 0) ? acc[rb][cb][r] : *p + acc[rb][cb][r];
          }
    }
    __syncthreads();
  }
  if (wave == 3) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[rb][cb][r] = red[((rb * 4 + cb) * 4 + r) * 64 + lane] + acc[rb][cb][r];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * 16 + q * 4 + r;
        if (row >= nrows) continue;
        const size_t prow = (size_t)(off + row0 + row);
        if (MODE == 0) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const int f = nb * 32 + pr * 16 + n;
            const float h = swiglu(acc[rb][2 * pr][r], acc[rb][2 * pr + 1][r], a.clamp);
            reinterpret_cast<_Float16*>(a.out)[prow * a.out_ld + f] = (_Float16)h;
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int d = nb * 64 + cb * 16 + n;
            store_y1<_Float16>(a.out, prow * a.out_ld + d, acc[rb][cb][r]);
          }
        }
      }
  }
  __syncthreads();
}

// f32 activations and weights: v_mfma_f32_16x16x4f32, super-step of 64.
template <int RB, int MODE>
__device__ __forceinline__ void splitk_body32(const GemmArgs& a, int item,
                                              int NNB, float* red) {
  constexpr int KSS = 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int g = item / NNB;
  const int nb = item - g * NNB;
  const int e = a.list[4 * g];
  const int row0 = a.list[4 * g + 1];
  const int nrows = a.list[4 * g + 2];
  const int off = a.offsets[e];
  const float* ap[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = row0 + min(rb * 16 + n, nrows - 1);
    if (MODE == 0)
      ap[rb] = (const float*)a.A + (size_t)a.pair_token[off + rr] * a.a_ld;
    else
      ap[rb] = (const float*)a.A + (size_t)(off + rr) * a.a_ld;
  }
  const float* bp[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int row;
    const void* base;
    if (MODE == 0) {
      row = nb * 32 + (cb >> 1) * 16 + n;
      base = (cb & 1) ? a.B1 : a.B0;
    } else {
      row = nb * 64 + cb * 16 + n;
      base = a.B0;
    }
    bp[cb] = (const float*)base + ((size_t)e * N + row) * K;
  }
  floatx4 acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int nss = K / KSS;
  const int s0 = wave * nss / 4, s1 = (wave + 1) * nss / 4;
  for (int s = s0; s < s1; ++s) {
    const int k0 = s * KSS + q * 16;
    float av[RB][16], bv[4][16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(ap[rb] + k0 + 4 * i);
        av[rb][4 * i] = v.x; av[rb][4 * i + 1] = v.y;
        av[rb][4 * i + 2] = v.z; av[rb][4 * i + 3] = v.w;
      }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(bp[cb] + k0 + 4 * i);
        bv[cb][4 * i] = v.x; bv[cb][4 * i + 1] = v.y;
        bv[cb][4 * i + 2] = v.z; bv[cb][4 * i + 3] = v.w;
      }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma16f32(av[rb][i], bv[cb][i], acc[rb][cb]);
  }
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* p = red + ((rb * 4 + cb) * 4 + r) * 64 + lane;
            *p = (w == 0) ? acc[rb][cb][r] : *p + acc[rb][cb][r];
          }
    }
    __syncthreads();
  }
  if (wave == 3) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[rb][cb][r] = red[((rb * 4 + cb) * 4 + r) * 64 + lane] + acc[rb][cb][r];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * 16 + q * 4 + r;
        if (row >= nrows) continue;
        const size_t prow = (size_t)(off + row0 + row);
        float* out = reinterpret_cast<float*>(a.out);
        if (MODE == 0) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const int f = nb * 32 + pr * 16 + n;
            out[prow * a.out_ld + f] = swiglu(acc[rb][2 * pr][r], acc[rb][2 * pr + 1][r], a.clamp);
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int d = nb * 64 + cb * 16 + n;
            out[prow * a.out_ld + d] = acc[rb][cb][r];
          }
        }
      }
  }
  __syncthreads();
}

template <class TT, int RB, int MODE, int LO>
__global__ __launch_bounds__(256) void gemm_splitk_kernel(GemmArgs a) {
  __shared__ float red[RB * 4 * 4 * 64];
  const int NNB = MODE == 0 ? a.N / 32 : a.N / 64;
  const int n_items = a.meta[a.meta_index] * NNB;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    if constexpr (TT::kBytes == 4)
      splitk_body32<RB, MODE>(a, item, NNB, red);
    else
      splitk_body16<TT, RB, MODE, LO>(a, item, NNB, red);
  }
}

// 4-bit weights, fp16 activations: four blocks per CU (128 registers), so
// that 16 waves keep their loads in flight. The column blocks of one group
// run on one XCD: its x rows, read by every column block, stay in that L2
// while the weights stream past.
template <int RB, int MODE, int FMT>
__global__ __launch_bounds__(256, 4) void gemm_splitk_q4_kernel(GemmArgs a) {
  __shared__ float red[RB * 4 * 4 * 64];
  const int NNB = MODE == 0 ? a.N / 32 : a.N / 64;
  const int n_items = a.meta[a.meta_index] * NNB;
  for (int rb0 = 0; rb0 < n_items; rb0 += gridDim.x) {
    const int item = xcd_item(rb0, blockIdx.x, gridDim.x, n_items);
    if (item >= 0) splitk_body_q4<RB, MODE, FMT>(a, item, NNB, red);
  }
}

template <class TT, int RB>
static hipError_t splitk_mode(const GemmArgs& a, int grid, hipStream_t s) {
  if (a.mode == 0)
    hipLaunchKernelGGL((gemm_splitk_kernel<TT, RB, 0, 0>), dim3(grid), dim3(256), 0, s, a);
  else if (TT::kBytes == 2 && a.A2)
    hipLaunchKernelGGL((gemm_splitk_kernel<TT, RB, 1, 1>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_splitk_kernel<TT, RB, 1, 0>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class TT>
static hipError_t splitk_rb(const GemmArgs& a, int rb, int grid, hipStream_t s) {
  return rb == 1 ? splitk_mode<TT, 1>(a, grid, s) : splitk_mode<TT, 4>(a, grid, s);
}

hipError_t launch_gemm_splitk(const GemmArgs& a, int xdt, int wdt, int rb,
                              int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (xdt == MOE_F32 && wdt == MOE_F32) return splitk_rb<F32T>(a, rb, grid, s);
  if (xdt == MOE_BF16 && wdt == MOE_BF16) return splitk_rb<BF16T>(a, rb, grid, s);
  if (xdt == MOE_F16 && wdt == MOE_F16) return splitk_rb<F16T>(a, rb, grid, s);
  const int fmt = q4_fmt(wdt);
  if (xdt == MOE_F16 && fmt >= 0) {
    // groups of <= 16 rows; the down stage reads H (fp16) as A in every case
    if (rb != 1) return hipErrorInvalidValue;
#define MOE_SKQ4(F_)                                                                      \
  do {                                                                                    \
    if (a.mode == 0)                                                                      \
      hipLaunchKernelGGL((gemm_splitk_q4_kernel<1, 0, F_>), dim3(grid), dim3(256), 0, s, a); \
    else                                                                                  \
      hipLaunchKernelGGL((gemm_splitk_q4_kernel<1, 1, F_>), dim3(grid), dim3(256), 0, s, a); \
  } while (0)
    if (fmt == 0) MOE_SKQ4(0);
    else if (fmt == 1) MOE_SKQ4(1);
    else MOE_SKQ4(2);
#undef MOE_SKQ4
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

// ---- combine ------------------------------------------------------------------------
//
// y[t, d..d+7] = sum over j of w[t, j] * Ypair[tok2pair[t, j], d..d+7] (j
// ascending, dropped pairs skipped) + the shared expert's row (weight 1).
// Ypair holds each kept pair's unweighted output (f32, or fp16 in an fp16
// layer); each product and the sum are f32 and the result is rounded once to
// y's dtype (mini-AGI PR #4, minagi/pool.py: the weighted gather back to
// tokens). Each output is written by one thread: no atomics.

template <class Y>
__device__ __forceinline__ void load_y8(const Y* p, float v[8]) {
  if constexpr (sizeof(Y) == 2) {
    const half8 h = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(p));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <class Y, class S>
__global__ __launch_bounds__(256) void combine_kernel(
    const Y* __restrict__ ypair, const int32_t* __restrict__ tok2pair,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets,
    int T, int D, int k, int n_shared, int E, S* __restrict__ y) {
  const int per_row = D / 8;
  const size_t total = (size_t)T * per_row;
  const size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int t = (int)(idx / per_row);
  const int d = (int)(idx - (size_t)t * per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // eight pairs at a time: their indices and weights, then all their rows,
  // are in flight together; the sum still runs in j order
  constexpr int kJ = 8;
  for (int j0 = 0; j0 < k; j0 += kJ) {
    int p[kJ];
    float w[kJ];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int j = j0 + jj;
      p[jj] = j < k ? tok2pair[(size_t)t * k + j] : -1;
      w[jj] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
    }
    float v[kJ][8];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
      if (p[jj] >= 0) load_y8(ypair + (size_t)p[jj] * D + d, v[jj]);
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
      if (p[jj] >= 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[jj][i] * w[jj];
      }
  }
  if (n_shared) {
    float v[8];
    load_y8(ypair + (size_t)(offsets[E] + t) * D + d, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  S* out = y + (size_t)t * D + d;
  if constexpr (sizeof(S) == 4) {
    reinterpret_cast<float4*>(out)[0] = float4{acc[0], acc[1], acc[2], acc[3]};
    reinterpret_cast<float4*>(out)[1] = float4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    typedef S s8 __attribute__((ext_vector_type(8)));
    s8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (S)acc[i];
    *reinterpret_cast<s8*>(out) = o;
  }
}

template <class Y>
static hipError_t combine_y(const void* ypair, const int32_t* tok2pair,
                            const float* topk_w, const int32_t* offsets, int T,
                            int D, int k, int n_shared, int E, int ydt, void* y,
                            int grid, hipStream_t s) {
  const Y* yp = (const Y*)ypair;
  if (ydt == MOE_F32)
    hipLaunchKernelGGL((combine_kernel<Y, float>), dim3(grid), dim3(256), 0, s,
                       yp, tok2pair, topk_w, offsets, T, D, k, n_shared, E, (float*)y);
  else if (ydt == MOE_BF16)
    hipLaunchKernelGGL((combine_kernel<Y, __bf16>), dim3(grid), dim3(256), 0, s,
                       yp, tok2pair, topk_w, offsets, T, D, k, n_shared, E, (__bf16*)y);
  else
    hipLaunchKernelGGL((combine_kernel<Y, _Float16>), dim3(grid), dim3(256), 0, s,
                       yp, tok2pair, topk_w, offsets, T, D, k, n_shared, E, (_Float16*)y);
  return hipGetLastError();
}

hipError_t launch_combine(const void* ypair, int ypair_f16,
                          const int32_t* tok2pair, const float* topk_w,
                          const int32_t* offsets, int T, int D, int k,
                          int n_shared, int E, int ydt, void* y, hipStream_t s) {
  const size_t total = (size_t)T * (D / 8);
  if (total == 0) return hipSuccess;
  const int grid = (int)((total + 255) / 256);
  return ypair_f16 ? combine_y<_Float16>(ypair, tok2pair, topk_w, offsets, T, D, k,
                                         n_shared, E, ydt, y, grid, s)
                   : combine_y<float>(ypair, tok2pair, topk_w, offsets, T, D, k,
                                      n_shared, E, ydt, y, grid, s);
}

}  // namespace moe
