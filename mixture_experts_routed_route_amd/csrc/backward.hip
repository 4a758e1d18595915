// Backward pass of the routed MoE layer on gfx950: gradients of
// L = sum_t dy[t] . y[t] for x, the three expert weights, the routing
// weights and (through the renormalised top-k softmax) the logits. Every
// expert slot gets the sum over its kept pairs, whatever the dispatch -- the
// property mini-AGI PR #3's tests/test_dispatch.py checks.
//
// Per kept pair p = (token t, expert e, weight w) in the plan's expert-sorted
// order (a pair of the shared expert has w = 1):
//   X_p  = x[t]        dYu = dy[t], dYp = w dy[t]   (compute dtype; dYp only
//                                                     as its transposed copy)
//   [G | U] = X_p [W_gate; W_up]^T      (f32, recomputed)
//   H    = silu(min(G, c)) clamp(U)     (compute dtype, as the forward)
//   dH'  = dYu W_down,  dH = w dH'      (f32)
//   dw_j = dH' . H  (= dy[t] . H W_down^T, the expert's output, regrouped:
//                    no product for the per-pair outputs is needed)
//   [dG | dU] = SwiGLU backward         (compute dtype)
//   dXp  = dG W_gate + dU W_up          dx[t] = sum over its pairs (fixed order)
//   dW_gate[e] = sum_p dG_p x_p^T,  dW_up[e] likewise,  dW_down[e] = sum_p dYp H_p^T
// The five products run on grouped MFMA kernels over 128 x 128 tiles whose
// operands stream HBM -> LDS by buffer_load ... lds through a ring of
// 64-deep stages: the weight gradients, whose K is the pair index, on
// pair-transposed copies of their operands; dH and dX, which read their
// weights as [K, N], with those rows kept in LDS as in memory and each K
// fragment assembled from 2-byte reads.
#include <algorithm>
#include <type_traits>

#include "device_common.h"

namespace moe {

namespace {

struct BF16B { using S = __bf16; using V8 = bf16x8; };
struct F16B { using S = _Float16; using V8 = half8; };

constexpr int kBT = 64;   // rows of a tile of the transposes

}  // namespace

// One operand of a grouped product. Element (i, k) of expert e:
//   KC (contiguous along K): base[(row0 + i) * ld + k]
//   IC (contiguous along i): base[(row0 + k) * ld + i]
// base = p + e * estride (a weight, estride > 0) or p (a per-pair buffer,
// estride == 0, whose rows start at the expert's first pair: row0 =
// offsets[e]). With p2, K values from k_split on come from p2 (k - k_split).
struct BOp {
  const void* p;
  const void* p2;
  int ld;
  int k_split;
  int64_t estride;
};

struct BGemmArgs {
  BOp a, b;
  int mode;                 // 0: per pair (rows = the expert's pairs), 1:
                            // weight gradient (K = the expert's pairs)
  int M, N, K;              // mode 0: N, K fixed; mode 1: M, N fixed
  float* c;                 // f32 output
  int ldc;
  int64_t c_estride;        // mode 1: output matrix of expert e at e * c_estride
  const int32_t* offsets;   // [n_exp + 1]
  const int32_t* tiles;     // mode 0: (expert, first row) per 128-row tile
  const int32_t* n_tiles;   // mode 0: number of tiles (device)
  const int32_t* koff;      // mode 1 on pair-transposed operands: expert e's
                            // K columns start at koff[e] (a multiple of 8)
  const int32_t* eord;      // mode 1: the experts, most K columns first
                            // and run to koff[e + 1] (zero padded)
  int n_exp;
};

// Products of two K-contiguous operands on 128 x 128 tiles, operands
// streamed HBM -> LDS by buffer_load ... lds through a ring of four 32 KB
// stages (64 K values, one whole 128-byte line per row), so that several
// stages' loads are in flight: waves 0..3 load the A rows, 4..7 the B rows;
// waves w and w + 4 own the same 64 x 64 outputs and take the first and
// second half of each stage's K, their sums added through LDS at the end.
// MODE 0: A = 128 pair rows of an expert (the 128-row tile list), B = rows
// of its weight, K fixed. MODE 1: both operands pair-transposed, rows are
// features, K = the expert's columns koff[e] .. koff[e + 1] (a multiple of
// 64, zero padded).
__device__ __forceinline__ int dswz(int r, int c) {
  return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

// The 128 x 128 f32 C tile of an 8-wave block (waves w and w + 4 hold the
// two k-halves of the same 64 x 64 quarter) through LDS: [128][128] f32,
// 16-byte chunks XOR 8 on rows with bit 2 set (the two row halves of an
// MFMA store land on other banks). The k-half kq = 1 stores its sums, kq = 0
// adds its own in place, then all eight waves write whole rows with 16-byte
// stores; rows at or past Me are not written. ct must hold 64 KB and be free.
__device__ __forceinline__ void store_c_tile(float* ct, const floatx16 (&acc)[2][2],
                                             int tid, int kq, int wm, int wn, int Me,
                                             float* c, int ldc) {
  const int lane = tid & 63;
  auto cix = [](int m, int n) {
    return m * 128 + (((n >> 2) ^ (((m >> 2) & 1) << 3)) << 2) + (n & 3);
  };
  if (kq == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          ct[cix(m, n)] = acc[i][j][r];
        }
      }
  }
  __syncthreads();
  if (kq == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          ct[cix(m, n)] += acc[i][j][r];
        }
      }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int q = tid + 512 * it;
    const int m = q >> 5, ch = q & 31;
    if (m < Me)
      *reinterpret_cast<float4*>(c + (size_t)m * ldc + ch * 4) =
          *reinterpret_cast<const float4*>(ct + cix(m, ch * 4));
  }
}

template <class TT, int MODE, int NS>
__global__ __launch_bounds__(512, NS == 2 ? 2 : 1) void bgemm_dma_kernel(BGemmArgs g) {
  using V8 = typename TT::V8;
  constexpr int kStage = 256 * 128;           // 128 A + 128 B rows
  constexpr int kDma = kStage / 1024 / 8;     // 4 loads per wave per stage
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];
  static_assert(NS * kStage >= 128 * 128 * 4, "the C tile is staged in the ring");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = wave >> 2, wq = wave & 3;
  const int wm = wq >> 1, wn = wq & 1;
  int e, m0, Me, n0, nk, kcol;
  const char* abase;
  const char* bbase;
  uint32_t a_rows, b_rows;      // rows each descriptor may touch
  float* cbase;
  size_t crow0;
  if constexpr (MODE == 0) {
    const int nt = g.N / 128;
    const int ti = blockIdx.x / nt;
    if (ti >= *g.n_tiles) return;   // block-uniform, before any barrier
    n0 = (blockIdx.x - ti * nt) * 128;
    e = g.tiles[2 * ti];
    m0 = g.tiles[2 * ti + 1];
    const int off = g.offsets[e];
    Me = min(128, g.offsets[e + 1] - off - m0);
    nk = g.K / 64;
    kcol = 0;
    abase = (const char*)g.a.p + (size_t)(off + m0) * g.a.ld * 2;
    a_rows = (uint32_t)Me;
    bbase = (const char*)g.b.p + ((size_t)e * g.b.estride + (size_t)n0 * g.b.ld) * 2;
    b_rows = 128;
    cbase = g.c;
    crow0 = (size_t)(off + m0);
  } else {
    const int mt = g.M / 128, nt = g.N / 128;
    const int per = mt * nt;
    // longest processing time first: the experts with the most pairs take
    // the first blocks, so their long tiles do not run alone at the end
    const int ei = blockIdx.x / per;
    const int r = blockIdx.x - ei * per;
    e = g.eord[ei];
    m0 = (r / nt) * 128;
    n0 = (r % nt) * 128;
    Me = 128;
    kcol = g.koff[e];
    nk = (g.koff[e + 1] - kcol) / 64;
    abase = (const char*)g.a.p + ((size_t)m0 * g.a.ld + kcol) * 2;
    a_rows = 128;
    bbase = (const char*)g.b.p + ((size_t)n0 * g.b.ld + kcol) * 2;
    b_rows = 128;
    cbase = g.c + (size_t)e * g.c_estride;
    crow0 = (size_t)m0;
  }
  if (nk == 0) {   // an expert without pairs: zero gradients (block-uniform)
    for (int i = tid; i < 128 * 128; i += 512)
      cbase[(crow0 + (i >> 7)) * g.ldc + n0 + (i & 127)] = 0.f;
    return;
  }
  const bool is_a = wave < 4;
  const int ld = is_a ? g.a.ld : g.b.ld;
  const int nrows = (int)(is_a ? a_rows : b_rows);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(
      is_a ? abase : bbase, (uint32_t)((size_t)(nrows - 1) * ld * 2 + (size_t)nk * 128));
  uint32_t voff[kDma];
#pragma unroll
  for (int jj = 0; jj < kDma; ++jj) {
    const int R = 8 * (wave * kDma + jj) + (lane >> 3);   // stage row 0..255
    const int r = min(is_a ? R : R - 128, nrows - 1);
    voff[jj] = (uint32_t)r * (uint32_t)ld * 2u + (uint32_t)((lane & 7) ^ ((R >> 1) & 7)) * 16u;
  }
  auto issue = [&](int kt) {
#pragma unroll
    for (int jj = 0; jj < kDma; ++jj) {
      char* dst = smem + (kt % NS) * kStage + (wave * kDma + jj) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, (int)voff[jj],
                                               min(kt, nk - 1) * 128, 0, 0);
    }
  };
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  struct Frag { V8 a[2]; V8 b[2]; };
  auto read = [&](int kt, int step, Frag& f) {
    const char* S = smem + (kt % NS) * kStage;
    const int ch = step * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      f.a[i] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(
          S + dswz(wm * 64 + i * 32 + (lane & 31), ch)));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      f.b[j] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(
          S + dswz(128 + wn * 64 + j * 32 + (lane & 31), ch)));
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st);
  wait_vmcnt<(NS - 2) * kDma>();
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
  read(0, 2 * kq, f0);
  for (int kt = 0; kt < nk; ++kt) {
    read(kt, 2 * kq + 1, f1);
    issue(kt + NS - 1);
    mma(f0);
    mma(f1);
    // stage kt+1 landed for this wave, then for every wave; the reads of
    // stage kt were consumed above, so its slot may be refilled next
    wait_vm_lgkm0<(NS - 2) * kDma>();
    __builtin_amdgcn_s_barrier();
    read(kt + 1, 2 * kq, f0);
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();   // the ring is free
  store_c_tile(reinterpret_cast<float*>(smem), acc, tid, kq, wm, wn, Me,
               cbase + crow0 * g.ldc + n0, g.ldc);
}

// Per-pair products whose weight is read as [K, N] (dH' = dYu W_down, and
// dX = [dG | dU] [W_gate; W_up], whose K runs through both weights): the
// same 128 x 128 tiles and ring as above, but a stage's 64 weight rows land
// in LDS as they are in memory (64 rows of 128 N values, 256 bytes; the
// 16-byte chunk c of row k at c ^ 4 for k / 8 odd, so that the two halves of
// a wave, reading rows k and k + 8, hit different banks), and each lane
// assembles its 8-deep K fragment from eight 2-byte reads.
__device__ __forceinline__ int icoff(int k, int n) {
  return k * 256 + ((((n >> 3) ^ (((k >> 3) & 1) << 2))) << 4) + (n & 7) * 2;
}

template <class TT, int NS>
__global__ __launch_bounds__(512, 1) void bgemm_dma_ic_kernel(BGemmArgs g) {
  using V8 = typename TT::V8;
  constexpr int kA = 128 * 128;               // A: 128 pair rows x 128 B
  constexpr int kB = 64 * 256;                // B: 64 K rows x 256 B
  constexpr int kStage = kA + kB;             // 32 KB
  constexpr int kDma = kStage / 1024 / 8;     // 4 loads per wave per stage
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = wave >> 2, wq = wave & 3;
  const int wm = wq >> 1, wn = wq & 1;
  const int nt = g.N / 128;
  const int ti = blockIdx.x / nt;
  if (ti >= *g.n_tiles) return;   // block-uniform, before any barrier
  const int n0 = (blockIdx.x - ti * nt) * 128;
  const int e = g.tiles[2 * ti];
  const int m0 = g.tiles[2 * ti + 1];
  const int off = g.offsets[e];
  const int Me = min(128, g.offsets[e + 1] - off - m0);
  const int nk = g.K / 64;
  const size_t crow0 = (size_t)(off + m0);
  // waves 0..3: A rows (8 rows of 128 B per 1 KB load); 4..7: B K-rows
  // (4 rows of 256 B per 1 KB load)
  const bool is_a = wave < 4;
  __amdgpu_buffer_rsrc_t rs, rs2;
  uint32_t voff[kDma];
  if (is_a) {
    const char* abase = (const char*)g.a.p + (size_t)(off + m0) * g.a.ld * 2;
    rs = make_rsrc(abase, (uint32_t)((size_t)(Me - 1) * g.a.ld * 2 + (size_t)nk * 128));
    rs2 = rs;
#pragma unroll
    for (int jj = 0; jj < kDma; ++jj) {
      const int R = 8 * (wave * kDma + jj) + (lane >> 3);
      const int r = min(R, Me - 1);
      voff[jj] = (uint32_t)r * (uint32_t)g.a.ld * 2u +
                 (uint32_t)((lane & 7) ^ ((R >> 1) & 7)) * 16u;
    }
  } else {
    // the weight rows of this expert: [K rows][ld] with the N columns n0..;
    // with p2, K values from k_split on come from the second matrix
    const char* b1 = (const char*)g.b.p + ((size_t)e * g.b.estride + n0) * 2;
    const char* b2 = g.b.p2 ? (const char*)g.b.p2 + ((size_t)e * g.b.estride + n0) * 2 : b1;
    const int k1 = g.b.p2 ? g.b.k_split : g.K;
    rs = make_rsrc(b1, (uint32_t)((size_t)(k1 - 1) * g.b.ld * 2 + 256));
    rs2 = make_rsrc(b2, (uint32_t)((size_t)(g.K - k1 > 0 ? g.K - k1 - 1 : 0) * g.b.ld * 2 + 256));
#pragma unroll
    for (int jj = 0; jj < kDma; ++jj) {
      const int kr = 4 * ((wave - 4) * kDma + jj) + (lane >> 4);   // K row 0..63
      const int p = lane & 15;                                      // LDS chunk
      const int c = p ^ (((kr >> 3) & 1) << 2);                     // its N chunk
      voff[jj] = (uint32_t)kr * (uint32_t)g.b.ld * 2u + (uint32_t)c * 16u;
    }
  }
  const int ksplit = g.b.p2 ? g.b.k_split : g.K;
  auto issue = [&](int kt) {
    const int kc = min(kt, nk - 1);
#pragma unroll
    for (int jj = 0; jj < kDma; ++jj) {
      char* dst = smem + (kt % NS) * kStage + (wave * kDma + jj) * 1024;
      if (is_a) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, (int)voff[jj],
                                                 kc * 128, 0, 0);
      } else {
        const int k0 = kc * 64;
        const bool second = k0 >= ksplit;
        const int krow = second ? k0 - ksplit : k0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rs2 : rs, (lds_ptr_t)dst, 16,
                                                 (int)voff[jj], krow * g.b.ld * 2, 0, 0);
      }
    }
  };
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  struct Frag { V8 a[2]; V8 b[2]; };
  auto read = [&](int kt, int step, Frag& f) {
    const char* S = smem + (kt % NS) * kStage;
    const int ch = step * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      f.a[i] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(
          S + dswz(wm * 64 + i * 32 + (lane & 31), ch)));
    const char* B = S + kA;
    const int kb = step * 16 + 8 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * 64 + j * 32 + (lane & 31);
      uint16_t h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        h[q] = *reinterpret_cast<const uint16_t*>(B + icoff(kb + q, n));
      f.b[j] = __builtin_bit_cast(V8, h);
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st);
  wait_vmcnt<(NS - 2) * kDma>();
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
  read(0, 2 * kq, f0);
  for (int kt = 0; kt < nk; ++kt) {
    read(kt, 2 * kq + 1, f1);
    issue(kt + NS - 1);
    mma(f0);
    mma(f1);
    wait_vm_lgkm0<(NS - 2) * kDma>();
    __builtin_amdgcn_s_barrier();
    read(kt + 1, 2 * kq, f0);
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();   // the ring is free
  store_c_tile(reinterpret_cast<float*>(smem), acc, tid, kq, wm, wn, Me,
               g.c + crow0 * g.ldc + n0, g.ldc);
}

// Exclusive prefix sums of v[0, n) in place, by a block of 1024 threads;
// returns the total to every thread. wsum: 17 ints of shared memory.
__device__ int block_scan_excl(int32_t* v, int n, int32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int C = (n + 1023) / 1024;   // items per thread, consecutive
  int loc = 0;
  for (int i = 0; i < C; ++i) {
    const int e = tid * C + i;
    if (e < n) loc += v[e];
  }
  int incl = loc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 16; ++i) {
      const int t = wsum[i];
      wsum[i] = acc;
      acc += t;
    }
    wsum[16] = acc;
  }
  __syncthreads();
  int run = wsum[w] + incl - loc;
  for (int i = 0; i < C; ++i) {
    const int e = tid * C + i;
    if (e < n) {
      const int t = v[e];
      v[e] = run;
      run += t;
    }
  }
  const int total = wsum[16];
  __syncthreads();
  return total;
}

// The work lists of the backward's products, one block of 1024 threads:
//  - (expert, first row) of every 64-row tile (the transposes) and every
//    128-row tile (dH', dX), in expert order, with their counts;
//  - the padded column offsets of the pair-transposed buffers: expert e's
//    pairs at columns koff[e] .. koff[e] + n_e, koff[e + 1] = koff[e] + n_e
//    rounded up to 64 (zeros in between);
//  - eord, the experts by padded column count, most first (ties by index);
//  - the full tile's lists, in eord order: the 256-row pair tiles of the
//    recompute of [G | U] (q[0] of them), and the 256-row tiles of the two
//    weight-gradient products over every expert, m_gu = 2F rows of
//    [dG | dU]^T (q[1] of them) and m_dn = D rows of (w dy)^T (q[2]); their
//    work-queue counters q[8..15], q[16..23], q[24..31] are zeroed.
__global__ __launch_bounds__(1024) void bwd_tiles_kernel(
    const int32_t* __restrict__ offsets, int n_exp, int m_gu, int m_dn,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ tiles128, int32_t* __restrict__ n_tiles128,
    int32_t* __restrict__ koff, int32_t* __restrict__ eord,
    int32_t* __restrict__ tiles256, int32_t* __restrict__ wl_gu,
    int32_t* __restrict__ wl_dn, int32_t* __restrict__ q) {
  __shared__ int32_t cnt[kMaxExperts + 2];
  __shared__ int32_t s1[kMaxExperts + 2], s2[kMaxExperts + 2];
  __shared__ int32_t s3[kMaxExperts + 2], s4[kMaxExperts + 2];
  __shared__ int32_t ord[kMaxExperts + 2];
  __shared__ int32_t wsum[17];
  const int tid = threadIdx.x;
  for (int e = tid; e < n_exp; e += blockDim.x) {
    const int ne = offsets[e + 1] - offsets[e];
    cnt[e] = ne;
    s1[e] = (ne + kBT - 1) / kBT;
    s2[e] = (ne + 127) / 128;
    s3[e] = (ne + 63) & ~63;
  }
  __syncthreads();
  const int n1 = block_scan_excl(s1, n_exp, wsum);
  const int n2 = block_scan_excl(s2, n_exp, wsum);
  const int ncol = block_scan_excl(s3, n_exp, wsum);
  for (int e = tid; e < n_exp; e += blockDim.x) {
    koff[e] = s3[e];
    const int kc = (cnt[e] + 63) & ~63;
    int rank = 0;
    for (int f = 0; f < n_exp; ++f) {
      const int kf = (cnt[f] + 63) & ~63;
      rank += kf > kc || (kf == kc && f < e);
    }
    eord[rank] = e;
    ord[rank] = e;
  }
  __syncthreads();
  for (int r = tid; r < n_exp; r += blockDim.x) s4[r] = (cnt[ord[r]] + 255) / 256;
  __syncthreads();
  const int n4 = block_scan_excl(s4, n_exp, wsum);
  if (tid == 0) {
    koff[n_exp] = ncol;
    *n_tiles = n1;
    *n_tiles128 = n2;
  }
  const int tg = (m_gu + 255) / 256, td = (m_dn + 255) / 256;
  if (tid < 32) q[tid] = tid == 0 ? n4 : tid == 1 ? n_exp * tg : tid == 2 ? n_exp * td : 0;
  for (int e = tid; e < n_exp; e += blockDim.x) {
    const int ne = cnt[e];
    for (int i = 0; i * kBT < ne; ++i) {
      tiles[2 * (s1[e] + i)] = e;
      tiles[2 * (s1[e] + i) + 1] = i * kBT;
    }
    for (int i = 0; i * 128 < ne; ++i) {
      tiles128[2 * (s2[e] + i)] = e;
      tiles128[2 * (s2[e] + i) + 1] = i * 128;
    }
  }
  for (int r = tid; r < n_exp; r += blockDim.x) {
    const int e = ord[r];
    for (int i = 0; i * 256 < cnt[e]; ++i) {
      tiles256[2 * (s4[r] + i)] = e;
      tiles256[2 * (s4[r] + i) + 1] = i * 256;
    }
    for (int i = 0; i < tg; ++i) {
      wl_gu[2 * (r * tg + i)] = e;
      wl_gu[2 * (r * tg + i) + 1] = i * 256;
    }
    for (int i = 0; i < td; ++i) {
      wl_dn[2 * (r * td + i)] = e;
      wl_dn[2 * (r * td + i) + 1] = i * 256;
    }
  }
}

// out[c, koff[e] + i] = in[offsets[e] + i, c] for the pairs of a 64-row
// tile (a tile holds one expert's pairs) and a 64-column block, with zeros
// in the padding columns after an expert's last pair. Staged through LDS
// (65-element rows: the column reads of the write-out avoid bank clashes).
template <class S>
__global__ __launch_bounds__(256) void bwd_transpose_kernel(
    const S* __restrict__ in, int C, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const int32_t* __restrict__ koff, int ld_out, const float* __restrict__ rw,
    S* __restrict__ out) {
  __shared__ S t[64][65];
  const int nc = C / 64;
  const int ti = blockIdx.x / nc;
  if (ti >= *n_tiles) return;
  const int c0 = (blockIdx.x - ti * nc) * 64;
  const int e = tiles[2 * ti], m0 = tiles[2 * ti + 1];
  const int off = offsets[e];
  const int ne = offsets[e + 1] - off;
  const int Me = min(64, ne - m0);
  const int tid = threadIdx.x;
  for (int q = tid; q < 64 * 8; q += 256) {
    const int r = q >> 3, ch = q & 7;
    S v[8];
    if (r < Me) {
      const uint4 u = *reinterpret_cast<const uint4*>(in + (size_t)(off + m0 + r) * C + c0 + ch * 8);
      __builtin_memcpy(v, &u, 16);
      if (rw) {
        const float w = rw[off + m0 + r];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (S)(w * (float)v[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (S)0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) t[r][ch * 8 + j] = v[j];
  }
  __syncthreads();
  // all 64 columns: past the expert's last pair they are its zero padding
  for (int q = tid; q < 64 * 8; q += 256) {
    const int c = q >> 3, ch = q & 7;
    S v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = t[ch * 8 + j][c];
    uint4 u;
    __builtin_memcpy(&u, v, 16);
    *reinterpret_cast<uint4*>(out + (size_t)(c0 + c) * ld_out + koff[e] + m0 + ch * 8) = u;
  }
}

// X_p = x[pair_token[p]] and dYu = dy[t], 8 values a thread.
template <class S>
__global__ __launch_bounds__(256) void bwd_gather_kernel(
    const S* __restrict__ x, const float* __restrict__ dy,
    const int32_t* __restrict__ pair_token, const int32_t* __restrict__ offsets,
    int n_exp, int D, S* __restrict__ Xp, S* __restrict__ dYu) {
  const int P = offsets[n_exp];
  const int upr = D / 8;
  for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < (size_t)P * upr;
       u += (size_t)gridDim.x * blockDim.x) {
    const size_t p = u / upr;
    const int c = (int)(u - p * upr) * 8;
    const int t = pair_token[p];
    *reinterpret_cast<uint4*>(Xp + p * D + c) =
        *reinterpret_cast<const uint4*>(x + (size_t)t * D + c);
    const float4 d0 = *reinterpret_cast<const float4*>(dy + (size_t)t * D + c);
    const float4 d1 = *reinterpret_cast<const float4*>(dy + (size_t)t * D + c + 4);
    S ou[8] = {(S)d0.x, (S)d0.y, (S)d0.z, (S)d0.w, (S)d1.x, (S)d1.y, (S)d1.z, (S)d1.w};
    __builtin_memcpy(dYu + p * D + c, ou, 16);
  }
}

__device__ __forceinline__ float clamp_hi(float v, float c) { return c > 0.f ? fminf(v, c) : v; }

// dG = dH * clamp(U) * silu'(min(G, c)) * [G <= c];
// dU = dH * silu(min(G, c)) * [-c <= U <= c]; silu'(z) = s (1 + z (1 - s)),
// s = 1 / (1 + e^-z). Written side by side, [P, 2F], compute dtype; 4
// features a thread.
__device__ __forceinline__ void swiglu_back1(float g, float u, float dh, float c,
                                             float& dg, float& du) {
  float gc = g, uc = u, mg = 1.f, mu = 1.f;
  if (c > 0.f) {
    if (g > c) { gc = c; mg = 0.f; }
    if (u < -c) { uc = -c; mu = 0.f; }
    if (u > c) { uc = c; mu = 0.f; }
  }
  const float s = 1.f / (1.f + expf(-gc));
  dg = dh * uc * s * (1.f + gc * (1.f - s)) * mg;
  du = dh * gc * s * mu;
}

// dH = pair_w[p] dH'_p; dG, dU from dH as above; H_p = SwiGLU(G, U) (silu
// with the hardware's 2^x and reciprocal), stored rounded once to the
// compute dtype for the dW_down product -- the plain one-value H of the
// forward; a bf16 forward that also carries H's low plane keeps about 16
// bits, so its dW_down differs from this one by that one rounding -- and
// dtw_p = dH'_p . H_p taken on the unrounded f32 H.
// One wave per pair: lanes over F four values at a time in a fixed stride,
// then a fixed butterfly for dtw_p.
template <class S>
__global__ __launch_bounds__(256) void bwd_swiglu_back_kernel(
    const float* __restrict__ GU, const float* __restrict__ dHu,
    const float* __restrict__ pair_w, const int32_t* __restrict__ offsets,
    int n_exp, int F, float c, S* __restrict__ dGU, S* __restrict__ H,
    float* __restrict__ dtwp) {
  const int lane = threadIdx.x & 63;
  const int P = offsets[n_exp];
  for (int p = blockIdx.x * 4 + (threadIdx.x >> 6); p < P; p += gridDim.x * 4) {
    const float w = pair_w[p];
    const float* gr = GU + (size_t)p * 2 * F;
    float acc = 0.f;
    for (int f = lane * 4; f < F; f += 256) {
      const float4 g = *reinterpret_cast<const float4*>(gr + f);
      const float4 u = *reinterpret_cast<const float4*>(gr + F + f);
      const float4 d = *reinterpret_cast<const float4*>(dHu + (size_t)p * F + f);
      const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
      const float dv[4] = {d.x, d.y, d.z, d.w};
      S og[4], ou[4], oh[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float hq = swiglu(gv[q], uv[q], c);
        oh[q] = (S)hq;
        acc = fmaf(dv[q], hq, acc);
        float dg, du;
        swiglu_back1(gv[q], uv[q], w * dv[q], c, dg, du);
        og[q] = (S)dg;
        ou[q] = (S)du;
      }
      __builtin_memcpy(dGU + (size_t)p * 2 * F + f, og, 8);
      __builtin_memcpy(dGU + (size_t)p * 2 * F + F + f, ou, 8);
      __builtin_memcpy(H + (size_t)p * F + f, oh, 8);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) dtwp[p] = acc;
  }
}

// dtw[t, j] = dtw_p of the token's j-th pair (0 for a dropped pair).
__global__ __launch_bounds__(256) void bwd_dtw_kernel(
    const float* __restrict__ dtwp, const int32_t* __restrict__ tok2pair, int64_t n,
    float* __restrict__ dtw) {
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int p = tok2pair[q];
    dtw[q] = p >= 0 ? dtwp[p] : 0.f;
  }
}

// dx[t] = sum over j of dXp[tok2pair[t, j]] (j ascending, dropped skipped)
// + the shared pair's row; each output written by one thread, 4 at a time.
__global__ __launch_bounds__(256) void bwd_dx_kernel(
    const float* __restrict__ dXp, const int32_t* __restrict__ tok2pair,
    const int32_t* __restrict__ offsets, int T, int k, int D, int n_shared,
    int E, float* __restrict__ dx) {
  const size_t n = (size_t)T * (D / 4);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / (D / 4);
    const int d = (int)(i - t * (D / 4)) * 4;
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int p = tok2pair[t * k + j];
      if (p >= 0) {
        const float4 v = *reinterpret_cast<const float4*>(dXp + (size_t)p * D + d);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
      }
    }
    if (n_shared) {
      const float4 v = *reinterpret_cast<const float4*>(dXp + ((size_t)offsets[E] + t) * D + d);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    *reinterpret_cast<float4*>(dx + t * D + d) = s;
  }
}

// dl[t, e_j] = w_j (dtw_j - sum_i w_i dtw_i), 0 for experts not chosen.
__global__ __launch_bounds__(256) void bwd_dlogits_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w,
    const float* __restrict__ dtw, int T, int E, int k, float* __restrict__ dl) {
  const int t = blockIdx.x;
  if (t >= T) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += w[(size_t)t * k + j] * dtw[(size_t)t * k + j];
  for (int e = threadIdx.x; e < E; e += blockDim.x) dl[(size_t)t * E + e] = 0.f;
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += blockDim.x)
    dl[(size_t)t * E + ids[(size_t)t * k + j]] =
        w[(size_t)t * k + j] * (dtw[(size_t)t * k + j] - s);
}

// ---- launcher ---------------------------------------------------------------

// pair columns of the transposed buffers: every expert padded to 64
static int64_t bwd_pcols(int64_t Pmax, int n_exp) {
  return (Pmax + 64 * (int64_t)n_exp + 63) & ~(int64_t)63;
}

size_t bwd_workspace_bytes(int64_t Pmax, int n_exp, int D, int F) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t tiles = (size_t)((Pmax + kBT - 1) / kBT + n_exp + 1);
  const size_t Pp = (size_t)bwd_pcols(Pmax, n_exp);
  return al(tiles * 8) * 2 + al(16) * 2 + al((n_exp + 1) * 4) + al(n_exp * 4) + al(Pmax * D * 2) +
         al(Pmax * 2 * F * 4) + al(Pmax * F * 2) + al(Pmax * D * 2) + al(Pmax * 4) +
         al(Pmax * F * 4) + al(Pmax * 2 * F * 2) + al(Pmax * D * 4) +
         al(Pp * D * 2) * 2 + al(Pp * 2 * F * 2) + al(Pp * F * 2) +
         al(tiles * 8) + al(128) +
         al((size_t)n_exp * ((2 * F + 255) / 256) * 8) +
         al((size_t)n_exp * ((D + 255) / 256) * 8);
}

// stage 0: gather, recompute [G | U] and H; 1: dH', dG / dU and dtw_p, dXp, dx;
// 2: the weight gradients; 3: the routing-weight and logit gradients
template <class TT>
static hipError_t run_bwd(const BwdArgs& a, int stage, hipStream_t s) {
  using S = typename TT::S;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const int64_t Pm = a.Pmax;
  const int D = a.D, F = a.F, n_exp = a.n_exp;
  char* b = static_cast<char*>(a.ws);
  const size_t ntile_cap = (size_t)((Pm + kBT - 1) / kBT + n_exp + 1);
  int32_t* tiles = reinterpret_cast<int32_t*>(b);        b += al(ntile_cap * 8);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(b);      b += al(16);
  int32_t* tiles128 = reinterpret_cast<int32_t*>(b);     b += al(ntile_cap * 8);
  int32_t* n_tiles128 = reinterpret_cast<int32_t*>(b);   b += al(16);
  int32_t* koff = reinterpret_cast<int32_t*>(b);         b += al((n_exp + 1) * 4);
  int32_t* eord = reinterpret_cast<int32_t*>(b);         b += al(n_exp * 4);
  S* Xp = reinterpret_cast<S*>(b);                       b += al(Pm * D * 2);
  float* GU = reinterpret_cast<float*>(b);               b += al(Pm * 2 * F * 4);
  S* H = reinterpret_cast<S*>(b);                        b += al(Pm * F * 2);
  S* dYu = reinterpret_cast<S*>(b);                      b += al(Pm * D * 2);
  float* dtwp = reinterpret_cast<float*>(b);             b += al(Pm * 4);
  float* dH = reinterpret_cast<float*>(b);               b += al(Pm * F * 4);
  S* dGU = reinterpret_cast<S*>(b);                      b += al(Pm * 2 * F * 2);
  float* dXp = reinterpret_cast<float*>(b);              b += al(Pm * D * 4);
  const int64_t Pp = bwd_pcols(Pm, n_exp);
  S* Xt = reinterpret_cast<S*>(b);                       b += al(Pp * D * 2);
  S* dYt = reinterpret_cast<S*>(b);                      b += al(Pp * D * 2);
  S* dGUt = reinterpret_cast<S*>(b);                     b += al(Pp * 2 * F * 2);
  S* Ht = reinterpret_cast<S*>(b);                       b += al(Pp * F * 2);
  int32_t* tiles256 = reinterpret_cast<int32_t*>(b);     b += al(ntile_cap * 8);
  int32_t* q = reinterpret_cast<int32_t*>(b);            b += al(128);
  int32_t* wl_gu = reinterpret_cast<int32_t*>(b);
  b += al((size_t)n_exp * ((2 * F + 255) / 256) * 8);
  int32_t* wl_dn = reinterpret_cast<int32_t*>(b);
  // the full tile addresses its operands with 32-bit buffer offsets
  const bool full_ok = (size_t)a.T * D * 2 < ((size_t)1 << 31) &&
                       (size_t)std::max(2 * F, D) * (size_t)Pp * 2 < ((size_t)1 << 32);

  const int ew_grid = a.ncu * 8;
  const int ub = (int)ntile_cap;
  const int ub128 = (int)((Pm + 127) / 128 + n_exp + 1);
  auto per_pair = [&](auto akc, auto bkc, const BOp& A, const BOp& B, int N,
                      int K, float* C, int ldc) {
    BGemmArgs g{};
    g.a = A; g.b = B; g.mode = 0; g.N = N; g.K = K; g.c = C; g.ldc = ldc;
    g.offsets = a.offsets; g.tiles = tiles; g.n_tiles = n_tiles; g.n_exp = n_exp;
    if constexpr (decltype(bkc)::value) {
      g.tiles = tiles128;
      g.n_tiles = n_tiles128;
      hipLaunchKernelGGL((bgemm_dma_kernel<TT, 0, 4>), dim3(ub128 * (N / 128)), dim3(512),
                         0, s, g);
    } else {
      g.tiles = tiles128;
      g.n_tiles = n_tiles128;
      hipLaunchKernelGGL((bgemm_dma_ic_kernel<TT, 4>), dim3(ub128 * (N / 128)), dim3(512),
                         0, s, g);
    }
  };
  // weight gradients on the pair-transposed copies: both operands
  // contiguous along the pair index
  auto weight_grad = [&](const BOp& A, const BOp& B, int M, int N, float* C) {
    BGemmArgs g{};
    g.a = A; g.b = B; g.mode = 1; g.M = M; g.N = N; g.c = C; g.ldc = N;
    g.c_estride = (int64_t)M * N; g.offsets = a.offsets; g.koff = koff; g.eord = eord;
    g.n_exp = n_exp;
    hipLaunchKernelGGL((bgemm_dma_kernel<TT, 1, 2>),
                       dim3(n_exp * (M / 128) * (N / 128)), dim3(512), 0, s, g);
  };
  auto transpose = [&](const S* in, int C, S* outp, const float* rw) {
    hipLaunchKernelGGL((bwd_transpose_kernel<S>), dim3(ub * (C / 64)), dim3(256), 0, s,
                       in, C, a.offsets, tiles, n_tiles, koff, (int)Pp, rw, outp);
  };
  using KCt = std::true_type;
  using ICt = std::false_type;
  const int64_t wFD = (int64_t)F * D;
  if (stage == 0) {
    hipLaunchKernelGGL(bwd_tiles_kernel, dim3(1), dim3(1024), 0, s, a.offsets,
                       n_exp, 2 * F, D, tiles, n_tiles, tiles128, n_tiles128, koff,
                       eord, tiles256, wl_gu, wl_dn, q);
    hipLaunchKernelGGL((bwd_gather_kernel<S>), dim3(ew_grid), dim3(256), 0, s,
                       (const S*)a.x, a.dy, a.pair_token, a.offsets,
                       n_exp, D, Xp, dYu);
    // [G | U] = X_p [W_gate; W_up]^T on the forward's full tile (x rows
    // gathered through the pair list, raw f32 outputs)
    if (full_ok) {
      GemmArgs gf{};
      gf.mode = 2; gf.K = D; gf.N = F;
      gf.A = a.x; gf.a_bytes = (uint32_t)((size_t)a.T * D * 2); gf.a_ld = D;
      gf.out = GU; gf.out_ld = 2 * F;
      gf.pair_token = a.pair_token; gf.offsets = a.offsets; gf.pair_w = a.pair_w;
      gf.B0 = a.wg; gf.B1 = a.wu; gf.fat_slot = nullptr;
      gf.list = tiles256; gf.meta = q; gf.meta_index = 0; gf.queue = q + 8;
      gf.clamp = a.clamp;
      const int grid = (int)std::min<int64_t>((int64_t)ntile_cap * (F / 128), a.ncu);
      const hipError_t e = launch_gemm_full(gf, a.xdt, grid, s);
      if (e != hipSuccess) return e;
    } else {
      per_pair(KCt{}, KCt{}, BOp{Xp, nullptr, D, 0, 0}, BOp{a.wg, nullptr, D, 0, wFD},
               F, D, GU, 2 * F);
      per_pair(KCt{}, KCt{}, BOp{Xp, nullptr, D, 0, 0}, BOp{a.wu, nullptr, D, 0, wFD},
               F, D, GU + F, 2 * F);
    }
  } else if (stage == 1) {
    // dH' = dYu W_down (unscaled; the SwiGLU backward applies pair_w)
    per_pair(KCt{}, ICt{}, BOp{dYu, nullptr, D, 0, 0}, BOp{a.wd, nullptr, F, 0, wFD},
             F, D, dH, F);
    hipLaunchKernelGGL((bwd_swiglu_back_kernel<S>), dim3(ew_grid), dim3(256), 0, s,
                       GU, dH, a.pair_w, a.offsets, n_exp, F, a.clamp, dGU, H, dtwp);
    // dXp = [dG | dU] [W_gate; W_up]
    per_pair(KCt{}, ICt{}, BOp{dGU, nullptr, 2 * F, 0, 0}, BOp{a.wg, a.wu, D, F, wFD},
             D, 2 * F, dXp, D);
    if (a.dx)
      hipLaunchKernelGGL(bwd_dx_kernel, dim3(ew_grid), dim3(256), 0, s, dXp,
                         a.tok2pair, a.offsets, a.T, a.k, D, a.n_shared, a.E, a.dx);
  } else if (stage == 2) {
    // weight gradients (every expert, zero pairs give zeros)
    transpose(Xp, D, Xt, nullptr);
    transpose(dYu, D, dYt, a.pair_w);   // dYp = pair_w dy[t], transposed
    transpose(dGU, 2 * F, dGUt, nullptr);
    transpose(H, F, Ht, nullptr);
    if (full_ok) {
      // on the full tile: 256 x 256 tiles of every expert's gradient, K =
      // its padded pair columns, heaviest experts first
      auto wgrad_full = [&](const S* A, int M, const S* B, int N, float* out,
                            float* out2, int row_split, const int32_t* list,
                            int mi, int32_t* queue) {
        GemmArgs g{};
        g.mode = 3; g.K = kBT; g.N = N; g.M = M; g.row_split = row_split;
        g.A = A; g.a_bytes = (uint32_t)((size_t)M * Pp * 2); g.a_ld = (int)Pp;
        g.B0 = B; g.b_bytes = (uint32_t)((size_t)N * Pp * 2); g.b_ld = (int)Pp;
        // expert e's gradient: row_split rows of N at e row_split N
        g.koff = koff; g.out = out; g.out2 = out2; g.out_estride = (int64_t)row_split * N;
        g.list = list; g.meta = q; g.meta_index = mi; g.queue = queue;
        const int64_t items = (int64_t)n_exp * ((M + 255) / 256) * ((N + 255) / 256);
        return launch_gemm_full(g, a.xdt, (int)std::min<int64_t>(items, a.ncu), s);
      };
      hipError_t e = wgrad_full(dGUt, 2 * F, Xt, D, a.dwg, a.dwu, F, wl_gu, 1, q + 16);
      if (e != hipSuccess) return e;
      e = wgrad_full(dYt, D, Ht, F, a.dwd, a.dwd, D, wl_dn, 2, q + 24);
      if (e != hipSuccess) return e;
    } else {
      weight_grad(BOp{dGUt, nullptr, (int)Pp, 0, 0}, BOp{Xt, nullptr, (int)Pp, 0, 0},
                  F, D, a.dwg);
      weight_grad(BOp{dGUt + (size_t)F * Pp, nullptr, (int)Pp, 0, 0},
                  BOp{Xt, nullptr, (int)Pp, 0, 0}, F, D, a.dwu);
      weight_grad(BOp{dYt, nullptr, (int)Pp, 0, 0}, BOp{Ht, nullptr, (int)Pp, 0, 0},
                  D, F, a.dwd);
    }
  } else if (a.dtw || a.dlogits) {
    float* dtw = a.dtw ? a.dtw : a.dtw_scratch;
    const int64_t q = (int64_t)a.T * a.k;
    if (q > 0)
      hipLaunchKernelGGL(bwd_dtw_kernel, dim3((unsigned)std::min<int64_t>((q + 255) / 256, ew_grid)),
                         dim3(256), 0, s, dtwp, a.tok2pair, q, dtw);
    if (a.dlogits && a.T > 0)
      hipLaunchKernelGGL(bwd_dlogits_kernel, dim3(a.T), dim3(256), 0, s, a.ids,
                         a.topk_w, dtw, a.T, a.E, a.k, a.dlogits);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, int stage, hipStream_t s) {
  if (a.xdt == MOE_BF16) return run_bwd<BF16B>(a, stage, s);
  if (a.xdt == MOE_F16) return run_bwd<F16B>(a, stage, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
