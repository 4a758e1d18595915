// Router of the routed MoE layer on gfx950: the linear map from d_model to
// the E expert logits, and the routing statistics kept beside the routing.
//
// The pages route the output of a linear router over each token's hidden
// state and, in the same call, keep three numbers about it (mini-AGI PR #3,
// minagi/pool.py, `requested(scores)`): the softmax mass of the k chosen
// experts before their weights are renormalised, how many experts the router
// wants (the fewest holding 90 % of the mass), and an auxiliary loss made of
// a balance term (E times the sum over experts of the share of first choices
// times the mean probability) plus z_weight times the mean squared
// log-sum-exp of the logits (the z-loss; z_weight defaults to 1e-3 in that
// class's constructor).
//
// Kernels:
//  * router_mfma_kernel: logits = x Wr^T on the fp16/bf16 matrix cores, one
//    block per (token tile, expert tile), operands streamed HBM -> LDS with
//    buffer_load ... lds through a 4-stage ring (the full expert tile's
//    scheme at a smaller tile: a long prompt has T x E / 16384 tiles of
//    128 x 128, enough for the chip; shorter ones take 64 x 64 tiles).
//  * router_dot_kernel: one wave per expert and up to 8 tokens, fp32 FMAs in
//    a fixed order (fp32 inputs, and prompts too short for a tile).
//  * router_stats_kernel: per token softmax, log-sum-exp, top-k mass (over the
//    plan's chosen experts) and the wanted count (an exact threshold search
//    in fp32); per block, the sums per expert go into cross-block totals as
//    fixed-point integers (integer atomics: the same total in any order) and
//    the scalar sums into per-block partials, which router_final_kernel adds
//    in a fixed order in double. No float atomics anywhere: every result is
//    the same bits from run to run.
#include <type_traits>

#include "device_common.h"

namespace moe {

namespace {

struct RF16 { using V8 = half8; };
struct RBF16 { using V8 = bf16x8; };

// 64-byte LDS rows (32 K values): chunk c of row r sits at c ^ ((r >> 2) & 3).
__device__ __forceinline__ int rswz(int r, int c) {
  return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}

constexpr int kRBK = 32;      // K values per stage
// Ring depth: a stage's loads take about a microsecond to land, so the
// tile keeps NS - 1 stages (7 x 16 KB or 7 x 8 KB) in flight.
constexpr int kRNS = 8;
constexpr int kStatTok = 16;  // tokens per statistics block

}  // namespace

// logits[t, e] for a BT (tokens) x BE (experts) tile per block of 4 waves;
// wave (we, wt) owns experts we * BE/2 .. and tokens wt * BT/2 ... The expert
// rows are the MFMA's A operand and the token rows its B operand, so a lane's
// 32x32 accumulator holds 4 consecutive experts of one token per group of
// four registers (16-byte stores into the token-major logits).
template <class TT, int BT, int BE, int NS>
__global__ __launch_bounds__(256, 2) void router_mfma_kernel(
    const void* __restrict__ x, const void* __restrict__ w,
    float* __restrict__ logits, int T, int D, int E,
    uint32_t* __restrict__ zero, int zero_words) {
  using V8 = typename TT::V8;
  constexpr int kRows = BT + BE;               // LDS rows per stage
  constexpr int kStage = kRows * 64;
  constexpr int kDma = kStage / 1024 / 4;      // 1 KB loads per wave per stage
  constexpr int kEarly = kDma / 2;             // of them before mid-stage
  constexpr int NI = BE / 64, NJ = BT / 64;    // 32-row blocks per wave
  static_assert(kDma >= 2 && (BE % 64) == 0 && (BT % 64) == 0, "tile shape");
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int we = wave >> 1, wt = wave & 1;
  const int n_eb = (E + BE - 1) / BE;
  const int n_items = n_eb * ((T + BT - 1) / BT);
  // the expert tiles of one token tile run on one XCD and share its x rows
  const int item = xcd_item(0, blockIdx.x, gridDim.x, n_items);
  if (item < 0) return;   // block-uniform, before any barrier
  // block 0 clears the statistics accumulators the next kernels add into
  if (blockIdx.x == 0)
    for (int i = tid; i < zero_words; i += 256) zero[i] = 0u;
  const int tb = item / n_eb, eb = item - tb * n_eb;
  const int e0 = eb * BE, t0 = tb * BT;
  const int ne = min(BE, E - e0), nt = min(BT, T - t0);
  const int nk = D / kRBK;

  // Stage rows 0 .. BE-1 hold expert rows, BE .. BE+BT-1 token rows: waves
  // 0, 1 load the former, 2, 3 the latter, kDma 16-row blocks each; a lane
  // loads the global 16-byte chunk that lands in the swizzled slot its
  // position in the 1 KB block maps to. Rows past the tile's end repeat its
  // last row (their results are not stored).
  // one descriptor per wave (an array of buffer descriptors in this kernel
  // template left its host launch stub undefined at link time)
  static_assert(BE % (16 * kDma) == 0, "a wave loads one operand");
  const bool is_w = 16 * kDma * wave < BE;   // wave-uniform
  const int nrows = is_w ? ne : nt;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(
      is_w ? (const char*)w + (size_t)e0 * D * 2 : (const char*)x + (size_t)t0 * D * 2,
      (uint32_t)nrows * (uint32_t)D * 2u);
  uint32_t voff[kDma];
#pragma unroll
  for (int jj = 0; jj < kDma; ++jj) {
    const int R = 16 * (wave * kDma + jj) + (lane >> 2);
    const int r = min(is_w ? R : R - BE, nrows - 1);
    voff[jj] = (uint32_t)r * (uint32_t)D * 2u +
               (uint32_t)((lane & 3) ^ ((R >> 2) & 3)) * 16u;
  }
  // refill of ring stage kt; past the last stage the last slice is read again
  // into a slot no one reads, so every wait below counts a constant number
  auto issue_one = [&](int kt, int jj) {
    char* dst = smem + (kt % NS) * kStage + (wave * kDma + jj) * 1024;
    const int soff = min(kt, nk - 1) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16,
                                             (int)voff[jj], soff, 0, 0);
  };

  floatx16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frag { V8 a[NI]; V8 b[NJ]; };
  constexpr int kRd = NI + NJ;
  auto read_piece = [&](int kt, int ks, int idx, Frag& f) {
    const char* S = smem + (kt % NS) * kStage;
    const int ch = ks * 2 + (lane >> 5);
    if (idx < NI) {
      const int r = we * (BE / 2) + idx * 32 + (lane & 31);
      f.a[idx] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(S + rswz(r, ch)));
    } else {
      const int j = idx - NI;
      const int r = BE + wt * (BT / 2) + j * 32 + (lane & 31);
      f.b[j] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(S + rswz(r, ch)));
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int jj = 0; jj < kDma; ++jj) issue_one(s, jj);
  wait_vmcnt<(NS - 2) * kDma>();   // stage 0 landed for this wave
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
#pragma unroll
  for (int q = 0; q < kRd; ++q) read_piece(0, 0, q, f0);

  constexpr int kMf = NI * NJ;
  constexpr int kSl = kMf > kRd ? kMf : kRd;
  for (int kt = 0; kt < nk; ++kt) {
    // first half of the stage: refill three stages ahead, read step 1 while
    // step 0 multiplies
#pragma unroll
    for (int q = 0; q < kRd; ++q) {
      if (q < kEarly) issue_one(kt + NS - 1, q);
      read_piece(kt, 1, q, f1);
    }
#pragma unroll
    for (int q = kRd; q < kEarly; ++q) issue_one(kt + NS - 1, q);
    mma(f0);
#pragma unroll
    for (int q = 0; q < kSl; ++q) {
      if (q < kMf) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < kEarly) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (q < kRd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 landed for this wave, then (barrier) for every wave; all
    // reads of stage kt are done before anyone refills its slot
    wait_vm_lgkm0<(NS - 3) * kDma + kEarly>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < kRd; ++q) {
      if (q < kDma - kEarly) issue_one(kt + NS - 1, kEarly + q);
      read_piece(kt + 1, 0, q, f0);
    }
#pragma unroll
    for (int q = kRd; q < kDma - kEarly; ++q) issue_one(kt + NS - 1, kEarly + q);
    mma(f1);
#pragma unroll
    for (int q = 0; q < kSl; ++q) {
      if (q < kMf) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < kDma - kEarly) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (q < kRd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();

  // accumulator r of a 32x32 block: expert 8 (r / 4) + 4 (lane / 32) + r % 4,
  // token lane % 32
  const int hi4 = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int t = t0 + wt * (BT / 2) + j * 32 + (lane & 31);
    if (t >= T) continue;
    float* row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int e = e0 + we * (BE / 2) + i * 32 + rq * 8 + hi4;
        if ((E & 3) == 0) {
          if (e < E)
            *reinterpret_cast<float4*>(row + e) =
                float4{acc[i][j][rq * 4], acc[i][j][rq * 4 + 1],
                       acc[i][j][rq * 4 + 2], acc[i][j][rq * 4 + 3]};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (e + q < E) row[e + q] = acc[i][j][rq * 4 + q];
        }
      }
  }
}

// The 128 x 128 tile on 8 waves with 64-deep stages: each stage holds 256
// rows of 128 bytes (one whole cache line per row: a stage of 64-byte row
// slices made every line arrive in two halves, a stage apart). Waves w and
// w + 4 own the same 64 x 64 outputs; w takes the first two 16-deep steps of
// every stage and w + 4 the last two, each with its own accumulators, added
// (first + second) through LDS at the end. Chunk c of LDS row r sits at
// c ^ ((r >> 1) & 7): the 16 rows one phase of a fragment read touches land
// on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int rswz128(int r, int c) {
  return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

template <class TT, int NS>
__global__ __launch_bounds__(512, 1) void router_mfma8_kernel(
    const void* __restrict__ x, const void* __restrict__ w,
    float* __restrict__ logits, int T, int D, int E,
    uint32_t* __restrict__ zero, int zero_words) {
  using V8 = typename TT::V8;
  constexpr int BT = 128, BE = 128, BK = 64;
  constexpr int kStage = (BT + BE) * 128;     // 32 KB
  constexpr int kDma = kStage / 1024 / 8;     // 4 loads per wave per stage
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = wave >> 2, wq = wave & 3;
  const int we = wq >> 1, wt = wq & 1;
  const int n_eb = (E + BE - 1) / BE;
  const int n_items = n_eb * ((T + BT - 1) / BT);
  const int item = xcd_item(0, blockIdx.x, gridDim.x, n_items);
  if (item < 0) return;   // block-uniform, before any barrier
  if (blockIdx.x == 0)
    for (int i = tid; i < zero_words; i += 512) zero[i] = 0u;
  const int tb = item / n_eb, eb = item - tb * n_eb;
  const int e0 = eb * BE, t0 = tb * BT;
  const int ne = min(BE, E - e0), nt = min(BT, T - t0);
  const int nk = D / BK;

  // waves 0..3 load the expert rows (stage rows 0..127), 4..7 the tokens';
  // a 1 KB load is 8 rows of 128 bytes, lane L taking row L / 8
  const bool is_w = wave < 4;
  const int nrows = is_w ? ne : nt;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(
      is_w ? (const char*)w + (size_t)e0 * D * 2 : (const char*)x + (size_t)t0 * D * 2,
      (uint32_t)nrows * (uint32_t)D * 2u);
  uint32_t voff[kDma];
#pragma unroll
  for (int jj = 0; jj < kDma; ++jj) {
    const int R = 8 * (wave * kDma + jj) + (lane >> 3);
    const int r = min(is_w ? R : R - BE, nrows - 1);
    voff[jj] = (uint32_t)r * (uint32_t)D * 2u +
               (uint32_t)((lane & 7) ^ ((R >> 1) & 7)) * 16u;
  }
  auto issue_one = [&](int kt, int jj) {
    char* dst = smem + (kt % NS) * kStage + (wave * kDma + jj) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16,
                                             (int)voff[jj],
                                             min(kt, nk - 1) * 128, 0, 0);
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  struct Frag { V8 a[2]; V8 b[2]; };
  // fragments of 16-deep step `step` (0..3) of stage kt
  auto read = [&](int kt, int step, Frag& f) {
    const char* S = smem + (kt % NS) * kStage;
    const int ch = step * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = we * 64 + i * 32 + (lane & 31);
      f.a[i] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(S + rswz128(r, ch)));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = BE + wt * 64 + j * 32 + (lane & 31);
      f.b[j] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(S + rswz128(r, ch)));
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int jj = 0; jj < kDma; ++jj) issue_one(s, jj);
  wait_vmcnt<(NS - 2) * kDma>();   // stage 0 landed for this wave
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
  read(0, 2 * kq, f0);
  for (int kt = 0; kt < nk; ++kt) {
    // second step's reads and the refill three stages ahead, between the
    // first step's MFMAs
    read(kt, 2 * kq + 1, f1);
#pragma unroll
    for (int jj = 0; jj < kDma; ++jj) issue_one(kt + NS - 1, jj);
    mma(f0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    // stage kt+1 landed for this wave, then for every wave; every wave's
    // reads of stage kt were consumed by its MFMAs above, so the slot can be
    // refilled from the next iteration on
    wait_vm_lgkm0<(NS - 2) * kDma>();
    __builtin_amdgcn_s_barrier();
    read(kt + 1, 2 * kq, f0);
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();   // the ring is free
  // the second-half waves hand their sums over: [wq][register][lane] floats
  float* red = reinterpret_cast<float*>(smem) + wq * (64 * 64);
  if (kq == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((i * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];
  }
  __syncthreads();
  if (kq == 1) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * 2 + j) * 16 + r) * 64 + lane];

  const int hi4 = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + wt * 64 + j * 32 + (lane & 31);
    if (t >= T) continue;
    float* row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int e = e0 + we * 64 + i * 32 + rq * 8 + hi4;
        if ((E & 3) == 0) {
          if (e < E)
            *reinterpret_cast<float4*>(row + e) =
                float4{acc[i][j][rq * 4], acc[i][j][rq * 4 + 1],
                       acc[i][j][rq * 4 + 2], acc[i][j][rq * 4 + 3]};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (e + q < E) row[e + q] = acc[i][j][rq * 4 + q];
        }
      }
  }
}

namespace {

template <class X> __device__ __forceinline__ float to_f(X v) { return (float)v; }

// Sum over the 64 lanes by xor butterflies: every lane ends with the same
// value (each step adds the same two numbers in both lanes of a pair).
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}

}  // namespace

// One wave per expert and TT tokens: each lane takes 16-byte slices of D in
// a fixed stride, fp32 FMAs in slice order, then the butterfly sum.
template <class X, int TT>
__global__ __launch_bounds__(256) void router_dot_kernel(
    const X* __restrict__ x, const X* __restrict__ w,
    float* __restrict__ logits, int T, int D, int E,
    uint32_t* __restrict__ zero, int zero_words) {
  constexpr int V = 16 / sizeof(X);
  const int lane = threadIdx.x & 63;
  // block (0, 0) clears the statistics accumulators the next kernels add into
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < zero_words; i += 256) zero[i] = 0u;
  const int e = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.x * TT;
  if (e >= E) return;   // wave-uniform; the kernel has no barrier
  const int nt = min(TT, T - t0);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
  const X* wr = w + (size_t)e * D;
  for (int d = lane * V; d < D; d += 64 * V) {
    const uint4 wu = ldg16(wr + d);
    X wv[V];
    __builtin_memcpy(wv, &wu, 16);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t < nt) {
        const uint4 xu = ldg16(x + (size_t)(t0 + t) * D + d);
        X xv[V];
        __builtin_memcpy(xv, &xu, 16);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[t] = fmaf(to_f(xv[v]), to_f(wv[v]), acc[t]);
      }
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float s = wave_sum_f(acc[t]);
    if (lane == t) mine = s;
  }
  if (lane < nt) logits[(size_t)(t0 + lane) * E + e] = mine;
}

namespace {

// DPP moves within a 16-lane row: quad_perm [1,0,3,2], [2,3,0,1], the
// half-row mirror and the row mirror. After the four steps every lane of a
// row holds the row's total, added in the same order in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row_sum_f(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}
__device__ __forceinline__ float row_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
__device__ __forceinline__ int row_sum_i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x141>(v);
  v += dpp_i<0x140>(v);
  return v;
}
// group reductions: G = 16 lanes (one DPP row) or the whole wave (the four
// row totals added in row order)
template <int G>
__device__ __forceinline__ float grp_sum_f(float v) {
  v = row_sum_f(v);
  if constexpr (G == 64) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    v = (r0 + r1) + (r2 + r3);
  }
  return v;
}
template <int G>
__device__ __forceinline__ float grp_max_f(float v) {
  v = row_max_f(v);
  if constexpr (G == 64) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
  }
  return v;
}
template <int G>
__device__ __forceinline__ int grp_sum_i(int v) {
  v = row_sum_i(v);
  if constexpr (G == 64)
    v = (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
        (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
  return v;
}

}  // namespace

// Per token (a group of G lanes; expert e in lane e % G, slot e / G):
//   m = max logit, s = sum exp(l - m), lse = m + log s, p = exp(l - m) / s;
//   kept = sum of p over the plan's k chosen experts;
//   want = the fewest experts whose p, largest first, reach 0.9: the largest
//   threshold tau (on the bits of p, which order like the values) whose mass
//   sum(p >= tau) is at least 0.9, found bit by bit; the experts above tau
//   then count once each and the ones equal to tau as many as the sum needs.
// Each block takes kStatTok tokens: its sums of p and of first choices per
// expert are added into the zeroed totals acc_p (fixed point) and acc_c, and
// its kept / want / lse^2 sums written to part_s.
template <int G, int PER>
__global__ __launch_bounds__(256) void router_stats_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ids, int T,
    int E, int k, int32_t* __restrict__ want_out,
    unsigned long long* __restrict__ acc_p, uint32_t* __restrict__ acc_c,
    float* __restrict__ part_s) {
  constexpr int kGroups = 64 / G;                 // tokens per wave at once
  constexpr int kPasses = (kStatTok / 4) / kGroups;
  __shared__ float sh_p[4][kMaxExperts];
  __shared__ int32_t sh_c[kMaxExperts];
  __shared__ float sh_s[4][3];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane % G, grp = lane / G;
  for (int e = threadIdx.x; e < E; e += 256) sh_c[e] = 0;
  __syncthreads();

  float psum[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) psum[j] = 0.f;
  float a_kept = 0.f, a_want = 0.f, a_z = 0.f;
  for (int pass = 0; pass < kPasses; ++pass) {
    const int t = blockIdx.x * kStatTok + wave * (kStatTok / 4) + pass * kGroups + grp;
    const bool vt = t < T;
    float l[PER];
    bool ve[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = gl + G * j;
      ve[j] = vt && e < E;
      l[j] = ve[j] ? logits[(size_t)t * E + e] : -__builtin_inff();
    }
    float mx = l[0];
#pragma unroll
    for (int j = 1; j < PER; ++j) mx = fmaxf(mx, l[j]);
    const float m = grp_max_f<G>(mx);
    float ex[PER], sl = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      ex[j] = ve[j] ? expf(l[j] - m) : 0.f;
      sl += ex[j];
    }
    const float s = grp_sum_f<G>(sl);
    const float lse = m + logf(s);
    float p[PER];
    uint32_t pb[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      p[j] = ve[j] ? ex[j] / s : 0.f;
      pb[j] = __float_as_uint(p[j]);
      psum[j] += p[j];
    }
    // top-k mass over the plan's choices (lanes take the ids in turn)
    float kp = 0.f;
    if (vt)
      for (int j = gl; j < k; j += G) {
        const int id = ids[(size_t)t * k + j];
        kp += expf(logits[(size_t)t * E + id] - m) / s;
      }
    const float kept = grp_sum_f<G>(kp);
    if (vt && gl == 0) atomicAdd(&sh_c[ids[(size_t)t * k]], 1);
    // threshold search: p <= 1, so bits 30 and 31 of tau stay clear
    uint32_t tau = 0u;
    for (int b = 29; b >= 0; --b) {
      const uint32_t cand = tau | (1u << b);
      float ms = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) ms += pb[j] >= cand ? p[j] : 0.f;
      if (grp_sum_f<G>(ms) >= 0.9f) tau = cand;
    }
    float mg = 0.f;
    int cg = 0, ceq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool gt = ve[j] && pb[j] > tau;
      mg += gt ? p[j] : 0.f;
      cg += gt ? 1 : 0;
      ceq += (ve[j] && pb[j] == tau) ? 1 : 0;
    }
    const float mgt = grp_sum_f<G>(mg);
    const int cgt = grp_sum_i<G>(cg);
    const int neq = grp_sum_i<G>(ceq);
    const float ptau = __uint_as_float(tau);
    int want = cgt + 1;
    while (want < cgt + neq && mgt + (float)(want - cgt) * ptau < 0.9f) ++want;
    if (vt) {
      if (want_out && gl == 0) want_out[t] = want;
      a_kept += kept;
      a_want += (float)want;
      a_z += lse * lse;
    }
  }
  // the wave's groups in group order, then the block's waves in wave order
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kGroups; ++q) v += __shfl(psum[j], gl + G * q);
    const int e = gl + G * j;
    if (grp == 0 && e < E) sh_p[wave][e] = v;
  }
  float wk = 0.f, ww = 0.f, wz = 0.f;
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    wk += __shfl(a_kept, G * q);
    ww += __shfl(a_want, G * q);
    wz += __shfl(a_z, G * q);
  }
  if (lane == 0) { sh_s[wave][0] = wk; sh_s[wave][1] = ww; sh_s[wave][2] = wz; }
  __syncthreads();
  // the block's sums per expert go into the cross-block totals as 2^-40
  // fixed-point integers: integer adds give the same total in any order
  for (int e = threadIdx.x; e < E; e += 256) {
    const float v = ((sh_p[0][e] + sh_p[1][e]) + sh_p[2][e]) + sh_p[3][e];
    const unsigned long long f = __double2ull_rn((double)v * 1099511627776.0);
    if (f) atomicAdd(&acc_p[e], f);
    if (sh_c[e]) atomicAdd(&acc_c[e], (uint32_t)sh_c[e]);
  }
  if (threadIdx.x < 3)
    part_s[blockIdx.x * 4 + threadIdx.x] =
        ((sh_s[0][threadIdx.x] + sh_s[1][threadIdx.x]) + sh_s[2][threadIdx.x]) +
        sh_s[3][threadIdx.x];
}

// The totals in double: balance from the per-expert totals, the means from
// the blocks' partials (each thread's share in block order, then a fixed
// tree). out = {kept mass, want_k, z loss, balance, aux, 0, 0, 0}, zeros for
// T == 0.
__global__ __launch_bounds__(1024) void router_final_kernel(
    const unsigned long long* __restrict__ acc_p,
    const uint32_t* __restrict__ acc_c, const float* __restrict__ part_s,
    int nblk, int T, int E, float z_weight, float* __restrict__ out) {
  __shared__ double sh[4][1024];
  const int tid = threadIdx.x;
  double bal = 0.0, sk = 0.0, sw = 0.0, sz = 0.0;
  if (T > 0) {
    for (int e = tid; e < E; e += 1024)
      bal += (double)acc_c[e] * ((double)acc_p[e] * 0x1p-40);
    for (int b = tid; b < nblk; b += 1024) {
      sk += (double)part_s[b * 4 + 0];
      sw += (double)part_s[b * 4 + 1];
      sz += (double)part_s[b * 4 + 2];
    }
  }
  sh[0][tid] = bal; sh[1][tid] = sk; sh[2][tid] = sw; sh[3][tid] = sz;
  __syncthreads();
  for (int h = 512; h >= 1; h >>= 1) {
    if (tid < h)
#pragma unroll
      for (int q = 0; q < 4; ++q) sh[q][tid] += sh[q][tid + h];
    __syncthreads();
  }
  if (tid < 8) {
    float v = 0.f;
    if (T > 0) {
      const double inv = 1.0 / (double)T;
      const double z = sh[3][0] * inv;
      const double b = (double)E * sh[0][0] * inv * inv;
      if (tid == 0) v = (float)(sh[1][0] * inv);
      if (tid == 1) v = (float)(sh[2][0] * inv);
      if (tid == 2) v = (float)z;
      if (tid == 3) v = (float)b;
      if (tid == 4) v = (float)(b + (double)z_weight * z);
    }
    out[tid] = v;
  }
}

// ---- launchers ------------------------------------------------------------

// Statistics scratch: acc_p [E] u64, acc_c [E] u32 (cleared by the router
// kernel), part_s [nblk][4] f32.
struct StatLayout { size_t acc_c, part_s, zero_words, bytes; };
StatLayout stat_layout(int T, int E) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t nblk = (size_t)(T + kStatTok - 1) / kStatTok;
  StatLayout L;
  L.acc_c = al((size_t)E * 8);
  L.part_s = L.acc_c + al((size_t)E * 4);
  L.zero_words = (L.acc_c + (size_t)E * 4) / 4;
  L.bytes = L.part_s + al(nblk * 16);
  return L;
}

size_t router_scratch_bytes(int T, int E) { return stat_layout(T, E).bytes; }

hipError_t launch_router_gemm(const void* x, int xdt, const void* w,
                              float* logits, int T, int D, int E,
                              void* scratch, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  uint32_t* zero = static_cast<uint32_t*>(scratch);
  const int zw = scratch ? (int)stat_layout(T, E).zero_words : 0;
  const bool mfma_ok = xdt != MOE_F32 && D % kRBK == 0 && T > kRouterDotT;
  if (mfma_ok) {
    const int64_t big = (int64_t)((T + 127) / 128) * ((E + 127) / 128);
    if (big >= kRouterBigTiles && D % 64 == 0) {
      const int grid = (int)big;
      if (xdt == MOE_F16)
        hipLaunchKernelGGL((router_mfma8_kernel<RF16, 4>), dim3(grid), dim3(512), 0, s,
                           x, w, logits, T, D, E, zero, zw);
      else
        hipLaunchKernelGGL((router_mfma8_kernel<RBF16, 4>), dim3(grid), dim3(512), 0, s,
                           x, w, logits, T, D, E, zero, zw);
    } else {
      const int grid = ((T + 63) / 64) * ((E + 63) / 64);
      if (xdt == MOE_F16)
        hipLaunchKernelGGL((router_mfma_kernel<RF16, 64, 64, kRNS>), dim3(grid), dim3(256), 0, s,
                           x, w, logits, T, D, E, zero, zw);
      else
        hipLaunchKernelGGL((router_mfma_kernel<RBF16, 64, 64, kRNS>), dim3(grid), dim3(256), 0, s,
                           x, w, logits, T, D, E, zero, zw);
    }
    return hipGetLastError();
  }
  const dim3 grid((T + 7) / 8, (E + 3) / 4);
  if (xdt == MOE_F32)
    hipLaunchKernelGGL((router_dot_kernel<float, 8>), grid, dim3(256), 0, s,
                       (const float*)x, (const float*)w, logits, T, D, E, zero, zw);
  else if (xdt == MOE_F16)
    hipLaunchKernelGGL((router_dot_kernel<_Float16, 8>), grid, dim3(256), 0, s,
                       (const _Float16*)x, (const _Float16*)w, logits, T, D, E, zero, zw);
  else
    hipLaunchKernelGGL((router_dot_kernel<__bf16, 8>), grid, dim3(256), 0, s,
                       (const __bf16*)x, (const __bf16*)w, logits, T, D, E, zero, zw);
  return hipGetLastError();
}

hipError_t launch_router_stats(const float* logits, const int32_t* ids, int T,
                               int E, int k, int32_t* want_out, void* scratch,
                               float* stats, float z_weight, hipStream_t s) {
  const int nblk = (T + kStatTok - 1) / kStatTok;
  const StatLayout L = stat_layout(T, E);
  char* b = static_cast<char*>(scratch);
  unsigned long long* acc_p = reinterpret_cast<unsigned long long*>(b);
  uint32_t* acc_c = reinterpret_cast<uint32_t*>(b + L.acc_c);
  float* part_s = reinterpret_cast<float*>(b + L.part_s);
  if (nblk > 0) {
#define MOE_STATS(G_, PER_)                                                     \
  hipLaunchKernelGGL((router_stats_kernel<G_, PER_>), dim3(nblk), dim3(256), 0, \
                     s, logits, ids, T, E, k, want_out, acc_p, acc_c, part_s)
    if (E <= 64) MOE_STATS(16, 4);
    else if (E <= 128) MOE_STATS(16, 8);
    else if (E <= 256) MOE_STATS(16, 16);
    else if (E <= 512) MOE_STATS(64, 8);
    else MOE_STATS(64, 16);
#undef MOE_STATS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stats) {
    hipLaunchKernelGGL(router_final_kernel, dim3(1), dim3(1024), 0, s, acc_p,
                       acc_c, part_s, nblk, T, E, z_weight, stats);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace moe
