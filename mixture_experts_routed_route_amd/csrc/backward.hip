// Backward pass of the routed MoE layer on gfx950: gradients of
// L = sum_t dy[t] . y[t] for x, the three expert weights, the routing
// weights and (through the renormalised top-k softmax) the logits. Every
// expert slot gets the sum over its kept pairs, whatever the dispatch -- the
// property mini-AGI PR #3's tests/test_dispatch.py checks.
//
// Per kept pair p = (token t, expert e, weight w) in the plan's expert-sorted
// order (a pair of the shared expert has w = 1):
//   X_p  = x[t]        dYu = dy[t]                  (compute dtype)
//   [G | U] = X_p [W_gate; W_up]^T      (f32, recomputed)
//   H    = silu(min(G, c)) clamp(U)     (compute dtype, as the forward)
//   dH'  = dYu W_down,  dH = w dH'      (f32)
//   dw_j = dH' . H  (= dy[t] . H W_down^T, the expert's output, regrouped:
//                    no product for the per-pair outputs is needed)
//   [dG | dU] = SwiGLU backward         (compute dtype)
//   dXp  = dG W_gate + dU W_up          dx[t] = sum over its pairs (fixed order)
//   dW_gate[e] = sum_p dG_p x_p^T,  dW_up[e] likewise,
//   dW_down[e] = sum_p dYu_p (w H_p)^T   (w H_p rounded to the compute dtype)
// The three per-pair products run on the forward's full tile (gemm_full.hip):
// 256 x 256 tiles of 8 waves on 32x32x16 MFMAs, operands streamed HBM -> LDS
// by buffer_load ... lds through a four-stage ring, persistent blocks fed
// from per-XCD work queues, the heaviest experts first. [G | U] gathers x's
// rows through the pair list as the forward does; dH' and dX read the
// weights as [K, N], staged K-row-major and read with the transposing LDS
// read; every f32 output row is stored whole. The weight gradients, whose
// reduction runs over the pairs, have their own kernel (gemm_wgrad.hip).
#include <algorithm>

#include "device_common.h"

namespace moe {

namespace {

struct BF16B { using S = __bf16; };
struct F16B { using S = _Float16; };

// ints of the work-queue block: the tile count at 0, three launches' eight
// counters from 8 on
constexpr int kBwdQueueInts = 32;

}  // namespace

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

// The work lists, one block of 1024 threads, the experts taken by pair
// count, most first (ties by index):
//  - eord, that order (the weight gradients' expert order);
//  - q[0] 256-row tiles (expert, first pair row) of the per-pair products
//    ([G | U], dH', dX) in the list tiles256;
//  - the work-queue counters, q[8 + 8 i .. 15 + 8 i] of launch i, zeroed.
__global__ __launch_bounds__(1024) void bwd_tiles_kernel(
    const int32_t* __restrict__ offsets, int n_exp,
    int32_t* __restrict__ tiles256, int32_t* __restrict__ q,
    int32_t* __restrict__ eord) {
  __shared__ int32_t cnt[kMaxExperts + 2];
  __shared__ int32_t s4[kMaxExperts + 2];
  __shared__ int32_t ord[kMaxExperts + 2];
  __shared__ int32_t wsum[17];
  const int tid = threadIdx.x;
  for (int e = tid; e < n_exp; e += blockDim.x) cnt[e] = offsets[e + 1] - offsets[e];
  __syncthreads();
  for (int e = tid; e < n_exp; e += blockDim.x) {
    const int c = cnt[e];
    int rank = 0;
    for (int f = 0; f < n_exp; ++f) rank += cnt[f] > c || (cnt[f] == c && f < e);
    ord[rank] = e;
    eord[rank] = e;
  }
  __syncthreads();
  for (int r = tid; r < n_exp; r += blockDim.x) s4[r] = (cnt[ord[r]] + 255) / 256;
  __syncthreads();
  const int n4 = block_scan_excl(s4, n_exp, wsum);
  if (tid < kBwdQueueInts) q[tid] = tid == 0 ? n4 : 0;
  for (int r = tid; r < n_exp; r += blockDim.x) {
    const int e = ord[r];
    for (int i = 0; i * 256 < cnt[e]; ++i) {
      tiles256[2 * (s4[r] + i)] = e;
      tiles256[2 * (s4[r] + i) + 1] = i * 256;
    }
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
// with the hardware's 2^x and reciprocal) rounded once to the compute dtype
// -- the plain one-value H of the forward; a bf16 forward that also carries
// H's low plane keeps about 16 bits, so its dW_down differs from this one by
// that one rounding -- then scaled by pair_w and rounded again for the
// dW_down product (Hw); dtw_p = dH'_p . H_p taken on the unrounded f32 H.
// One wave per pair: lanes over F four values at a time in a fixed stride,
// then a fixed butterfly for dtw_p.
template <class S>
__global__ __launch_bounds__(256) void bwd_swiglu_back_kernel(
    const float* __restrict__ GU, const float* __restrict__ dHu,
    const float* __restrict__ pair_w, const int32_t* __restrict__ offsets,
    int n_exp, int F, float c, S* __restrict__ dGU, S* __restrict__ Hw,
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
        oh[q] = (S)(w * (float)(S)hq);
        acc = fmaf(dv[q], hq, acc);
        float dg, du;
        swiglu_back1(gv[q], uv[q], w * dv[q], c, dg, du);
        og[q] = (S)dg;
        ou[q] = (S)du;
      }
      __builtin_memcpy(dGU + (size_t)p * 2 * F + f, og, 8);
      __builtin_memcpy(dGU + (size_t)p * 2 * F + F + f, ou, 8);
      __builtin_memcpy(Hw + (size_t)p * F + f, oh, 8);
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

namespace {
// byte size of each workspace region, in order
struct BwdLayout {
  size_t tiles256, q, eord, Xp, GU, Hw, dYu, dtwp, dH, dGU, dXp;
};
BwdLayout bwd_layout(int64_t Pmax, int n_exp, int D, int F) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t P = (size_t)Pmax;
  BwdLayout L;
  L.tiles256 = al(((P + 255) / 256 + n_exp + 1) * 8);
  L.q = al(kBwdQueueInts * 4);
  L.eord = al((size_t)n_exp * 4);
  L.Xp = al(P * D * 2);
  L.GU = al(P * 2 * F * 4);
  L.Hw = al(P * F * 2);
  L.dYu = al(P * D * 2);
  L.dtwp = al(P * 4);
  L.dH = al(P * F * 4);
  L.dGU = al(P * 2 * F * 2);
  L.dXp = al(P * D * 4);
  return L;
}
}  // namespace

size_t bwd_workspace_bytes(int64_t Pmax, int n_exp, int D, int F) {
  const BwdLayout L = bwd_layout(Pmax, n_exp, D, F);
  return L.tiles256 + L.q + L.eord + L.Xp + L.GU + L.Hw + L.dYu +
         L.dtwp + L.dH + L.dGU + L.dXp;
}

// stage 0: gather, recompute [G | U]; 1: dH', H, dG / dU and dtw_p, dXp,
// dx; 2: the weight gradients; 3: the routing-weight and logit gradients
template <class TT>
static hipError_t run_bwd(const BwdArgs& a, int stage, hipStream_t s) {
  using S = typename TT::S;
  const int64_t Pm = a.Pmax;
  const int D = a.D, F = a.F, n_exp = a.n_exp;
  const BwdLayout L = bwd_layout(Pm, n_exp, D, F);
  char* b = static_cast<char*>(a.ws);
  int32_t* tiles256 = reinterpret_cast<int32_t*>(b);  b += L.tiles256;
  int32_t* q = reinterpret_cast<int32_t*>(b);         b += L.q;
  int32_t* eord = reinterpret_cast<int32_t*>(b);      b += L.eord;
  S* Xp = reinterpret_cast<S*>(b);                    b += L.Xp;
  float* GU = reinterpret_cast<float*>(b);            b += L.GU;
  S* Hw = reinterpret_cast<S*>(b);                    b += L.Hw;
  S* dYu = reinterpret_cast<S*>(b);                   b += L.dYu;
  float* dtwp = reinterpret_cast<float*>(b);          b += L.dtwp;
  float* dH = reinterpret_cast<float*>(b);            b += L.dH;
  S* dGU = reinterpret_cast<S*>(b);                   b += L.dGU;
  float* dXp = reinterpret_cast<float*>(b);

  const int ew_grid = a.ncu * 8;
  const int64_t tile_cap = (Pm + 255) / 256 + n_exp + 1;
  // a per-pair product on the full tile over the 256-row pair tiles
  auto per_pair = [&](int mode, const void* A, int a_ld, int K, const void* B0,
                      const void* B1, int N, float* out, int out_ld, int qi) {
    GemmArgs g{};
    g.mode = mode; g.K = K; g.N = N;
    g.A = A; g.a_ld = a_ld;
    g.a_bytes = (uint32_t)(mode == 2 ? (size_t)a.T * D * 2 : (size_t)Pm * a_ld * 2);
    g.pair_token = a.pair_token; g.offsets = a.offsets; g.pair_w = a.pair_w;
    g.B0 = B0; g.B1 = B1; g.fat_slot = nullptr;
    g.out = out; g.out_ld = out_ld; g.clamp = a.clamp;
    g.list = tiles256; g.meta = q; g.meta_index = 0; g.queue = q + 8 + 8 * qi;
    const int64_t nnb = mode == 2 ? N / 128 : (N + 255) / 256;
    return launch_gemm_full(g, a.xdt, (int)std::min<int64_t>(tile_cap * nnb, a.ncu), s);
  };
  hipError_t e = hipSuccess;
  if (stage == 0) {
    hipLaunchKernelGGL(bwd_tiles_kernel, dim3(1), dim3(1024), 0, s, a.offsets,
                       n_exp, tiles256, q, eord);
    hipLaunchKernelGGL((bwd_gather_kernel<S>), dim3(ew_grid), dim3(256), 0, s,
                       (const S*)a.x, a.dy, a.pair_token, a.offsets,
                       n_exp, D, Xp, dYu);
    // [G | U] = X_p [W_gate; W_up]^T, x rows gathered through the pair list
    e = per_pair(2, a.x, D, D, a.wg, a.wu, F, GU, 2 * F, 0);
  } else if (stage == 1) {
    // dH' = dYu W_down (unscaled; the SwiGLU backward applies pair_w)
    e = per_pair(4, dYu, D, D, a.wd, nullptr, F, dH, F, 1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_swiglu_back_kernel<S>), dim3(ew_grid), dim3(256), 0, s,
                       GU, dH, a.pair_w, a.offsets, n_exp, F, a.clamp, dGU, Hw, dtwp);
    // dXp = [dG | dU] [W_gate; W_up]
    e = per_pair(5, dGU, 2 * F, 2 * F, a.wg, a.wu, D, dXp, D, 2);
    if (e != hipSuccess) return e;
    if (a.dx)
      hipLaunchKernelGGL(bwd_dx_kernel, dim3(ew_grid), dim3(256), 0, s, dXp,
                         a.tok2pair, a.offsets, a.T, a.k, D, a.n_shared, a.E, a.dx);
  } else if (stage == 2) {
    // weight gradients of every expert (no pairs: zeros), two 128 x 256
    // tiles a CU
    auto wgrad2 = [&](const S* A, int M, const S* B, int N, float* out,
                      float* out2, int row_split) {
      WgradArgs w{};
      w.A = A; w.a_bytes = (uint32_t)((size_t)Pm * M * 2); w.a_ld = M; w.M = M;
      w.B = B; w.b_bytes = (uint32_t)((size_t)Pm * N * 2); w.b_ld = N; w.N = N;
      w.offsets = a.offsets; w.eord = eord; w.n_exp = n_exp;
      w.out = out; w.out2 = out2; w.row_split = row_split;
      w.out_estride = (int64_t)row_split * N;
      return launch_wgrad(w, a.xdt, s);
    };
    e = wgrad2(dGU, 2 * F, Xp, D, a.dwg, a.dwu, F);
    if (e != hipSuccess) return e;
    e = wgrad2(dYu, D, Hw, F, a.dwd, a.dwd, D);
  } else if (a.dtw || a.dlogits) {
    float* dtw = a.dtw ? a.dtw : a.dtw_scratch;
    const int64_t nq = (int64_t)a.T * a.k;
    if (nq > 0)
      hipLaunchKernelGGL(bwd_dtw_kernel, dim3((unsigned)std::min<int64_t>((nq + 255) / 256, ew_grid)),
                         dim3(256), 0, s, dtwp, a.tok2pair, nq, dtw);
    if (a.dlogits && a.T > 0)
      hipLaunchKernelGGL(bwd_dlogits_kernel, dim3(a.T), dim3(256), 0, s, a.ids,
                         a.topk_w, dtw, a.T, a.E, a.k, a.dlogits);
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, int stage, hipStream_t s) {
  if (a.xdt == MOE_BF16) return run_bwd<BF16B>(a, stage, s);
  if (a.xdt == MOE_F16) return run_bwd<F16B>(a, stage, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
