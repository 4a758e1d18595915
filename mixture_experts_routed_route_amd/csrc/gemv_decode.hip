// One-token calls (T = 1) on bf16 / fp16 layers and on 4-bit layers with
// fp16 activations, on gfx950.
//
// A single token's k choices are k distinct experts, each holding exactly
// one of its pairs, and only those experts' weights need to be read
// (mini-AGI PR #3, minagi/pool.py: the one-row case needs no per-expert
// counts; PR #4, minagi/pool.py: the one-character case is a single group
// of k experts with one assignment each). Every product of such a call is
// a matrix-vector product: one weight row against one activation row, so
// the matrix cores have nothing to tile and the call is the weight stream
// alone. The stream tile takes its items whole at this size, 128 weight
// rows a workgroup, which leaves most compute units idle (9 experts of
// F = 768 make 108 items); here every compute unit streams its share:
//
//  * gate/up: a workgroup takes (pair, 16 features); each wave the 8 rows
//    of 4 features (gate and up), every lane 16-byte pieces of all 8 rows
//    in flight at once, the activation row's matching pieces in registers;
//    the 8 dot products are reduced across the wave with 10 exchanges (each
//    step halves the values a lane carries), then the clamped SwiGLU
//    (mini-AGI PR #4, minagi/pool.py, `experts()`; clamp from Strata PR
//    #4366, "Approach") and the H store, as the tiles store it (one 16-bit
//    value, or the bf16 hi + lo pair).
//  * down + combine: a workgroup takes 8 output columns for every pair of
//    the token, one wave a pair (up to 16 waves), the pair's 8 rows in one
//    pass.
//    Each pair's expert output is stored to the pair buffer in its usual
//    type and kept in LDS; the workgroup then sums them in slot order with
//    the routing weights, the shared expert's last, in f32, rounded once to
//    y's dtype: the combine kernel's arithmetic, without its launch.
#include "device_common.h"

namespace moe {

namespace {

constexpr int kGvFB = 16;   // gate/up features per workgroup (4 a wave)
constexpr int kGvDB = 8;    // down columns per workgroup
constexpr int kGvSlots = 4; // 16-byte pieces a lane holds per row at once
constexpr int kGvSlotsD = 2;   // the same, down

template <class S> struct Vec8;
template <> struct Vec8<__bf16> { using T = bf16x8; };
template <> struct Vec8<_Float16> { using T = half8; };

template <class S>
__device__ __forceinline__ void to_f8(uint4 u, float (&f)[8]) {
  using V = typename Vec8<S>::T;
  const V v = __builtin_bit_cast(V, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
}

// 8 per-lane values -> lane l holds the wave's sum of value
// 4 b5 + 2 b4 + b3 (b_i = bit i of l): at each of the first three steps a
// lane keeps the half of its values its own bit selects, adds the other
// lane's copy of that half and passes on the other half; then the last
// three steps sum the one value left.
__device__ __forceinline__ float wave_sum8(const float (&v)[8], int lane) {
  float a[4], b[2];
  const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = h5 ? v[4 + i] : v[i];
    const float give = h5 ? v[i] : v[4 + i];
    a[i] = keep + __shfl_xor(give, 32);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = h4 ? a[2 + i] : a[i];
    const float give = h4 ? a[i] : a[2 + i];
    b[i] = keep + __shfl_xor(give, 16);
  }
  float c = (h3 ? b[1] : b[0]) + __shfl_xor(h3 ? b[0] : b[1], 8);
  c += __shfl_xor(c, 4);
  c += __shfl_xor(c, 2);
  c += __shfl_xor(c, 1);
  return c;
}

// the expert and pair row of slot j of the token (j == k: the shared expert)
__device__ __forceinline__ void pair_of(const GemvArgs& a, int j, int& e, int& p) {
  if (j < a.k) {
    e = a.ids[j];
    p = a.tok2pair[j];
  } else {
    e = a.E;
    p = a.offsets[a.E];
  }
}

template <class S>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(GemvArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nfb = a.F / kGvFB;
  const int j = blockIdx.x / nfb;
  const int f0 = (blockIdx.x - j * nfb) * kGvFB + wave * 4;
  int e, p;
  pair_of(a, j, e, p);
  if (p < 0) return;   // a dropped pair: no row
  const S* x = (const S*)a.x;
  const size_t mat = (size_t)a.F * a.D;
  const S* rows[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rows[r] = (const S*)a.wg + e * mat + (size_t)(f0 + r) * a.D;
    rows[4 + r] = (const S*)a.wu + e * mat + (size_t)(f0 + r) * a.D;
  }
  const int nch = a.D / 8;   // 16-byte pieces a row
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nch; c0 += 64 * kGvSlots) {
    uint4 wv[8][kGvSlots], xv[kGvSlots];
#pragma unroll
    for (int c = 0; c < kGvSlots; ++c) {
      const int ci = c0 + c * 64 + lane;
      const bool ok = ci < nch;
      xv[c] = ok ? ldg16(x + (size_t)ci * 8) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < 8; ++r)
        wv[r][c] = ok ? ldg16(rows[r] + (size_t)ci * 8) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < kGvSlots; ++c) {
      float xf[8];
      to_f8<S>(xv[c], xf);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float wf[8];
        to_f8<S>(wv[r][c], wf);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r] += wf[i] * xf[i];
      }
    }
  }
  // lane l: row 4 b5 + 2 b4 + b3; gate rows 0..3 on lanes with b5 = 0, the
  // up row of the same feature on lane l ^ 32
  const float v = wave_sum8(acc, lane);
  const float u = __shfl_xor(v, 32);
  if ((lane & 39) == 0) {   // lanes 0, 8, 16, 24: features f0 .. f0 + 3
    const int f = f0 + ((lane >> 3) & 3);
    const float h = swiglu(v, u, a.clamp);
    const S hv = (S)h;
    const size_t o = (size_t)p * a.h_ld + f;
    ((S*)a.h)[o] = hv;
    if (a.h2) ((S*)a.h2)[o] = (S)(h - (float)hv);
  }
}

// blockDim.x = 64 min(J, 16): wave w takes pairs w, w + waves, ...; each
// pair's 8 rows of the block's columns in one pass (all its loads in
// flight together), so one round trip of the weight stream per pair
template <class S, class Y, class O, bool LO>
__global__ __launch_bounds__(1024) void gemv_down_kernel(GemvArgs a) {
  extern __shared__ float ys[];   // [J][kGvDB]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int d0 = blockIdx.x * kGvDB;
  const int J = a.k + a.n_shared;
  const int nch = a.F / 8;
  const size_t mat = (size_t)a.D * a.F;
  const S* H = (const S*)a.h;
  const S* H2 = (const S*)a.h2;
  for (int j = wave; j < J; j += nw) {
    int e, p;
    pair_of(a, j, e, p);
    if (p < 0) continue;   // wave-uniform: a dropped pair
    const S* w0 = (const S*)a.wd + (size_t)e * mat + (size_t)d0 * a.F;
    const S* hp = H + (size_t)p * a.h_ld;
    const S* lp = LO ? H2 + (size_t)p * a.h_ld : nullptr;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nch; c0 += 64 * kGvSlotsD) {
      uint4 wv[8][kGvSlotsD], hv[kGvSlotsD], lv[kGvSlotsD];
#pragma unroll
      for (int c = 0; c < kGvSlotsD; ++c) {
        const int ci = c0 + c * 64 + lane;
        const bool ok = ci < nch;
        hv[c] = ok ? ldg16(hp + (size_t)ci * 8) : uint4{0u, 0u, 0u, 0u};
        if (LO) lv[c] = ok ? ldg16(lp + (size_t)ci * 8) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < 8; ++r)
          wv[r][c] = ok ? ldg16(w0 + (size_t)r * a.F + (size_t)ci * 8) : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < kGvSlotsD; ++c) {
        float hf[8];
        to_f8<S>(hv[c], hf);
        if (LO) {
          float lf[8];
          to_f8<S>(lv[c], lf);
#pragma unroll
          for (int i = 0; i < 8; ++i) hf[i] += lf[i];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          float wf[8];
          to_f8<S>(wv[r][c], wf);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[r] += wf[i] * hf[i];
        }
      }
    }
    const float v = wave_sum8(acc, lane);
    if ((lane & 7) == 0) {   // lane 8 r holds column d0 + r
      const int r = lane >> 3;
      const Y yv = (Y)v;
      ((Y*)a.ypair)[(size_t)p * a.D + d0 + r] = yv;
      ys[j * kGvDB + r] = (float)yv;
    }
  }
  __syncthreads();
  if (threadIdx.x < kGvDB) {
    const int c = threadIdx.x;
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j)
      if (a.tok2pair[j] >= 0) acc += ys[j * kGvDB + c] * a.w[j];
    if (a.n_shared) acc += ys[a.k * kGvDB + c];
    ((O*)a.y)[d0 + c] = (O)acc;
  }
}

template <class S, class Y, bool LO>
hipError_t down_launch(const GemvArgs& a, int ydt, hipStream_t s) {
  const int grid = a.D / kGvDB;
  const int J = a.k + a.n_shared;
  const int threads = 64 * (J < 16 ? J : 16);
  const size_t lds = (size_t)J * kGvDB * 4;
  if (ydt == MOE_F32)
    hipLaunchKernelGGL((gemv_down_kernel<S, Y, float, LO>), dim3(grid), dim3(threads), lds, s, a);
  else if (ydt == MOE_BF16)
    hipLaunchKernelGGL((gemv_down_kernel<S, Y, __bf16, LO>), dim3(grid), dim3(threads), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_down_kernel<S, Y, _Float16, LO>), dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}


// ---- 4-bit weights, fp16 activations -----------------------------------
//
// A 16-byte piece of a 4-bit weight row holds 32 consecutive K values: one
// parameter block of the signed and affine-32 formats, half a group of the
// affine-64 one. A lane decodes its pieces in registers to the values the
// thin tiles use (fp16_rne(q s), or q s + b rounded once: Strata PR #4366,
// "Approach", decodes a 4-bit expert's weights to FP16; the affine groups
// are TensorFold PR #1607's) and takes the dot products with the matching
// 32 values of the activation row two at a time, f32 accumulation
// (v_dot2_f32_f16). Same workgroup shapes as the 16-bit kernels.

constexpr int kGvSlotsQ = 1;    // pieces a lane holds per row at once, gate/up
constexpr int kGvSlotsQD = 1;   // the same, down

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// sum over the 32 values of one piece: decoded weights times x (4 x 16 B)
template <int FMT>
__device__ __forceinline__ float dot_piece_q4(uint4 wq, uint32_t prm,
                                              const uint4 (&xv)[4], float acc) {
  const uint32_t words[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half8 w8 = dequant_word_f<FMT>(words[i], prm);
    const half8 x8 = __builtin_bit_cast(half8, xv[i]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc = __builtin_amdgcn_fdot2(h2v{w8[2 * t], w8[2 * t + 1]},
                                   h2v{x8[2 * t], x8[2 * t + 1]}, acc, false);
  }
  return acc;
}

// the parameter word of piece ci (32 K values from 32 ci) of a row whose
// parameters start at prow
template <int FMT>
__device__ __forceinline__ uint32_t piece_param(const char* prow, int ci) {
  return q4p_block<FMT>(load_q4p<FMT, 1>(prow, ci * 32), 0);
}

template <int FMT>
__global__ __launch_bounds__(256) void gemv_gateup_q4_kernel(GemvArgs a) {
  using Q = Q4F<FMT>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nfb = a.F / kGvFB;
  const int j = blockIdx.x / nfb;
  const int f0 = (blockIdx.x - j * nfb) * kGvFB + wave * 4;
  int e, p;
  pair_of(a, j, e, p);
  if (p < 0) return;   // a dropped pair: no row
  const _Float16* x = (const _Float16*)a.x;
  const char* rows[8];
  const char* prms[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const size_t wrow = (size_t)e * a.F + f0 + (r & 3);
    const char* base = (const char*)(r < 4 ? a.wg : a.wu);
    const char* pbase = (const char*)(r < 4 ? a.wgs : a.wus);
    rows[r] = base + wrow * (size_t)(a.D / 2);
    prms[r] = pbase + wrow * (size_t)(a.D / Q::kGroup) * Q::kPB;
  }
  const int np = a.D / 32;   // pieces a row
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < np; c0 += 64 * kGvSlotsQ) {
    uint4 wv[8][kGvSlotsQ], xv[kGvSlotsQ][4];
    uint32_t pv[8][kGvSlotsQ];
#pragma unroll
    for (int c = 0; c < kGvSlotsQ; ++c) {
      const int ci = c0 + c * 64 + lane;
      const bool ok = ci < np;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        wv[r][c] = ok ? ldg16(rows[r] + (size_t)ci * 16) : uint4{0u, 0u, 0u, 0u};
        pv[r][c] = ok ? piece_param<FMT>(prms[r], ci) : 0u;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[c][i] = ok ? ldg16(x + (size_t)ci * 32 + 8 * i) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < kGvSlotsQ; ++c)
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = dot_piece_q4<FMT>(wv[r][c], pv[r][c], xv[c], acc[r]);
  }
  // lane l: row 4 b5 + 2 b4 + b3; gate rows 0..3 on lanes with b5 = 0, the
  // up row of the same feature on lane l ^ 32
  const float v = wave_sum8(acc, lane);
  const float u = __shfl_xor(v, 32);
  if ((lane & 39) == 0) {   // lanes 0, 8, 16, 24: features f0 .. f0 + 3
    const int f = f0 + ((lane >> 3) & 3);
    ((_Float16*)a.h)[(size_t)p * a.h_ld + f] = (_Float16)swiglu(v, u, a.clamp);
  }
}

// blockDim.x = 64 min(J, 16): wave w takes pairs w, w + waves, ...; the
// pair outputs are fp16 (the fp16 layer's pair buffer) and summed as the
// 16-bit down kernel sums them
template <int FMT, class O>
__global__ __launch_bounds__(1024) void gemv_down_q4_kernel(GemvArgs a) {
  using Q = Q4F<FMT>;
  extern __shared__ float ys[];   // [J][kGvDB]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int d0 = blockIdx.x * kGvDB;
  const int J = a.k + a.n_shared;
  const int np = a.F / 32;
  const _Float16* H = (const _Float16*)a.h;
  for (int j = wave; j < J; j += nw) {
    int e, p;
    pair_of(a, j, e, p);
    if (p < 0) continue;   // wave-uniform: a dropped pair
    const size_t wrow0 = (size_t)e * a.D + d0;
    const char* w0 = (const char*)a.wd + wrow0 * (size_t)(a.F / 2);
    const char* p0 = (const char*)a.wds + wrow0 * (size_t)(a.F / Q::kGroup) * Q::kPB;
    const _Float16* hp = H + (size_t)p * a.h_ld;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < np; c0 += 64 * kGvSlotsQD) {
      uint4 wv[8][kGvSlotsQD], hv[kGvSlotsQD][4];
      uint32_t pv[8][kGvSlotsQD];
#pragma unroll
      for (int c = 0; c < kGvSlotsQD; ++c) {
        const int ci = c0 + c * 64 + lane;
        const bool ok = ci < np;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          wv[r][c] = ok ? ldg16(w0 + (size_t)r * (a.F / 2) + (size_t)ci * 16)
                        : uint4{0u, 0u, 0u, 0u};
          pv[r][c] = ok ? piece_param<FMT>(p0 + (size_t)r * (a.F / Q::kGroup) * Q::kPB, ci)
                        : 0u;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hv[c][i] = ok ? ldg16(hp + (size_t)ci * 32 + 8 * i) : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < kGvSlotsQD; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = dot_piece_q4<FMT>(wv[r][c], pv[r][c], hv[c], acc[r]);
    }
    const float v = wave_sum8(acc, lane);
    if ((lane & 7) == 0) {   // lane 8 r holds column d0 + r
      const int r = lane >> 3;
      const _Float16 yv = (_Float16)v;
      ((_Float16*)a.ypair)[(size_t)p * a.D + d0 + r] = yv;
      ys[j * kGvDB + r] = (float)yv;
    }
  }
  __syncthreads();
  if (threadIdx.x < kGvDB) {
    const int c = threadIdx.x;
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j)
      if (a.tok2pair[j] >= 0) acc += ys[j * kGvDB + c] * a.w[j];
    if (a.n_shared) acc += ys[a.k * kGvDB + c];
    ((O*)a.y)[d0 + c] = (O)acc;
  }
}

template <int FMT>
hipError_t down_q4_launch(const GemvArgs& a, int ydt, hipStream_t s) {
  const int grid = a.D / kGvDB;
  const int J = a.k + a.n_shared;
  const int threads = 64 * (J < 16 ? J : 16);
  const size_t lds = (size_t)J * kGvDB * 4;
  if (ydt == MOE_F32)
    hipLaunchKernelGGL((gemv_down_q4_kernel<FMT, float>), dim3(grid), dim3(threads), lds, s, a);
  else if (ydt == MOE_BF16)
    hipLaunchKernelGGL((gemv_down_q4_kernel<FMT, __bf16>), dim3(grid), dim3(threads), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_down_q4_kernel<FMT, _Float16>), dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool gemv_supported(int D, int F, int k, int n_shared) {
  return D > 0 && F > 0 && D % kGvDB == 0 && F % kGvFB == 0 && D % 8 == 0 &&
         F % 8 == 0 && (size_t)(k + n_shared) * kGvDB * 4 <= 65536;
}

// 4-bit weights: K values in whole pieces of 32 (whole groups of 64 for
// the affine-64 format) along both products
bool gemv_q4_supported(int D, int F, int k, int n_shared, int fmt) {
  const int grp = fmt == 2 ? 64 : 32;
  return fmt >= 0 && fmt <= 2 && gemv_supported(D, F, k, n_shared) &&
         D % grp == 0 && F % grp == 0;
}

hipError_t launch_gemv_gateup(const GemvArgs& a, int xdt, hipStream_t s) {
  const int grid = (a.k + a.n_shared) * (a.F / kGvFB);
  if (a.fmt >= 0) {
    if (xdt != MOE_F16 || !gemv_q4_supported(a.D, a.F, a.k, a.n_shared, a.fmt))
      return hipErrorInvalidValue;
    if (a.fmt == 0)
      hipLaunchKernelGGL((gemv_gateup_q4_kernel<0>), dim3(grid), dim3(256), 0, s, a);
    else if (a.fmt == 1)
      hipLaunchKernelGGL((gemv_gateup_q4_kernel<1>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemv_gateup_q4_kernel<2>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (!gemv_supported(a.D, a.F, a.k, a.n_shared)) return hipErrorInvalidValue;
  if (xdt == MOE_BF16)
    hipLaunchKernelGGL((gemv_gateup_kernel<__bf16>), dim3(grid), dim3(256), 0, s, a);
  else if (xdt == MOE_F16)
    hipLaunchKernelGGL((gemv_gateup_kernel<_Float16>), dim3(grid), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemv_down(const GemvArgs& a, int xdt, int ydt, hipStream_t s) {
  if (a.fmt >= 0) {
    if (xdt != MOE_F16 || a.h2 || !gemv_q4_supported(a.D, a.F, a.k, a.n_shared, a.fmt))
      return hipErrorInvalidValue;
    if (a.fmt == 0) return down_q4_launch<0>(a, ydt, s);
    if (a.fmt == 1) return down_q4_launch<1>(a, ydt, s);
    return down_q4_launch<2>(a, ydt, s);
  }
  if (!gemv_supported(a.D, a.F, a.k, a.n_shared)) return hipErrorInvalidValue;
  // the pair buffer's type is the tiles': fp16 in an fp16 layer, else f32
  if (xdt == MOE_BF16)
    return a.h2 ? down_launch<__bf16, float, true>(a, ydt, s)
                : down_launch<__bf16, float, false>(a, ydt, s);
  if (xdt == MOE_F16 && !a.h2) return down_launch<_Float16, _Float16, false>(a, ydt, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
