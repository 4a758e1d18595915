// Weight gradients of the backward on gfx950, two workgroups per CU.
//
// For expert e with kept pairs pb .. pb + np of the plan, the gradient is
// C_e = A_e^T B_e summed over its pairs: A [P, M] and B [P, N] are per-pair
// rows (dW_gate / dW_up: A = [dG | dU], M = 2F, B = X_p, N = D; dW_down:
// A = dY, M = D, B = w H, N = F), so K is the pair index and both operands
// are read with K as their row index. Every expert's f32 gradient is
// written whole (zeros for an expert without pairs): the launch writes
// 3 E' D F x 4 bytes and is bound by HBM, and a tile's stores cannot overlap
// its own next loads (one in-order counter covers both). So each workgroup
// takes one 128 x 256 tile and ends: four waves of 64 x 128 each, a
// three-stage ring of 24 KB (72 KB of LDS), and two workgroups per CU, so
// one tile's K loop runs while the other's f32 rows drain to HBM.
//
// A stage holds 32 K rows of both operands, K-row-major (A: 256-byte rows of
// 128 values, B: 512-byte rows of 256), loaded by buffer_load ... lds, with
// 16-byte chunk c of K row k at c ^ 2 (k mod 4). The MFMA fragments come
// from the transposing LDS read (ds_read_b64_tr_b16: lane i of a 16-lane
// group names 4 values of K row i / 4, lane l receives column l of the
// group's 4 rows), in asm blocks that wait for their own reads (the
// compiler would wait for every LDS-DMA load in flight before each such
// read it issues itself). K rows past the expert's last pair load zeros (an
// offset past the buffer descriptor's range).
//
// Tiles go to XCDs in runs: run r = (expert, 256-column block), its M / 128
// row tiles consecutive on XCD r mod 8, so they share the block's B slice in
// that XCD's L2; runs follow the experts' order by pair count, most first.
#include "device_common.h"

namespace moe {

namespace {

struct WgBF16 { using V8 = bf16x8; };
struct WgF16 { using V8 = half8; };

constexpr int kWgM = 128, kWgN = 256, kWgK = 32;   // tile rows, columns, K a stage
constexpr int kWgNS = 3;                           // ring stages
constexpr int kWgRowA = kWgM * 2, kWgRowB = kWgN * 2;
constexpr int kWgStageA = kWgK * kWgRowA;          // 8 KB
constexpr int kWgStage = kWgStageA + kWgK * kWgRowB;   // 24 KB
constexpr int kWgDmaB = 4, kWgDmaA = 2;            // 1 KB loads a wave a stage

typedef short wg_v4i16 __attribute__((ext_vector_type(4)));
typedef short wg_v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) const char* wg_lds_cptr;

// The NF fragments of 32 columns c0 + 32 j of a K-row-major operand with
// rows of PITCH bytes, K step ks: two transposing reads each (K rows +0..3
// and +4..7 of the lane group's 8), one asm block that waits for them.
template <int NF, int PITCH, class V8>
__device__ __forceinline__ void wg_frags(const char* base, int c0, int ks, int lane,
                                         V8* out) {
  const int g = lane >> 4, i = lane & 15;
  const int kr = ks * 16 + (g >> 1) * 8 + (i >> 2);
  uint32_t ad[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int col = c0 + 32 * j + (g & 1) * 16 + (i & 3) * 4;
    const int boff = ((((col >> 3) ^ (2 * (kr & 3))) << 4) | ((col & 7) * 2));
    ad[j] = (uint32_t)(uintptr_t)(wg_lds_cptr)(base + kr * PITCH + boff);
  }
  wg_v4i16 r[2 * NF];
  // K rows +4..7 sit 4 PITCH bytes further: 2048 for the 512-byte rows of
  // B (four fragments), 1024 for the 256-byte rows of A (two)
  if constexpr (NF == 4) {
    static_assert(PITCH == 512, "B rows");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\tds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\tds_read_b64_tr_b16 %5, %10 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\tds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]),
          "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  } else {
    static_assert(NF == 2 && PITCH == 256, "A rows");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %4 offset:1024\n\t"
        "ds_read_b64_tr_b16 %2, %5\n\tds_read_b64_tr_b16 %3, %5 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1])
        : "memory");
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const wg_v8i16 v = {r[2 * j][0], r[2 * j][1], r[2 * j][2], r[2 * j][3],
                        r[2 * j + 1][0], r[2 * j + 1][1], r[2 * j + 1][2],
                        r[2 * j + 1][3]};
    out[j] = __builtin_bit_cast(V8, v);
  }
}

}  // namespace

template <class TT>
__global__ __launch_bounds__(256, 2) void wgrad_kernel(WgradArgs a) {
  using V8 = typename TT::V8;
  // the ring; the epilogue stages each wave's f32 rows in it
  __shared__ __attribute__((aligned(1024))) char smem[kWgNS * kWgStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;   // 64-row half, 128-column half
  const int tm = (a.M + kWgM - 1) / kWgM, tn = (a.N + kWgN - 1) / kWgN;
  const int n_items = a.n_exp * tm * tn;
  // block b: XCD b mod 8; rounds of 8 runs of tm tiles
  const int b = blockIdx.x;
  const int q = b >> 3;
  const int item = (q / tm) * 8 * tm + (b & 7) * tm + (q % tm);
  if (item >= n_items) return;   // block-uniform, before any barrier
  const int run = item / tm, mt = item - run * tm;
  const int er = run / tn, nt = run - er * tn;
  const int e = __builtin_amdgcn_readfirstlane(a.eord[er]);
  const int pb = __builtin_amdgcn_readfirstlane(a.offsets[e]);
  const int np = __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - pb;
  const int nk = (np + kWgK - 1) / kWgK;
  const int m0 = mt * kWgM, n0 = nt * kWgN;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.B, a.b_bytes);
  // this lane's K row and byte offset in each of its DMA blocks: B block
  // bi = 4 wave + jj holds K rows 2 bi, 2 bi + 1; A block ai = 2 wave + jj
  // K rows 4 ai .. 4 ai + 3; the lane loads chunk p ^ 2 (k mod 4) of row k
  int krow[kWgDmaB + kWgDmaA];
  uint32_t voff[kWgDmaB + kWgDmaA];
#pragma unroll
  for (int jj = 0; jj < kWgDmaB; ++jj) {
    const int kr = 2 * (wave * kWgDmaB + jj) + (lane >> 5);
    const int cl = (lane & 31) ^ (2 * (kr & 3));
    krow[jj] = kr;
    voff[jj] = ((uint32_t)(pb + kr) * (uint32_t)a.b_ld + (uint32_t)(n0 + cl * 8)) * 2u;
  }
#pragma unroll
  for (int jj = 0; jj < kWgDmaA; ++jj) {
    const int kr = 4 * (wave * kWgDmaA + jj) + (lane >> 4);
    const int cl = (lane & 15) ^ (2 * (kr & 3));
    krow[kWgDmaB + jj] = kr;
    voff[kWgDmaB + jj] = ((uint32_t)(pb + kr) * (uint32_t)a.a_ld + (uint32_t)(m0 + cl * 8)) * 2u;
  }
  // stage kt into its ring slot; past the last stage the last is read again
  // (its loads still count, so every wait below is a constant)
  auto issue = [&](int kt) {
    const int kc = min(kt, nk - 1);
    char* st = smem + (kt % kWgNS) * kWgStage;
#pragma unroll
    for (int jj = 0; jj < kWgDmaB + kWgDmaA; ++jj) {
      const bool isb = jj < kWgDmaB;
      uint32_t vo = voff[jj];
      if (kc * kWgK + krow[jj] >= np) vo = 0x80000000u;   // loads zeros
      const int soff = kc * kWgK * (isb ? a.b_ld : a.a_ld) * 2;
      char* dst = isb ? st + kWgStageA + (wave * kWgDmaB + jj) * 1024
                      : st + (wave * kWgDmaA + (jj - kWgDmaB)) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isb ? rb : ra, (lds_ptr_t)dst, 16,
                                               (int)vo, soff, 0, 0);
    }
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int wi = 0; wi < 4; ++wi)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[wi][t][r] = 0.f;

  if (nk > 0) {
    issue(0);
    issue(1);
    for (int kt = 0; kt < nk; ++kt) {
      // this wave's loads of stage kt have landed (kt + 1's may be in
      // flight); after the barrier every wave's have, and every wave is
      // past its reads of stage kt - 1, whose slot the refill takes
      wait_vmcnt<kWgDmaB + kWgDmaA>();
      __builtin_amdgcn_s_barrier();
      issue(kt + kWgNS - 1);
      const char* st = smem + (kt % kWgNS) * kWgStage;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        V8 fb[4], fa[2];
        wg_frags<4, kWgRowB>(st + kWgStageA, wn * 128, ks, lane, fb);
        wg_frags<2, kWgRowA>(st, wm * 64, ks, lane, fa);
#pragma unroll
        for (int wi = 0; wi < 4; ++wi)
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[wi][t] = mfma32(fb[wi], fa[t], acc[wi][t]);
      }
    }
    wait_vmcnt<0>();
  }

  // f32 rows through LDS: each 32-row block of the wave's rows (32 x 128
  // outputs, 16 KB) is staged row-major in the wave's 16 KB of the ring,
  // 16-byte chunk c of row r at c ^ (r & 7), then written as whole
  // 512-byte row segments, two rows a store. Accumulator r of a 32x32
  // block is output column 8 (r / 4) + 4 (lane / 32) + r % 4 of the block,
  // row lane % 32.
  __builtin_amdgcn_s_barrier();   // every wave is done with the ring
  char* stg = smem + wave * 16384;
  const int jt = lane & 31, hi4 = (lane >> 5) * 4;
  const int c = lane & 31;
  const int col = n0 + wn * 128 + c * 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int wi = 0; wi < 4; ++wi)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int ch = wi * 8 + rq * 2 + (hi4 >> 2);
        *reinterpret_cast<float4*>(stg + jt * 512 + ((ch ^ (jt & 7)) << 4)) =
            float4{acc[wi][t][rq * 4 + 0], acc[wi][t][rq * 4 + 1],
                   acc[wi][t][rq * 4 + 2], acc[wi][t][rq * 4 + 3]};
      }
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int r = it * 2 + (lane >> 5);
      const float4 v = *reinterpret_cast<const float4*>(stg + r * 512 + ((c ^ (r & 7)) << 4));
      const int gm = m0 + wm * 64 + t * 32 + r;
      if (gm >= a.M || col >= a.N) continue;
      const bool lo = gm < a.row_split;
      float* dst = (lo ? a.out : a.out2) + (size_t)e * a.out_estride;
      // nontemporal: whole 128-byte lines, written once, read by no kernel
      // of the backward
      typedef float wg_f4 __attribute__((ext_vector_type(4)));
      const wg_f4 vv = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(
          vv, reinterpret_cast<wg_f4*>(dst + (size_t)(lo ? gm : gm - a.row_split) * a.N + col));
    }
  }
}

int wgrad_grid(const WgradArgs& a) {
  const int tm = (a.M + kWgM - 1) / kWgM, tn = (a.N + kWgN - 1) / kWgN;
  const int64_t runs = (int64_t)a.n_exp * tn;
  return (int)(((runs + 7) / 8) * 8 * tm);
}

hipError_t launch_wgrad(const WgradArgs& a, int xdt, hipStream_t s) {
  const int grid = wgrad_grid(a);
  if (grid <= 0) return hipSuccess;
  if (xdt == MOE_BF16)
    hipLaunchKernelGGL((wgrad_kernel<WgBF16>), dim3(grid), dim3(256), 0, s, a);
  else if (xdt == MOE_F16)
    hipLaunchKernelGGL((wgrad_kernel<WgF16>), dim3(grid), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
