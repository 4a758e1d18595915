// Wide fused-dequant tile for experts holding 17..64 rows of a prompt.
//
// For such an expert every output column is multiplied by the same few
// dozen gathered rows, so re-reading those rows per 64-column block (what the
// split-K tile does) costs several times the weight bytes. Here one block of
// 4 waves covers 256 output columns: the expert's rows (<= 64) are staged
// once per CK-deep K chunk in LDS by direct-to-LDS loads and shared by the
// four waves, while each wave streams its own 64 weight rows from HBM
// chunks ahead and, for 4-bit weights, dequantises them in registers (the
// fused-dequant tiles the Strata PR #4366 route description leaves to the
// experts under the fat-row threshold). CK = 256 when K allows: the four
// lanes of a weight row then read its whole 128-byte line per chunk (with
// CK = 128 a chunk reads half a line and the other half comes a chunk later,
// from L2 if it is still there).
//
// Lane (n = l % 16, q = l / 16) of v_mfma_f32_16x16x32 holds, for K sub-chunk
// i of a chunk, A/B values at k = (CK / 4) q + 8 i .. + 8, matched between
// operands. A row r of a chunk is 2 CK bytes in LDS with 16-byte chunk c at
// c ^ (r % 16), so the 16 rows of one operand read hit 16 distinct bank
// groups. Gate/up column blocks cb = 0..3 of a wave are W_gate f0.., W_up
// f0.., W_gate f0+16.., W_up f0+16.., f0 = 128 nb + 32 w.
#include <type_traits>

#include "device_common.h"

#ifndef WIDE_OCC
#define WIDE_OCC 2
#endif

namespace moe {

namespace {


struct WF16 { using S = _Float16; using V8 = half8; };
struct WBF16 { using S = __bf16; using V8 = bf16x8; };

constexpr int kRowsW = 64;              // token rows per item (4 blocks of 16)

// Chunk geometry: CK = 128 keeps three chunks in flight (A two ahead in LDS,
// weights three ahead in registers), CK = 256 two (same LDS: 64 KB a block).
template <int CK> struct WGeo {
  static constexpr int kChunkB = kRowsW * CK * 2;   // LDS bytes per chunk
  static constexpr int kN = CK == 128 ? 3 : 2;      // chunks in flight (A and W)
  static constexpr int kSl = CK / 32;               // 32-deep MFMA slices
  static constexpr int kAi = kChunkB / 1024 / 4;    // A loads per wave per chunk
  static constexpr int kRowB = CK * 2;              // bytes of an A row
};

}  // namespace

// Weight operand of one chunk for one lane: 4 column blocks, CK / 4 values
// each (4-bit: CK / 128 16-byte pieces and the one or two block scales).
template <int WQ, int CK>
struct WChunk;
template <int CK>
struct WChunk<1, CK> { uint4 q[4][CK / 128]; Q4P s[4]; };
template <int CK>
struct WChunk<0, CK> { uint4 d[4][CK / 32]; };

// FMT: the 4-bit format of the weights (signed with a scale per 32 values,
// or affine with a (scale, bias) word per 32 / 64 values)
template <class TT, int WQ, int MODE, int CK, int FMT>
__global__ __launch_bounds__(256, WIDE_OCC) void gemm_wide_kernel(GemmArgs a) {
  using S = typename TT::S;
  using V8 = typename TT::V8;
  using Gm = WGeo<CK>;
  constexpr int kChunkB = Gm::kChunkB, kN = Gm::kN, kSl = Gm::kSl;
  constexpr int kAi = Gm::kAi, kRowB = Gm::kRowB;
  __shared__ __attribute__((aligned(1024))) char smem[kN * kChunkB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int nch = K / CK;
  const int cols_per_item = MODE == 0 ? 128 : 256;      // features / outputs
  const int NNB = (N + cols_per_item - 1) / cols_per_item;
  const int n_items = a.meta[a.meta_index] * NNB;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.A, a.a_bytes);

  for (int rb0 = 0; rb0 < n_items; rb0 += gridDim.x) {
    // the column blocks of one group on one XCD (its rows stay in that L2)
    const int item = xcd_item(rb0, blockIdx.x, gridDim.x, n_items);
    if (item < 0) continue;
    const int g = item / NNB;
    const int nb = item - g * NNB;
    const int e = a.list[4 * g];
    const int nrows = a.list[4 * g + 2];
    // the group's first pair (offsets[e] + row0) and, for the gate/up
    // stage, its x rows (kStreamTokRows a group, clamped to its last row)
    // come from the group's entry and token table, not through the pair list
    const int pstart = a.list[4 * g + 3];

    // NRB: the row blocks of 16 that hold rows of the group (1..4); the
    // padding blocks' A rows are staged like the others but take no MFMAs
    auto item_body = [&](auto nrbc) {
      constexpr int NRB = decltype(nrbc)::value;
      // A staging: block of 16 x 1 KB per chunk, 4 per wave; lane writes row
      // 4 b + lane / 16 at physical chunk lane % 16 = logical (lane%16)^(row%16)
      constexpr int kLpr = kRowB / 16;          // lanes per A row in one 1 KB load
      constexpr int kRpi = 64 / kLpr;           // A rows per 1 KB load
      uint32_t aoff[kAi];
#pragma unroll
      for (int j = 0; j < kAi; ++j) {
        const int r = kRpi * (wave * kAi + j) + lane / kLpr;
        const uint32_t prow = MODE == 0
                                  ? (uint32_t)a.tok[(size_t)kStreamTokRows * g + r]
                                  : (uint32_t)(pstart + min(r, nrows - 1));
        const int c = (lane % kLpr) ^ (r & 15);
        aoff[j] = prow * (uint32_t)a.a_ld * 2u + (uint32_t)c * 16u;
      }
      // wave w stages the rows of row block w, so a wave past the group's
      // last row block stages nothing (no MFMA reads those rows). Its
      // weight registers are covered by the compiler's own waits; the
      // counted waits below only order the staged rows
      auto issue_a = [&](int ch) {
        if (wave >= NRB) return;
        char* base = smem + (ch % kN) * kChunkB + wave * kAi * 1024;
        const int soff = min(ch, nch - 1) * CK * 2;
#pragma unroll
        for (int j = 0; j < kAi; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_ptr_t)(base + j * 1024),
                                                   16, (int)aoff[j], soff, 0, 0);
      };

      // this wave's 4 weight rows-blocks (16 rows each)
      const int col0 = MODE == 0 ? nb * 128 + wave * 32 : nb * 256 + wave * 64;
      const bool active = col0 < N;       // wave-uniform
      const char* bp[4];
      const char* bsp[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        int row;
        const void* base;
        const void* sbase;
        if (MODE == 0) {
          row = min(col0 + (cb >> 1) * 16 + n, N - 1);
          base = (cb & 1) ? a.B1 : a.B0;
          sbase = (cb & 1) ? a.B1s : a.B0s;
        } else {
          row = min(col0 + cb * 16 + n, N - 1);
          base = a.B0;
          sbase = a.B0s;
        }
        const size_t wrow = (size_t)e * N + row;
        if (WQ) {
          bp[cb] = (const char*)base + wrow * (size_t)(K / 2);
          bsp[cb] = (const char*)sbase + wrow * (size_t)(K / Q4F<FMT>::kGroup) * Q4F<FMT>::kPB;
        } else {
          bp[cb] = (const char*)base + wrow * (size_t)K * 2;
          bsp[cb] = nullptr;
        }
      }
      // lane q takes the CK / 4 consecutive K values from k0
      auto load_w = [&](int ch, WChunk<WQ, CK>& w) {
        const int cc = min(ch, nch - 1);
        const int k0 = cc * CK + q * (CK / 4);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          if constexpr (WQ) {
#pragma unroll
            for (int h = 0; h < CK / 128; ++h) w.q[cb][h] = ldg16(bp[cb] + k0 / 2 + h * 16);
            w.s[cb] = load_q4p<FMT, CK / 128>(bsp[cb], k0);
          } else {
#pragma unroll
            for (int i = 0; i < kSl; ++i) w.d[cb][i] = ldg16(bp[cb] + (size_t)k0 * 2 + i * 16);
          }
        }
      };

      floatx4 acc[4][4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

      // per 32-value slice i: the NRB row blocks' A fragments, then each
      // column block's slice decoded just before its MFMAs (16 + 16 operand
      // registers instead of all 64 decoded values at once)
      auto compute = [&](int ch, const WChunk<WQ, CK>& w) {
        const char* As = smem + (ch % kN) * kChunkB;
#pragma unroll
        for (int i = 0; i < kSl; ++i) {
          V8 av[NRB];
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            const int r = rb * 16 + n;
            const int c = (q * kSl + i) ^ (r & 15);
            av[rb] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(As + r * kRowB + c * 16));
          }
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            V8 bv;
            if constexpr (WQ) {
              const uint4 wq = w.q[cb][i >> 2];
              const uint32_t word = (i & 3) == 0 ? wq.x : (i & 3) == 1 ? wq.y : (i & 3) == 2 ? wq.z : wq.w;
              // the lane's CK / 4 values span CK / 128 blocks of 32
              bv = __builtin_bit_cast(V8, dequant_word_f<FMT>(word, q4p_block<FMT>(w.s[cb], i >> 2)));
            } else {
              bv = __builtin_bit_cast(V8, w.d[cb][i]);
            }
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) acc[rb][cb] = mfma16(av[rb], bv, acc[rb][cb]);
          }
        }
      };

      // Ring of kN chunks: A kN - 1 chunks ahead in LDS, weights kN ahead in
      // registers. Issue order is W0 A0 W1 A1 .. W(kN - 1), then per step s:
      // A(s + kN - 1), compute(s), W(s + kN). vmcnt retires in order, and A(s)
      // was issued kN - 1 steps before step s, after W(s): at the top of step
      // s "A(s) landed" is "at most the kN - 1 weight chunks and kN - 2 A
      // chunks issued since outstanding", which retires W(s) too. The barrier
      // then publishes A(s) to all waves and frees the buffer A(s + kN - 1)
      // refills (last read by compute(s - 1), before this barrier). Past the
      // end, loads re-read the last chunk into buffers and slots no one reads.
      constexpr int kWvm = WQ ? 4 * (CK / 128) + 4 : 4 * kSl;   // weight loads per chunk per lane
      constexpr int kWait = (kN - 1) * kWvm + (kN - 2) * kAi;
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      WChunk<WQ, CK> wr[kN];
#pragma unroll
      for (int j = 0; j < kN; ++j) {
        load_w(j, wr[j]);
        __builtin_amdgcn_sched_barrier(0);
        if (j < kN - 1) issue_a(j);
        __builtin_amdgcn_sched_barrier(0);
      }
      auto step = [&](int ch, WChunk<WQ, CK>& w) {
        wait_vmcnt<kWait>();
        __builtin_amdgcn_s_barrier();
        issue_a(ch + kN - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (active && ch < nch) compute(ch, w);
        __builtin_amdgcn_sched_barrier(0);
        load_w(ch + kN, w);
        __builtin_amdgcn_sched_barrier(0);
      };
      // every path issues the same loads (steps past the end only load), so
      // the compiler's own waits agree with the counted ones
      const int nsteps = (nch + kN - 1) / kN * kN;
      for (int ch = 0; ch < nsteps; ch += kN) {
#pragma unroll
        for (int j = 0; j < kN; ++j) step(ch + j, wr[j]);
      }

      if (active) {
        // 16x16 accumulator r of lane l: row 4 (l / 16) + r, column l % 16
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rb * 16 + q * 4 + r;
            if (row >= nrows) continue;
            const size_t prow = (size_t)(pstart + row);
            if (MODE == 0) {
#pragma unroll
              for (int pr = 0; pr < 2; ++pr) {
                const int f = col0 + pr * 16 + n;
                const float h = swiglu(acc[rb][2 * pr][r], acc[rb][2 * pr + 1][r], a.clamp);
                const S hv = (S)h;
                reinterpret_cast<S*>(a.out)[prow * a.out_ld + f] = hv;
                if (a.out2) reinterpret_cast<S*>(a.out2)[prow * a.out_ld + f] = (S)(h - (float)hv);
              }
            } else {
#pragma unroll
              for (int cb = 0; cb < 4; ++cb) {
                const int d = col0 + cb * 16 + n;
                if (d < N)
                  store_y1<typename YPairOf<S>::T>(a.out, prow * a.out_ld + d, acc[rb][cb][r]);
              }
            }
          }
      }
    };
    const int nrb = (nrows + 15) >> 4;   // group-uniform
    if (nrb <= 1) item_body(std::integral_constant<int, 1>{});
    else if (nrb == 2) item_body(std::integral_constant<int, 2>{});
    else if (nrb == 3) item_body(std::integral_constant<int, 3>{});
    else item_body(std::integral_constant<int, 4>{});
  }
}

hipError_t launch_gemm_wide(const GemmArgs& a, int xdt, int wdt, int grid,
                            hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  // K is a multiple of 128 (the layer's D and F are)
#define MOE_WIDE(TT, WQ, CK, F_)                                                          \
  do {                                                                                    \
    if (a.mode == 0)                                                                      \
      hipLaunchKernelGGL((gemm_wide_kernel<TT, WQ, 0, CK, F_>), dim3(grid), dim3(256), 0, s, a); \
    else                                                                                  \
      hipLaunchKernelGGL((gemm_wide_kernel<TT, WQ, 1, CK, F_>), dim3(grid), dim3(256), 0, s, a); \
  } while (0)
#define MOE_WIDE_K(F_)                              \
  do {                                              \
    if (a.K % 256 == 0) MOE_WIDE(WF16, 1, 256, F_); \
    else MOE_WIDE(WF16, 1, 128, F_);                \
  } while (0)
  if (a.K % 128) return hipErrorInvalidValue;
  const int fmt = q4_fmt(wdt);
  if (xdt != MOE_F16 || fmt < 0) return hipErrorInvalidValue;   // 16-bit weights take the stream tile
  if (fmt == 0) MOE_WIDE_K(0);
  else if (fmt == 1) MOE_WIDE_K(1);
  else MOE_WIDE_K(2);
#undef MOE_WIDE_K
#undef MOE_WIDE
  return hipGetLastError();
}

}  // namespace moe
