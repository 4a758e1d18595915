// Full MFMA tile of the routed MoE layer on gfx950 (experts holding many
// rows, and the dequantised-once fp16 copies of 4-bit fat experts).
//
// One block = 8 waves (two per SIMD) computes a 256 (weight rows) x 256
// (token rows) tile; each wave owns 128 weight rows x 64 token rows (128
// accumulator registers). K streams through a ring of four 32 KB LDS stages
// (32 K values each) that buffer_load ... lds fills directly (no register
// staging): every wave issues four 1 KB loads per stage, three stages run
// ahead of the MFMAs, and each lane picks the global 16-byte chunk that lands
// in the XOR-swizzled LDS slot the MFMA operand reads expect. Eight issuing
// waves keep more of these loads in flight per CU than four (a CU's LDS-DMA
// stream runs about a third faster), and the second wave on a SIMD issues
// MFMAs while the first waits. Waits are explicit counted vmcnt waits plus
// s_barrier, and LDS loads and fragment reads are interleaved with the MFMA
// stream (sched_group_barrier) so the matrix pipe is not left idle.
//
// The weight rows are the MFMA's A operand and the gathered token rows its B
// operand, so a lane's 32x32 accumulator holds 4 consecutive output features
// of one token per group of four registers: the epilogue writes 8-byte (H)
// and 16-byte (per-pair output) vectors. Gate/up tiles interleave 32-row
// blocks of W_gate and W_up over the same features, so g and u of one
// (feature, token) sit in matching accumulators of one lane and the clamped
// SwiGLU runs in the epilogue (mini-AGI PR #4, minagi/pool.py, `experts()`;
// clamp from Strata PR #4366, "Approach"). Tokens are gathered on load
// through the plan's pair list; no gathered copy of x is materialised.
//
// The backward's products run on the same tile:
//  MODE 2 (recompute) loads as MODE 0 and writes the raw f32 G and U of
//    every pair instead of the SwiGLU output;
//  MODE 4 (dH' = dY W_down) and MODE 5 (dX = [dG | dU] [W_gate; W_up]):
//    per-pair rows of A times weights read as [K, N] (N contiguous; MODE 5's
//    K runs over W_gate, then W_up).
// Their weights, read with the K index as the row index, are staged
// K-row-major, [32 K rows][256] of 512 bytes,
// 16-byte chunk c of K row k at c ^ 2 (k & 3), and its MFMA fragments are
// read with the transposing LDS read (ds_read_b64_tr_b16): lane i of a
// 16-lane group names 4 values of K row i / 4, lane l receives column l of
// the group's 4 rows. The f32 outputs of MODES 4 and 5, and MODE 1's f32
// per-pair outputs (16-bit layers other than fp16), are staged through LDS
// and stored as whole rows. (The backward's weight gradients run on their
// own kernel, gemm_wgrad.hip.)
//
// Work is persistent, one block per CU, items taken from per-XCD queues.
// Items are tiles of the classify kernel's largest-first list crossed with
// output-column blocks; within a round the items of one XCD (blocks b = x
// mod 8) are a contiguous run of a 4 x 8 (row tiles x column tiles)
// grouping, so the 32 blocks resident on an XCD share their A and B slices
// in its L2.
#include <type_traits>

#include "device_common.h"

namespace moe {

namespace {

typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) const char* lds_cptr_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct F16T { using S = _Float16; using V8 = half8; using V4 = half4v; };
struct BF16T { using S = __bf16; using V8 = bf16x8; using V4 = bf16x4; };

// 64-byte LDS rows (32 K values); 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 2) & 3): the 16 rows one MFMA operand read touches per phase
// cover all 64 banks, and a wave's 1 KB direct-to-LDS write is contiguous.
__device__ __forceinline__ int swz64(int r, int c) {
  return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}


constexpr int kBW = 256;   // weight rows per tile
constexpr int kBK = 32;    // K per LDS stage
constexpr int kNS = 4;     // LDS stages (kNS - 1 in flight)
constexpr int kRowB = kBK * 2;
constexpr int kStage = 512 * kRowB;   // 256 weight + 256 token rows
constexpr int kGM = 4;     // row tiles per schedule group
constexpr int kWaves = 8;
constexpr int kDmaPerWave = 32 / kWaves;   // 1 KB blocks per wave per stage
constexpr int kDmaEarly = kDmaPerWave / 2;  // of them issued before mid-stage

}  // namespace

template <class TT, int MODE, int LO>
__global__ __launch_bounds__(512, 1) void gemm_full_kernel(GemmArgs a) {
  using S = typename TT::S;
  using V8 = typename TT::V8;
  using V4 = typename TT::V4;
  // The ring (128 KB). The block's next work item is passed through its first word (one LDS
  // object: with a second one the compiler guards every fragment read with
  // a wait for all LDS-DMA loads in flight). That word is wave 0's epilogue
  // staging and ring slot 0: thread 0 writes it after wave 0's epilogue and
  // after every wave's loads have landed (the wait and barrier that end the
  // K loop), all waves read it after the next barrier, and the next item's
  // first loads are issued only after the barrier that follows.
  __shared__ __attribute__((aligned(1024))) char smem[kNS * kStage];
  int* const next_item = reinterpret_cast<int*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index in a scalar register: descriptors and LDS bases stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ww = wave >> 2, wt = wave & 3;   // weight half, token quarter
  const int K = a.K, N = a.N;
  const int nk = K / kBK;
  constexpr bool kGU = MODE == 0 || MODE == 2;   // W_gate / W_up rows interleaved
  constexpr bool kWIC = MODE >= 4;   // weight side staged K-row-major
  const int NNB = kGU ? N / 128 : (N + kBW - 1) / kBW;
  const int n_tiles = a.meta[a.meta_index];
  const int n_items = n_tiles * NNB;
  const int G = gridDim.x;
  // this lane's row within each of its wave's 16-row DMA blocks
  const int dma_r = lane >> 2;

  // Work queues, one per XCD (block b runs on XCD b mod 8): queue x holds,
  // round by round, the items the XCD-aware order gives XCD x (a round is G
  // items; within it the G / 8 items of one XCD are a contiguous run of the
  // 4 x 8 grouping below), and each block takes the next item of its own
  // queue with an atomic counter. Blocks that run fast take more items; a
  // block whose queue is empty takes from the other XCDs' queues, so the
  // launch ends when the work does, not when the slowest block's static
  // share does. The counter for a block's next item is bumped before the
  // current one's epilogue, whose arithmetic hides its latency.
  const bool byx = (G & 7) == 0;
  const int per = G >> 3;
  const int xq = byx ? (int)(blockIdx.x & 7) : 0;
  auto queue_item = [&](int x, int j) -> int {
    if (!byx) return j < n_items ? j : -1;
    const int r = j / per;
    if (r * G >= n_items) return -1;
    return xcd_item(r * G, (j - r * per) * 8 + x, G, n_items);
  };
  // items in queue x: its share of the full rounds and of the last one
  auto queue_size = [&](int x) -> int {
    const int full = n_items / G, R = n_items - full * G;
    return full * per + (R >> 3) + (x < (R & 7) ? 1 : 0);
  };
  auto take = [&](int j_own) -> int {   // thread 0 only
    int it = queue_item(xq, j_own);
    if (it >= 0 || !byx) return it;
    // own queue empty: read the other counters in one batch and bump only
    // those with items left (the last blocks of a launch then pay one
    // round trip, not seven atomics)
    int seen[8];
#pragma unroll
    for (int d = 1; d < 8; ++d)
      seen[d] = __hip_atomic_load(&a.queue[(xq + d) & 7], __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    for (int d = 1; d < 8 && it < 0; ++d) {
      const int x = (xq + d) & 7;
      if (seen[d] < queue_size(x)) it = queue_item(x, atomicAdd(&a.queue[x], 1));
    }
    return it;
  };
  if (n_items == 0) return;
  if (threadIdx.x == 0) *next_item = take(atomicAdd(&a.queue[xq], 1));
  wait_vm_lgkm0<63>();
  __builtin_amdgcn_s_barrier();
  int L = __builtin_amdgcn_readfirstlane(*next_item);

  // an opaque per-lane zero: with a uniform address the compiler turns the
  // atomic into a wave-aggregated one (a readfirstlane of the result right
  // after it, waited for on the spot)
  int zq = 0;
  asm volatile("" : "+v"(zq));
  while (L >= 0) {
    int j_next = 0, jn = 0;
    // 4 x 8 grouping of (row tiles x column blocks)
    const int group = L / (kGM * NNB);
    const int first = group * kGM;
    const int gm = min(kGM, n_tiles - first);
    const int within = L - first * NNB;
    const int ti_ = first + within % gm;
    const int nb = within / gm;

    // item descriptors through the scalar cache: vector loads here would
    // make the waits for them also drain the previous item's stores
    typedef const __attribute__((address_space(4))) int32_t* sconst_i32;
    const int e = ((sconst_i32)a.list)[2 * ti_];
    const int tile_row0 = ((sconst_i32)a.list)[2 * ti_ + 1];
    const int off = ((sconst_i32)a.offsets)[e];
    const int ne = ((sconst_i32)a.offsets)[e + 1] - off;
    const int slot = a.fat_slot ? ((sconst_i32)a.fat_slot)[e] : -1;
    const size_t eix = slot >= 0 ? (size_t)slot : (size_t)e;
    // caller weights are [N, K] rows of K; the fp16 fat copies are
    // k-block-major, [K / 32][N][32], so one stage's 256 (or 2 x 128) weight
    // rows are a single contiguous 16 KB (2 x 8 KB) slab
    const bool tiled = slot >= 0;
    const uint32_t mat_bytes = (uint32_t)N * (uint32_t)K * 2u;

    // waves 0..3 load the stage's 256 weight rows, waves 4..7 its token rows
    const bool w_wave = wave < kWaves / 2;
    __amdgpu_buffer_rsrc_t r_even, r_odd;   // descriptors of this wave's blocks
    if (kWIC && w_wave) {
      // MODE 4: W_down [K = D][N = F]; MODE 5: W_gate, W_up [F][N = D]
      const uint32_t wb = (uint32_t)(MODE == 5 ? K / 2 : K) * (uint32_t)N * 2u;
      r_even = make_rsrc((const char*)a.B0 + (size_t)e * wb, wb);
      r_odd = MODE == 5 ? make_rsrc((const char*)a.B1 + (size_t)e * wb, wb) : r_even;
    } else if (w_wave) {
      const char* b0 = (const char*)(slot >= 0 ? a.S0 : a.B0);
      r_even = make_rsrc(b0 + eix * mat_bytes, mat_bytes);
      if (kGU) {
        const char* b1 = (const char*)(slot >= 0 ? a.S1 : a.B1);
        r_odd = make_rsrc(b1 + eix * mat_bytes, mat_bytes);
      } else {
        r_odd = r_even;
      }
    } else {
      r_even = make_rsrc((LO && wave >= 6) ? a.A2 : a.A, a.a_bytes);   // 6, 7: lo rows
      r_odd = r_even;
    }

    // One pass over BT token rows of the tile: 256, or 128 for a tile of at
    // most 128 rows (half the MFMA work; waves 6 and 7 load nothing) and for
    // each of the two passes of a split-H tile (LOP: rows 128..255 of the
    // stage hold the low plane of the same 128 tokens).
    auto run = [&](auto bt_c, auto lo_c, int pass) {
      constexpr int BT = decltype(bt_c)::value;
      constexpr bool LOP = decltype(lo_c)::value;
      constexpr int TW = BT / 4;               // token rows per wave
      constexpr int TB = TW / 32;              // 32-row token blocks per wave
      const int row0 = tile_row0 + pass * BT;
      // This lane's row of DMA block jj is stage row 16 (4 wave + jj) + lane / 4;
      // it loads logical chunk (lane % 4) ^ ((row >> 2) & 3). The branches
      // are wave-uniform and sit outside the per-block loops, so a token
      // wave issues its four pair-list loads back to back and waits once.
      uint32_t voff[kDmaPerWave];
      // K-row-major weights: DMA block jj of weight wave w holds K rows 2b
      // and 2b + 1, b = 4 w + jj; the lane loads chunk (lane % 32) ^ 2 (k & 3)
      // of K row k = 2b + lane / 32
      auto ic_row = [&](int jj) { return 2 * ((wave & 3) * kDmaPerWave + jj) + (lane >> 5); };
      auto ic_col = [&](int jj) { return (((lane & 31) ^ (2 * (ic_row(jj) & 3))) * 8); };
      if (kWIC && w_wave) {
#pragma unroll
        for (int jj = 0; jj < kDmaPerWave; ++jj) {
          const int col = nb * kBW + ic_col(jj);
          voff[jj] = ((uint32_t)ic_row(jj) * (uint32_t)N + (uint32_t)col) * 2u;
        }
      } else if (w_wave) {
#pragma unroll
        for (int jj = 0; jj < kDmaPerWave; ++jj) {
          const int R = 16 * (wave * kDmaPerWave + jj) + dma_r;
          int row;
          if (kGU)   // 32-row blocks alternate W_gate / W_up
            row = nb * 128 + (R >> 7) * 64 + ((R >> 6) & 1) * 32 + (R & 31);
          else
            row = min(nb * kBW + R, N - 1);
          const uint32_t rowoff = tiled ? (uint32_t)row * (uint32_t)kRowB
                                        : (uint32_t)row * (uint32_t)K * 2u;
          voff[jj] = rowoff + (uint32_t)((lane & 3) ^ ((R >> 2) & 3)) * 16u;
        }
      } else {
        int prow[kDmaPerWave];
#pragma unroll
        for (int jj = 0; jj < kDmaPerWave; ++jj) {
          const int Rt = 16 * (wave * kDmaPerWave + jj) + dma_r - 256;
          const int rr = min(row0 + (Rt % BT), ne - 1);
          // x rows are gathered through the pair list; the SwiGLU output of
          // full-tile experts is k-block-major, pair rows in order
          prow[jj] = kGU ? a.pair_token[off + rr] : off + rr;
        }
#pragma unroll
        for (int jj = 0; jj < kDmaPerWave; ++jj) {
          const int R = 16 * (wave * kDmaPerWave + jj) + dma_r;
          // MODE 1: the k-block-major H; else rows of a_ld values
          const uint32_t rowoff = MODE == 1 ? (uint32_t)prow[jj] * (uint32_t)kRowB
                                            : (uint32_t)prow[jj] * (uint32_t)a.a_ld * 2u;
          voff[jj] = rowoff + (uint32_t)((lane & 3) ^ ((R >> 2) & 3)) * 16u;
        }
      }
      // bytes from one stage's slice of a row to the next stage's (K-row-
      // major operands: 32 rows further)
      const int s_step = (kWIC && w_wave) ? kBK * N * 2
                       : w_wave ? (tiled ? N * kRowB : kRowB)
                                : (MODE == 1 ? a.h_rows * kRowB : kRowB);
      // Refill of ring stage kt. Past the last stage the slice nk-1 is read
      // again (an L2 hit) into a buffer no one reads any more, so every
      // stage issues the same number of loads and every wait below is a
      // constant count.
      auto issue_one = [&](int kt, int jj) {
        if (!LOP && BT == 128 && wave >= 6) return;   // no rows 384..511
        char* base = smem + (kt % kNS) * kStage + wave * kDmaPerWave * 1024;
        const int kc = min(kt, nk - 1);
        int soff = kc * s_step;
        __amdgpu_buffer_rsrc_t rs = (kGU && ((jj >> 1) & 1)) ? r_odd : r_even;
        if (MODE == 5 && w_wave && kc * kBK >= (K >> 1)) {   // W_up's K rows
          rs = r_odd;
          soff = (kc * kBK - (K >> 1)) * N * 2;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_ptr_t)(base + jj * 1024), 16, (int)voff[jj], soff, 0, 0);
      };
      auto issue = [&](int kt) {
#pragma unroll
        for (int jj = 0; jj < kDmaPerWave; ++jj) issue_one(kt, jj);
      };

      floatx16 acc[4][TB];
#pragma unroll
      for (int wi = 0; wi < 4; ++wi)
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[wi][t][r] = 0.f;

      // operand fragments of one 16-deep K step (hi and, for LOP, lo planes)
      struct Frag { V8 w[4]; V8 t[TB]; V8 tl[LOP ? TB : 1]; };
      // the NF fragments of 32 columns c0 + 32 j (j < NF) of a K-row-major
      // operand, K step ks: per fragment two transposing reads (K rows +0..3
      // and +4..7 of the lane group's 8). In one asm block that waits for
      // them: the compiler would put a wait for every LDS-DMA load in flight
      // before each such read it issues itself.
      auto rd_ic = [&](const char* base, int c0, int ks, V8* out, auto nf_c) {
        constexpr int NF = decltype(nf_c)::value;
        const int g = lane >> 4, i = lane & 15;
        const int kr = ks * 16 + (g >> 1) * 8 + (i >> 2);
        uint32_t ad[NF];
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int col = c0 + 32 * j + (g & 1) * 16 + (i & 3) * 4;
          const int boff = ((((col >> 3) ^ (2 * (kr & 3))) << 4) | ((col & 7) * 2));
          ad[j] = (uint32_t)(uintptr_t)(lds_cptr_t)(base + kr * 512 + boff);
        }
        v4i16_t r[2 * NF];
        if constexpr (NF == 4) {
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
        } else if constexpr (NF == 2) {
          asm volatile(
              "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %4 offset:2048\n\t"
              "ds_read_b64_tr_b16 %2, %5\n\tds_read_b64_tr_b16 %3, %5 offset:2048\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
              : "v"(ad[0]), "v"(ad[1])
              : "memory");
        } else {
          static_assert(NF == 1, "1, 2 or 4 fragments");
          asm volatile(
              "ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:2048\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(r[0]), "=&v"(r[1])
              : "v"(ad[0])
              : "memory");
        }
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const v8i16_t v = {r[2 * j][0], r[2 * j][1], r[2 * j][2], r[2 * j][3],
                             r[2 * j + 1][0], r[2 * j + 1][1], r[2 * j + 1][2],
                             r[2 * j + 1][3]};
          out[j] = __builtin_bit_cast(V8, v);
        }
      };
      auto read_frag = [&](int kt, int ks, Frag& f) {
        const char* Ws = smem + (kt % kNS) * kStage;
        const char* Ts = Ws + kBW * kRowB;
        const int ch = ks * 2 + (lane >> 5);
        if constexpr (kWIC) rd_ic(Ws, ww * 128, ks, f.w, std::integral_constant<int, 4>{});
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          const int r = ww * 128 + wi * 32 + (lane & 31);
          if constexpr (!kWIC)
            f.w[wi] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(Ws + swz64(r, ch)));
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const int r = wt * TW + t * 32 + (lane & 31);
          f.t[t] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(Ts + swz64(r, ch)));
          if (LOP)
            f.tl[t] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(Ts + swz64(r + BT, ch)));
        }
      };
      // one fragment read of a step: pieces 0..3 weights, then tokens (hi,
      // lo interleaved for LOP)
      auto read_piece = [&](int kt, int ks, int idx, Frag& f) {
        const char* Ws = smem + (kt % kNS) * kStage;
        const char* Ts = Ws + kBW * kRowB;
        const int ch = ks * 2 + (lane >> 5);
        if (idx < 4) {
          const int r = ww * 128 + idx * 32 + (lane & 31);
          if constexpr (kWIC) {   // all four in the first piece
            if (idx == 0) rd_ic(Ws, ww * 128, ks, f.w, std::integral_constant<int, 4>{});
          } else {
            f.w[idx] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(Ws + swz64(r, ch)));
          }
        } else {
          const int j = idx - 4;
          const int t = LOP ? j >> 1 : j;
          const int r = wt * TW + t * 32 + (lane & 31);
          if (LOP && (j & 1))
            f.tl[t] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(Ts + swz64(r + BT, ch)));
          else
            f.t[t] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(Ts + swz64(r, ch)));
        }
      };
      auto mma = [&](const Frag& f) {
#pragma unroll
        for (int wi = 0; wi < 4; ++wi)
#pragma unroll
          for (int t = 0; t < TB; ++t) acc[wi][t] = mfma32(f.w[wi], f.t[t], acc[wi][t]);
        if (LOP) {
          // low plane of H: (hi + lo) W accumulated in f32
#pragma unroll
          for (int wi = 0; wi < 4; ++wi)
#pragma unroll
            for (int t = 0; t < TB; ++t) acc[wi][t] = mfma32(f.w[wi], f.tl[t], acc[wi][t]);
        }
      };

      // every wave is past its reads of the ring before it is refilled; the
      // previous pass's refills are done (their wait sits before its
      // epilogue), so only its stores may still be in flight: they drain
      // while the first stages load
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int s = 0; s < kNS - 1; ++s) issue(s);
      wait_vmcnt<(kNS - 2) * kDmaPerWave>();   // stage 0 landed
      __builtin_amdgcn_s_barrier();
      Frag f0, f1;
      read_frag(0, 0, f0);

      // Per stage kt (two 16-deep steps): refill the ring three stages
      // ahead, read step 1 while step 0 multiplies, then (once stage kt+1
      // has landed for every wave) read its step 0 while step 1 multiplies.
      // Every read of stage kt completes before the mid-stage barrier, so
      // the refill of its buffer at the next stage's top never races it.
      // MFMAs issue in order behind each other; loads placed between them
      // issue while the matrix pipe is busy instead of in a burst that
      // leaves it idle: MFMA, LDS read, MFMA, ring refill, ...
      constexpr int kMf = 4 * TB * (LOP ? 2 : 1);  // MFMAs per 16-deep step
      constexpr int kRd = 4 + TB * (LOP ? 2 : 1);  // fragment reads per step
      constexpr int kSl = kMf > kRd ? kMf : kRd;   // interleave slots
      static_assert(kRd >= kDmaPerWave, "one refill per fragment read at most");
      for (int kt = 0; kt < nk; ++kt) {
        // LDS writes of the refill and LDS reads keep source order (the
        // compiler cannot tell them apart), so alternate them here. Half of
        // the refill issues here, half after the mid-stage barrier: spread
        // thin, a refill that waits for a free load slot holds up fewer MFMAs
#pragma unroll
        for (int q = 0; q < kRd; ++q) {
          if (q < kDmaEarly) issue_one(kt + kNS - 1, q);
          read_piece(kt, 1, q, f1);
        }
        mma(f0);
#pragma unroll
        for (int q = 0; q < kSl; ++q) {
          if (q < kMf) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          if (q < kDmaEarly) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
          if (q < kRd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        __builtin_amdgcn_sched_barrier(0);
        // step-1 reads done, stage kt+1 landed for this wave (stage kt+2 and
        // the early half of kt+3 may be in flight); after the barrier, for
        // every wave (past the end: unread refill data)
        wait_vm_lgkm0<(kNS - 3) * kDmaPerWave + kDmaEarly>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int q = 0; q < kRd; ++q) {
          if (q < kDmaPerWave - kDmaEarly) issue_one(kt + kNS - 1, kDmaEarly + q);
          read_piece(kt + 1, 0, q, f0);
        }
        mma(f1);
#pragma unroll
        for (int q = 0; q < kSl; ++q) {
          if (q < kMf) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          if (q < kDmaPerWave - kDmaEarly)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
          if (q < kRd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // the refills issued past the last stage land before anything else
      // is issued, so the next pass's refills of the same ring slots are
      // ordered after them whatever order loads complete in
      wait_vmcnt<0>();
      // The counter for the block's next item is bumped here and read after
      // the epilogue's arithmetic, before its stores: the atomic is the only
      // load in flight then, so the compiler's wait for it costs nothing.
      if (pass == 0 && threadIdx.x == 0) j_next = atomicAdd(a.queue + xq + zq, 1);
      // epilogue: accumulator r of a 32x32 block is weight row
      // 8 (r / 4) + 4 (lane / 32) + r % 4, token column lane % 32
      // lane-derived epilogue values are defined here, after the K loop, so
      // their addresses are not hoisted above it (they would hold registers
      // the loop needs for operand fragments)
      int lane_e = lane;
      asm volatile("" : "+v"(lane_e));
      const int jt = lane_e & 31;
      const int hi4 = (lane_e >> 5) * 4;
      using Y = typename YPairOf<S>::T;
      if constexpr (MODE >= 4 || (MODE == 1 && sizeof(Y) == 4)) {
        // f32 rows through LDS: each 32-row block of the wave's
        // rows (32 x 128 outputs, 16 KB) is staged row-major in the wave's
        // 16 KB of the idle ring, 16-byte chunk c of row r at c ^ (r & 7)
        // (the 8 rows a write phase touches hit 8 different bank groups),
        // then written as whole 512-byte row segments, two rows a store
        __builtin_amdgcn_s_barrier();   // every wave is done with the ring
        char* stg = smem + wave * 16384;
        const int col0 = nb * kBW + ww * 128;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
#pragma unroll
          for (int wi = 0; wi < 4; ++wi)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int c = wi * 8 + rq * 2 + (hi4 >> 2);
              *reinterpret_cast<float4*>(stg + jt * 512 + ((c ^ (jt & 7)) << 4)) =
                  float4{acc[wi][t][rq * 4 + 0], acc[wi][t][rq * 4 + 1],
                         acc[wi][t][rq * 4 + 2], acc[wi][t][rq * 4 + 3]};
            }
          if (t == 0) {
            __builtin_amdgcn_sched_barrier(0);
            jn = __builtin_amdgcn_readfirstlane(j_next);
            __builtin_amdgcn_sched_barrier(0);
          }
          const int c = lane_e & 31;
          const int d = col0 + c * 4;
#pragma unroll 4
          for (int it = 0; it < 16; ++it) {
            const int r = it * 2 + (lane_e >> 5);
            const float4 v =
                *reinterpret_cast<const float4*>(stg + r * 512 + ((c ^ (r & 7)) << 4));
            const int trow_ = row0 + wt * TW + t * 32 + r;
            if (trow_ >= ne || d >= N) continue;
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) +
                                       (size_t)(off + trow_) * a.out_ld + d) = v;
          }
        }
      } else if constexpr (MODE == 0 || (MODE == 1 && sizeof(Y) == 2)) {
        // Through LDS: a lane holds 4 consecutive features of one token, so
        // stores straight from the accumulators would write 16 B to each of
        // 32 rows per instruction. Each wave stages its 64 tokens x (64
        // features, or 128 outputs) as 2-byte values in its own 16 KB of the
        // (now idle) ring, token-major with 8-byte chunks XOR-swizzled by
        // token, then stores whole 128 / 256-byte row segments.
        __builtin_amdgcn_s_barrier();   // every wave is done with the ring
        char* stg = smem + wave * 16384;
        constexpr int kRowB = MODE == 0 ? 128 : 256;     // staged bytes per token
        static_assert(TW * kRowB * (MODE == 0 ? 2 : 1) <= 16384, "staging fits");
        constexpr int kSwz = MODE == 0 ? 7 : 15;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const int tok = t * 32 + jt;
          const int sw = ((tok >> 1) & kSwz) << 1;
          if (MODE == 0) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
              for (int rq = 0; rq < 4; ++rq) {
                V4 hv, lv;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const float h = swiglu(acc[2 * p][t][rq * 4 + q],
                                         acc[2 * p + 1][t][rq * 4 + q], a.clamp);
                  hv[q] = (S)h;
                  lv[q] = (S)(h - (float)hv[q]);
                }
                const int pc = (p * 8 + rq * 2 + (hi4 >> 2)) ^ sw;
                *reinterpret_cast<V4*>(stg + tok * kRowB + pc * 8) = hv;
                if (a.out2) *reinterpret_cast<V4*>(stg + TW * kRowB + tok * kRowB + pc * 8) = lv;
              }
          } else {
#pragma unroll
            for (int wi = 0; wi < 4; ++wi)
#pragma unroll
              for (int rq = 0; rq < 4; ++rq) {
                typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                h4 v;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = (_Float16)acc[wi][t][rq * 4 + q];
                const int pc = (wi * 8 + rq * 2 + (hi4 >> 2)) ^ sw;
                *reinterpret_cast<h4*>(stg + tok * kRowB + pc * 8) = v;
              }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        jn = __builtin_amdgcn_readfirstlane(j_next);
        __builtin_amdgcn_sched_barrier(0);
        const int tok_base = row0 + wt * TW;
        if (MODE == 0) {
          // H of full-tile experts, k-block-major [F / 32][h_rows][32]: per
          // instruction 16 tokens x one 32-feature block = 1 KB contiguous
          const int rl = lane_e >> 2, jp = lane_e & 3;
          const int planes = a.out2 ? 2 : 1;
          for (int pl = 0; pl < planes; ++pl) {
            char* dst = reinterpret_cast<char*>(pl ? a.out2 : a.out);
#pragma unroll 4
            for (int it = 0; it < TW / 8; ++it) {
              const int kbl = it & 1;              // which 32 of the 64 features
              const int tok = (it >> 1) * 16 + rl;
              const int sw = ((tok >> 1) & kSwz) << 1;
              const int j = kbl * 4 + jp;          // 16-byte piece of the row
              const uint4 v = *reinterpret_cast<const uint4*>(
                  stg + pl * TW * kRowB + tok * kRowB + (((2 * j) ^ sw) * 8));
              if (tok_base + tok >= ne) continue;
              const size_t prow = (size_t)(off + tok_base + tok);
              const size_t kb = (size_t)((nb * 128 + ww * 64) / 32 + kbl);
              *reinterpret_cast<uint4*>(dst + ((kb * a.h_rows + prow) * 32) * sizeof(S) + jp * 16) = v;
            }
          }
        } else {
          // Ypair rows: 1 KB per instruction, 16 lanes per 256-byte row run
          const int rl = lane_e >> 4, jp = lane_e & 15;
          S* dst = reinterpret_cast<S*>(a.out);
#pragma unroll 4
          for (int it = 0; it < TW / 4; ++it) {
            const int tok = it * 4 + rl;
            const int sw = ((tok >> 1) & kSwz) << 1;
            const uint4 v = *reinterpret_cast<const uint4*>(
                stg + tok * kRowB + (((2 * jp) ^ sw) * 8));
            if (tok_base + tok >= ne) continue;
            const size_t prow = (size_t)(off + tok_base + tok);
            const int col = nb * kBW + ww * 128 + jp * 8;
            if (col >= N) continue;
            *reinterpret_cast<uint4*>(dst + prow * a.out_ld + col) = v;
          }
        }
      } else {
        jn = __builtin_amdgcn_readfirstlane(j_next);
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const int trow_ = row0 + wt * TW + t * 32 + jt;
          if (trow_ >= ne) continue;
          const size_t prow = (size_t)(off + trow_);
#pragma unroll
          for (int wi = 0; wi < 4; ++wi)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              if constexpr (MODE == 2) {
                // raw G (even 32-row blocks) and U (odd) of feature f, f32:
                // [G | U] rows of 2 N values
                const int f = nb * 128 + ww * 64 + (wi >> 1) * 32 + rq * 8 + hi4;
                store_y4<float>(a.out, prow * a.out_ld + f + ((wi & 1) ? N : 0),
                                acc[wi][t][rq * 4 + 0], acc[wi][t][rq * 4 + 1],
                                acc[wi][t][rq * 4 + 2], acc[wi][t][rq * 4 + 3]);
              } else {
                const int d = nb * kBW + ww * 128 + wi * 32 + rq * 8 + hi4;
                if (d >= N) continue;
                store_y4<Y>(a.out, prow * a.out_ld + d, acc[wi][t][rq * 4 + 0],
                            acc[wi][t][rq * 4 + 1], acc[wi][t][rq * 4 + 2],
                            acc[wi][t][rq * 4 + 3]);
              }
            }
        }
      }
    };
    if constexpr (LO) {
      run(std::integral_constant<int, 128>{}, std::true_type{}, 0);
      if (tile_row0 + 128 < ne) run(std::integral_constant<int, 128>{}, std::true_type{}, 1);
    } else if (ne - tile_row0 <= 128) {
      run(std::integral_constant<int, 128>{}, std::false_type{}, 0);
    } else {
      run(std::integral_constant<int, 256>{}, std::false_type{}, 0);
    }
    // every wave has read next_item before this item's first barrier
    if (threadIdx.x == 0) *next_item = take(jn);
    wait_vm_lgkm0<63>();
    __builtin_amdgcn_s_barrier();
    L = __builtin_amdgcn_readfirstlane(*next_item);
  }
}

hipError_t launch_gemm_full(const GemmArgs& a, int xdt, int grid,
                            hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (a.mode >= 2) {   // the backward's products
    const dim3 g(grid), b(kWaves * 64);
    if (xdt == MOE_F16) {
      switch (a.mode) {
        case 2: hipLaunchKernelGGL((gemm_full_kernel<F16T, 2, 0>), g, b, 0, s, a); break;
        case 4: hipLaunchKernelGGL((gemm_full_kernel<F16T, 4, 0>), g, b, 0, s, a); break;
        case 5: hipLaunchKernelGGL((gemm_full_kernel<F16T, 5, 0>), g, b, 0, s, a); break;
        default: return hipErrorInvalidValue;
      }
    } else if (xdt == MOE_BF16) {
      switch (a.mode) {
        case 2: hipLaunchKernelGGL((gemm_full_kernel<BF16T, 2, 0>), g, b, 0, s, a); break;
        case 4: hipLaunchKernelGGL((gemm_full_kernel<BF16T, 4, 0>), g, b, 0, s, a); break;
        case 5: hipLaunchKernelGGL((gemm_full_kernel<BF16T, 5, 0>), g, b, 0, s, a); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (xdt == MOE_F16) {
    if (a.mode == 0)
      hipLaunchKernelGGL((gemm_full_kernel<F16T, 0, 0>), dim3(grid), dim3(kWaves * 64), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_full_kernel<F16T, 1, 0>), dim3(grid), dim3(kWaves * 64), 0, s, a);
  } else if (xdt == MOE_BF16) {
    if (a.mode == 0)
      hipLaunchKernelGGL((gemm_full_kernel<BF16T, 0, 0>), dim3(grid), dim3(kWaves * 64), 0, s, a);
    else if (a.A2)
      hipLaunchKernelGGL((gemm_full_kernel<BF16T, 1, 1>), dim3(grid), dim3(kWaves * 64), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_full_kernel<BF16T, 1, 0>), dim3(grid), dim3(kWaves * 64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
