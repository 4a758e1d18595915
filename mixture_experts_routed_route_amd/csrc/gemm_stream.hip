// Stream tile: thin expert groups (at most 16 * RB pairs of one expert) on
// gfx950.
//
// What a thin group costs is one read of its expert's weights from HBM; the
// multiply is small. TensorFold PR #1607 ("What this changes") keeps such
// plans off the GEMM tile and on a K-parallel tile. Here the tile is built
// around the weight stream:
//
//  * Work units are (item, K-stage) pairs, item = (group, block of 128
//    weight rows: 64 gate + 64 up features, or 128 down rows). The units of
//    one launch are cut into equal contiguous runs, one per workgroup, so
//    every CU streams the same number of bytes whatever the item count.
//    An item cut by run boundaries leaves fp32 partial sums in the
//    workspace, one per run; per wave, each run then counts its arrival on
//    the item's counter, and the wave that arrives last adds the partials
//    in run order (deterministic: the same sums whoever arrives last) and
//    runs the epilogue, then zeroes the counter for the next launch. The
//    runs of one item may sit on different XCDs, whose L2s are not coherent
//    with each other: the partials are written and read with agent-scope
//    accesses (sc1: through to the coherent side of the L2s), and each wave
//    waits for its partial stores to complete before it counts. An
//    agent-scope release / acquire fence pair would do the same by writing
//    back and invalidating the whole L2 at every arrival, which cost more
//    than the separate fix-up launch it replaces.
//  * Each workgroup keeps an LDS ring of stages filled by direct-to-LDS
//    buffer loads (no register staging). A stage holds 128 weight rows of
//    256 contiguous bytes (128 bf16/fp16 values) and the group's 16 * RB
//    token rows. The ring is refilled NS - 1 stages ahead, across item
//    boundaries, so the stream does not drain between items.
//  * Rows in LDS are XOR-swizzled in 16-byte chunks so that the 16 rows an
//    MFMA operand read touches cover all 64 banks once.
//  * Wave w multiplies the 32 weight rows it loaded itself (16 gate + 16
//    up features, or 32 down rows) by the token rows with
//    v_mfma_f32_16x16x32. Gate and up of a feature land in matching
//    accumulators of one lane, so the clamped SwiGLU runs in the epilogue
//    (mini-AGI PR #4, minagi/pool.py, `experts()`; clamp from Strata PR
//    #4366, "Approach").
//  * Item descriptors and the wave's token rows come from scalar loads one
//    item ahead; the token rows of a gate/up group come from a table the
//    classify kernel fills.
//  * 4-bit experts do not come here: their thin groups are bound by the
//    decode arithmetic, not the stream, and take the register-streaming
//    split-K and wide tiles, which keep more waves per CU (a variant of
//    this tile that decodes the weights after they land in LDS, with two
//    or four workgroups per CU, ran 14-30 % slower than those).
#include "device_common.h"

namespace moe {

namespace {

typedef const __attribute__((address_space(4))) int32_t* sconst_i32;

// Fewest units a run takes (the short prompts ran 2-8 % faster with 2 than
// with 4 or 8: their 17..64-row launches hold a few hundred units)
constexpr int kStreamMinUnits = 2;

constexpr int kLdsBytes = 163840;

// Stage geometry: K step 128, 256-byte weight rows; token rows of 256 B,
// loaded 4 rows per 1 KB instruction; a low plane of them for LO.
template <int RB, int LO> struct Geo {
  static constexpr int BK = 128, WB = 256;
  static constexpr int kW = 128 * WB;
  static constexpr int kArow = BK * 2;
  static constexpr int kA = 16 * RB * kArow;          // one plane
  static constexpr int kAPlanes = LO ? 2 : 1;
  static constexpr int kStage = kW + kA * kAPlanes;
  static constexpr int NS = kStage * 4 <= kLdsBytes ? 4 : (kStage * 3 <= kLdsBytes ? 3 : 2);
  static constexpr int nW = 8, nA = RB;               // instructions per plane
  static constexpr int nI = nW + nA * kAPlanes;       // per wave per stage
};

template <int RB>
struct Item {
  int e, nb, nrows, pstart;
  int tok[4 * RB];   // gate/up: x rows of this wave's 4 RB token rows
};

template <int MODE, int RB>
__device__ __forceinline__ Item<RB> load_item(const GemmArgs& a, int item,
                                              int NNB, int wave) {
  const sconst_i32 L = (sconst_i32)a.list;
  const int g = item / NNB;
  Item<RB> it;
  it.e = L[4 * g];
  it.nrows = L[4 * g + 2];
  it.pstart = L[4 * g + 3];
  it.nb = item - g * NNB;
  if (MODE == 0) {
    const sconst_i32 tk = (sconst_i32)a.tok + kStreamTokRows * g + 4 * RB * wave;
#pragma unroll
    for (int i = 0; i < 4 * RB; ++i) it.tok[i] = tk[i];
  }
  return it;
}

// Epilogue of one item: accumulator r of lane l holds weight row
// 4 (l / 16) + r of the wave's 16-row block, token 16 rb + l % 16.
template <class S, int MODE, int RB>
__device__ __forceinline__ void stream_store(const GemmArgs& a,
                                             const floatx4 (&acc)[RB][2],
                                             int nb, int nrows, int pstart,
                                             int wave, int lane) {
  const int q = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = rb * 16 + (lane & 15);
    if (t >= nrows) continue;
    const size_t prow = (size_t)(pstart + t);
    if (MODE == 0) {
      typedef S s4 __attribute__((ext_vector_type(4)));
      const int f = nb * 64 + wave * 16 + q * 4;
      s4 hv, lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float h = swiglu(acc[rb][0][r], acc[rb][1][r], a.clamp);
        hv[r] = (S)h;
        lv[r] = (S)(h - (float)hv[r]);
      }
      *reinterpret_cast<s4*>(reinterpret_cast<S*>(a.out) + prow * a.out_ld + f) = hv;
      if (a.out2)
        *reinterpret_cast<s4*>(reinterpret_cast<S*>(a.out2) + prow * a.out_ld + f) = lv;
    } else {
      const int d = nb * 128 + wave * 32 + q * 4;
      using Y = typename YPairOf<S>::T;
      const size_t o = prow * a.out_ld + d;
      store_y4<Y>(a.out, o, acc[rb][0][0], acc[rb][0][1], acc[rb][0][2], acc[rb][0][3]);
      store_y4<Y>(a.out, o + 16, acc[rb][1][0], acc[rb][1][1], acc[rb][1][2], acc[rb][1][3]);
    }
  }
}

__device__ __forceinline__ int run_start(int U, int b, int G) {
  return (int)((int64_t)U * b / G);
}
// Partial sums cross XCDs: agent-scope stores and loads (sc1), which the
// L2s do not keep to themselves.
__device__ __forceinline__ void part_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float part_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// the two partial-sum slots of run b: 0 for an item the run starts in, 1
// for the item it ends in (when that is another one)
__device__ __forceinline__ float* part_slot(const GemmArgs& a, int b, int slot, int RB) {
  return a.part + ((size_t)b * 2 + slot) * (size_t)(kStreamSlotFloats1 * RB);
}
// the run holding unit u: largest b with run_start(b) <= u
__device__ __forceinline__ int run_of(int U, int u, int G) {
  return (int)(((int64_t)(u + 1) * G - 1) / U);
}

// The partial sums of item's runs j0 .. bl (this wave's share), added in
// run order, then the epilogue. Runs are read UR at a time, all loads
// before the first add (one round trip for UR runs, not one each).
template <class S, int MODE, int RB>
__device__ __forceinline__ void fixup_item(const GemmArgs& a, int U, int G,
                                           int item, int j0, int bl, int nb,
                                           int nrows, int pstart, int wave,
                                           int lane) {
  const int nk = a.K / 128;
  const int tid = wave * 64 + lane;
  floatx4 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    acc[rb][0] = acc[rb][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int UR = RB == 1 ? 8 : 4;
  for (int rn0 = j0; rn0 <= bl; rn0 += UR) {
    float v[UR][RB][8];
    bool live[UR];
#pragma unroll
    for (int q = 0; q < UR; ++q) {
      const int rn = min(rn0 + q, bl);
      const int s0 = run_start(U, rn, G);
      // past bl, or a run without units (a launch of more runs than units)
      live[q] = rn0 + q <= bl && s0 != run_start(U, rn + 1, G);
      // the run starts inside the item (slot 0) or before it (slot 1)
      const int slot = s0 / nk == item ? 0 : 1;
      const float* pp = part_slot(a, rn, slot, RB);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 8; ++r) v[q][rb][r] = part_load(pp + (rb * 8 + r) * 256 + tid);
    }
#pragma unroll
    for (int q = 0; q < UR; ++q) {
      if (!live[q]) continue;   // wave-uniform
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[rb][0][r] += v[q][rb][r];
          acc[rb][1][r] += v[q][rb][4 + r];
        }
    }
  }
  stream_store<S, MODE, RB>(a, acc, nb, nrows, pstart, wave, lane);
}

}  // namespace

template <class TT, int RB, int MODE, int LO>
__global__ __launch_bounds__(256, 1) void gemm_stream_kernel(GemmArgs a) {
  using S = typename TT::S;
  using V8 = typename TT::V8;
  using Gm = Geo<RB, LO>;
  constexpr int NS = Gm::NS;
  constexpr int kStage = Gm::kStage;
  constexpr int nI = Gm::nI;
  static_assert((NS - 1) * nI <= 63, "vmcnt holds at most 63 loads");
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, N = a.N;
  const int nk = K / Gm::BK;
  const int NNB = MODE == 0 ? N / 64 : N / 128;
  const int U = a.meta[a.meta_index] * NNB * nk;   // below 2^31 (host check)
  // runs of at least kStreamMinUnits units (fewer runs than workgroups when
  // the launch holds little work: every cut item's last run reads one
  // partial per run of the item)
  const int G = a.part ? min((int)gridDim.x, max(1, U / kStreamMinUnits)) : (int)gridDim.x;
  const int b = blockIdx.x;
  if (b >= G) return;   // whole block
  // a.part null: the launch has a workgroup for every item there can be,
  // and workgroup b takes item b whole (no partial sums, no fix-up)
  const int u0 = a.part ? run_start(U, b, G) : min(U, b * nk);
  const int u1 = a.part ? run_start(U, b + 1, G) : min(U, (b + 1) * nk);
  if (u0 >= u1) return;   // whole block
  const int first_item = u0 / nk;

  // lane offsets of the weight DMA (4 rows of 256 B per instruction), fixed
  // for the launch
  const uint32_t wrow_b = (uint32_t)K * 2u;   // weight row bytes
  uint32_t vw[Gm::nW];
#pragma unroll
  for (int jj = 0; jj < Gm::nW; ++jj) {
    const int rl = lane >> 4;
    const int c = (lane & 15) ^ ((jj * 4 + rl) & 15);
    vw[jj] = (uint32_t)rl * wrow_b + (uint32_t)c * 16u;
  }
  const uint32_t a_row_b = (uint32_t)a.a_ld * 2u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t ra2 = make_rsrc(LO ? a.A2 : a.A, a.a_bytes);

  // issue-side state
  int iss_item = -1, pf_item = -1;
  Item<RB> iss{}, pf{};
  __amdgpu_buffer_rsrc_t rw0 = ra, rw1 = ra;
  uint32_t va[Gm::nA];   // token-row lane offsets of the current item
  const int last_item = (u1 - 1) / nk;
  constexpr int kRowsPer = 4;   // token rows per 1 KB instruction

  auto set_item = [&](int item) {
    iss = (item == pf_item) ? pf : load_item<MODE, RB>(a, item, NNB, wave);
    iss_item = item;
    // one expert's matrix: N rows (F for gate/up, D for down)
    const size_t mat_b = (size_t)N * wrow_b;
    rw0 = make_rsrc((const char*)a.B0 + (size_t)iss.e * mat_b, (uint32_t)mat_b);
    rw1 = MODE == 0 ? make_rsrc((const char*)a.B1 + (size_t)iss.e * mat_b, (uint32_t)mat_b) : rw0;
    // token rows: instruction i of the wave covers rows kRowsPer i + rl of
    // its 4 RB; lane writes 16-byte chunk pc of its row
    const int rl = lane >> 4;
    const int pc = lane & 15;
#pragma unroll
    for (int i = 0; i < Gm::nA; ++i) {
      const int trow = 4 * RB * wave + kRowsPer * i + rl;   // row within the stage
      int arow;
      if (MODE == 0) {
        // this lane's row among the instruction's kRowsPer scalars, by masks
        // (an indexed pick would move the scalars to memory)
        int rlo = rl;
        asm volatile("" : "+v"(rlo));
        arow = 0;
#pragma unroll
        for (int s = 0; s < kRowsPer; ++s)
          arow |= iss.tok[kRowsPer * i + s] & -(int)(rlo == s);
      } else {
        arow = iss.pstart + min(trow, iss.nrows - 1);
      }
      va[i] = (uint32_t)arow * a_row_b + (uint32_t)(pc ^ (trow & 15)) * 16u;
    }
    if (item + 1 <= last_item) {
      pf = load_item<MODE, RB>(a, item + 1, NNB, wave);
      pf_item = item + 1;
    }
  };

  // DMA of unit v into ring slot sl
  auto issue = [&](int v, int sl) {
    const int item = v / nk;
    const int kt = v - item * nk;
    if (item != iss_item) set_item(item);
    char* st = smem + sl * kStage;
#pragma unroll
    for (int jj = 0; jj < Gm::nW; ++jj) {
      const int rowbase = MODE == 0 ? iss.nb * 64 + wave * 16 + (jj & 3) * 4
                                    : iss.nb * 128 + wave * 32 + jj * 4;
      const __amdgpu_buffer_rsrc_t r = (MODE == 0 && jj >= Gm::nW / 2) ? rw1 : rw0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(st + wave * 32 * Gm::WB + jj * 1024), 16, (int)vw[jj],
          (int)((uint32_t)rowbase * wrow_b + (uint32_t)kt * (uint32_t)Gm::WB), 0, 0);
    }
    // the wave's 4 RB token rows (and their low plane)
#pragma unroll
    for (int pl = 0; pl < Gm::kAPlanes; ++pl) {
#pragma unroll
      for (int i = 0; i < Gm::nA; ++i) {
        char* dst = st + Gm::kW + pl * Gm::kA +
                    (4 * RB * wave + kRowsPer * i) * Gm::kArow;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            pl ? ra2 : ra, (lds_ptr_t)dst, 16, (int)va[i],
            (int)((uint32_t)kt * (uint32_t)Gm::kArow), 0, 0);
      }
    }
  };

  const int r16 = lane & 15, q = lane >> 4;
  floatx4 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    acc[rb][0] = acc[rb][1] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int sl) {
    const char* Ws = smem + sl * kStage;
    const char* As = Ws + Gm::kW;
    const char* w0 = Ws + (wave * 32 + r16) * Gm::WB;
    const char* w1 = w0 + 16 * Gm::WB;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int pc = ((4 * s + q) ^ r16) * 16;
      const V8 wa = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(w0 + pc));
      const V8 wb = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(w1 + pc));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const char* ar = As + (rb * 16 + r16) * Gm::kArow + pc;
        const V8 bt = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(ar));
        acc[rb][0] = mfma16(wa, bt, acc[rb][0]);
        acc[rb][1] = mfma16(wb, bt, acc[rb][1]);
        if (LO) {
          const V8 bl = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(ar + Gm::kA));
          acc[rb][0] = mfma16(wa, bl, acc[rb][0]);
          acc[rb][1] = mfma16(wb, bl, acc[rb][1]);
        }
      }
    }
  };

  // prologue: NS - 1 units in flight
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(min(u0 + p, u1 - 1), p);

  int cmp_item = -1, c_nb = 0, c_nrows = 0, c_pstart = 0;
  int pend[2] = {-1, -1};   // cut items this run left partials of (slot 0, 1)
  for (int u = u0; u < u1; ++u) {
    const int j = u - u0;
    wait_vmcnt<(NS - 2) * nI>();    // unit u landed (this wave's share)
    __builtin_amdgcn_s_barrier();   // ... for every wave; slot (j-1) % NS free
    __builtin_amdgcn_sched_barrier(0);
    issue(min(u + NS - 1, u1 - 1), (j + NS - 1) % NS);
    const int item = u / nk;
    if (item != cmp_item) {
      const sconst_i32 Lc = (sconst_i32)a.list;
      const int g = item / NNB;
      cmp_item = item;
      c_nb = item - g * NNB;
      c_nrows = Lc[4 * g + 2];
      c_pstart = Lc[4 * g + 3];
    }
    compute(j % NS);
    const int kt = u - item * nk;
    if (kt == nk - 1 || u == u1 - 1) {
      const bool whole = item * nk >= u0 && (item + 1) * nk <= u1;
      if (whole) {
        stream_store<S, MODE, RB>(a, acc, c_nb, c_nrows, c_pstart, wave, lane);
      } else {
        float* pp = part_slot(a, b, item == first_item ? 0 : 1, RB);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            part_store(pp + (rb * 8 + r) * 256 + tid, acc[rb][0][r]);
            part_store(pp + (rb * 8 + 4 + r) * 256 + tid, acc[rb][1][r]);
          }
        pend[item == first_item ? 0 : 1] = item;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][0] = acc[rb][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();   // no direct-to-LDS write outlives the workgroup

  // Arrivals on the cut items, after the run (a fence drains every load in
  // flight, so none sits inside the stream). Runs j0 .. bl hold an item's
  // nk units, j0 the one holding its first unit: a cut item is the last
  // item of that run, so no two cut items share it. The counter of (j0,
  // wave) adds up the units each run did; the run whose units complete nk
  // arrives last.
  if (pend[0] >= 0 || pend[1] >= 0) {
    // the wait above also saw this wave's partial stores complete
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int item = pend[i];
      if (item < 0) continue;
      const int fu = item * nk;
      const int j0 = run_of(U, fu, G), bl = run_of(U, fu + nk - 1, G);
      const int mine = min(u1, fu + nk) - max(u0, fu);
      int32_t* cnt = a.fix + 4 * j0 + wave;
      int old = 0;
      if (lane == 0) old = atomicAdd(cnt, mine);
      old = __builtin_amdgcn_readfirstlane(old);
      if (old + mine != nk) continue;   // wave-uniform
      const sconst_i32 Lc = (sconst_i32)a.list;
      const int g = item / NNB;
      fixup_item<S, MODE, RB>(a, U, G, item, j0, bl, item - g * NNB,
                              Lc[4 * g + 2], Lc[4 * g + 3], wave, lane);
      if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

bool stream_supported(int mode, int K, int N, int wdt) {
  if (wdt != MOE_BF16 && wdt != MOE_F16) return false;
  if (K <= 0 || K % 128) return false;
  return mode == 0 ? (N % 64 == 0) : (N % 128 == 0);
}

template <class TT, int RB>
static hipError_t stream_launch(const GemmArgs& a, int grid, hipStream_t s) {
  if (a.mode == 0)
    hipLaunchKernelGGL((gemm_stream_kernel<TT, RB, 0, 0>), dim3(grid), dim3(256), 0, s, a);
  else if (a.A2)
    hipLaunchKernelGGL((gemm_stream_kernel<TT, RB, 1, 1>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<TT, RB, 1, 0>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

struct SF16 { using S = _Float16; using V8 = half8; };
struct SBF16 { using S = __bf16; using V8 = bf16x8; };

template <class TT>
static hipError_t stream_rb(const GemmArgs& a, int rows, int grid, hipStream_t s) {
  return rows <= 16 ? stream_launch<TT, 1>(a, grid, s)
                    : stream_launch<TT, 4>(a, grid, s);
}

hipError_t launch_gemm_stream(const GemmArgs& a, int xdt, int wdt, int rows,
                              int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (rows < 1 || rows > kStreamTokRows ||
      (a.part && (grid > stream_max_runs(rows <= 16 ? 1 : 4) ||
                  grid > kStreamMaxRuns || !a.fix)))
    return hipErrorInvalidValue;
  if (xdt == MOE_BF16 && wdt == MOE_BF16) return stream_rb<SBF16>(a, rows, grid, s);
  if (xdt == MOE_F16 && wdt == MOE_F16) return stream_rb<SF16>(a, rows, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
