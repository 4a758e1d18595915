// Stream tile: thin expert groups (at most 16 pairs of one expert) on gfx950.
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
//    An item cut by a run boundary leaves fp32 partial sums in the
//    workspace; a fix-up kernel adds them in run order (deterministic) and
//    runs the epilogue.
//  * Each workgroup keeps an LDS ring of stages filled by direct-to-LDS
//    buffer loads (no register staging). A stage holds 128 weight rows of
//    256 contiguous bytes (128 bf16/fp16 values, or 512 4-bit values plus
//    their 16 fp16 block scales per row) and the group's 16 token rows.
//    The ring is refilled NS - 1 stages ahead, across item boundaries, so
//    the stream does not drain between items.
//  * Rows in LDS are XOR-swizzled in 16-byte chunks (chunk c of row r sits
//    at c ^ (r % 16)): the 16 rows an MFMA operand read touches cover all
//    64 banks once.
//  * Wave w multiplies the 32 weight rows it loaded itself (16 gate + 16
//    up features, or 32 down rows) by the 16 token rows with
//    v_mfma_f32_16x16x32; 4-bit rows are decoded from LDS in registers.
//    Gate and up of a feature land in matching accumulators of one lane,
//    so the clamped SwiGLU runs in the epilogue (mini-AGI PR #4,
//    minagi/pool.py, `experts()`; clamp from Strata PR #4366, "Approach").
//  * Item descriptors come from scalar loads one item ahead; the token rows
//    of a gate/up group come from a table the classify kernel fills.
#include "device_common.h"

namespace moe {

namespace {

typedef const __attribute__((address_space(4))) int32_t* sconst_i32;

// Stage geometry. Dense: K step 128 (256-byte weight rows), token rows
// loaded as 4 x 256 B per wave (one row per instruction, 4-byte lanes).
// 4-bit: K step 512 (256-byte rows of nibbles) + 32 B of scales per row,
// token rows 1 KB each, one per instruction.
template <int WQ, int LO> struct Geo;
template <int LO> struct Geo<0, LO> {
  static constexpr int BK = 128, NS = 4;
  static constexpr int kW = 32768, kSc = 0, kA = 4096, kAPlanes = LO ? 2 : 1;
  static constexpr int nI = 8 + 4 * kAPlanes;   // DMA instructions / wave / stage
};
template <int LO> struct Geo<1, LO> {
  static constexpr int BK = 512, NS = 3;
  static constexpr int kW = 32768, kSc = 4096, kA = 16384, kAPlanes = 1;
  static constexpr int nI = 8 + 4 + 4;
};

struct Item {
  int e, nb, nrows, pstart;
  int tok[4];   // A rows of this wave's four token rows (clamped)
};

template <int MODE>
__device__ __forceinline__ Item load_item(const GemmArgs& a, int item, int NNB,
                                          int wave) {
  const sconst_i32 L = (sconst_i32)a.list;
  const int g = item / NNB;
  Item it;
  it.e = L[4 * g];
  it.nrows = L[4 * g + 2];
  it.pstart = L[4 * g + 3];
  it.nb = item - g * NNB;
  if (MODE == 0) {
    const sconst_i32 tk = (sconst_i32)a.tok;
#pragma unroll
    for (int i = 0; i < 4; ++i) it.tok[i] = tk[16 * g + 4 * wave + i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      it.tok[i] = it.pstart + min(4 * wave + i, it.nrows - 1);
  }
  return it;
}

// Epilogue of one item: accumulator r of lane l holds weight row
// 4 (l / 16) + r of the wave's 16-row block, token l % 16.
template <class S, int MODE>
__device__ __forceinline__ void stream_store(const GemmArgs& a, floatx4 acc0,
                                             floatx4 acc1, int nb, int nrows,
                                             int pstart, int wave, int lane) {
  const int t = lane & 15, q = lane >> 4;
  if (t >= nrows) return;
  const size_t prow = (size_t)(pstart + t);
  if (MODE == 0) {
    typedef S s4 __attribute__((ext_vector_type(4)));
    const int f = nb * 64 + wave * 16 + q * 4;
    s4 hv, lv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float h = swiglu(acc0[r], acc1[r], a.clamp);
      hv[r] = (S)h;
      lv[r] = (S)(h - (float)hv[r]);
    }
    *reinterpret_cast<s4*>(reinterpret_cast<S*>(a.out) + prow * a.out_ld + f) = hv;
    if (a.out2)
      *reinterpret_cast<s4*>(reinterpret_cast<S*>(a.out2) + prow * a.out_ld + f) = lv;
  } else {
    const int d = nb * 128 + wave * 32 + q * 4;
    float* o = reinterpret_cast<float*>(a.out) + prow * a.out_ld + d;
    *reinterpret_cast<float4*>(o) = float4{acc0[0], acc0[1], acc0[2], acc0[3]};
    *reinterpret_cast<float4*>(o + 16) = float4{acc1[0], acc1[1], acc1[2], acc1[3]};
  }
}

__device__ __forceinline__ int run_start(int U, int b, int G) {
  return (int)((int64_t)U * b / G);
}
// the run holding unit u: largest b with run_start(b) <= u
__device__ __forceinline__ int run_of(int U, int u, int G) {
  return (int)(((int64_t)(u + 1) * G - 1) / U);
}

}  // namespace

template <class TT, int WQ, int MODE, int LO>
__global__ __launch_bounds__(256, 1) void gemm_stream_kernel(GemmArgs a) {
  using S = typename TT::S;
  using V8 = typename TT::V8;
  using Gm = Geo<WQ, LO>;
  constexpr int NS = Gm::NS;
  constexpr int kStage = Gm::kW + Gm::kSc + Gm::kA * Gm::kAPlanes;
  constexpr int nI = Gm::nI;
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, N = a.N;
  const int nk = K / Gm::BK;
  const int NNB = MODE == 0 ? N / 64 : N / 128;
  const int U = a.meta[a.meta_index] * NNB * nk;   // below 2^31 (host check)
  const int G = gridDim.x, b = blockIdx.x;
  const int u0 = run_start(U, b, G), u1 = run_start(U, b + 1, G);
  if (u0 >= u1) return;   // whole block
  const int first_item = u0 / nk;

  // per-launch lane offsets of the DMA instructions
  const uint32_t wrow_b = WQ ? (uint32_t)K / 2u : (uint32_t)K * 2u;   // weight row bytes
  const uint32_t srow_b = (uint32_t)K / 16u;                          // scale row bytes
  uint32_t vw[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int rl = lane >> 4;                       // row within the instruction
    const int c = (lane & 15) ^ ((jj * 4 + rl) & 15);
    vw[jj] = (uint32_t)rl * wrow_b + (uint32_t)c * 16u;
  }
  const uint32_t vs = (uint32_t)(lane >> 3) * srow_b + (uint32_t)(lane & 7) * 4u;
  uint32_t va[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * wave + i;
    if (WQ) va[i] = (uint32_t)(lane ^ t) * 16u;                            // 1 KB rows
    else va[i] = (uint32_t)(((lane >> 2) ^ t) * 16 + (lane & 3) * 4);      // 256 B rows
  }
  const uint32_t a_row_b = (uint32_t)a.a_ld * 2u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t ra2 = make_rsrc(LO ? a.A2 : a.A, a.a_bytes);

  // issue-side state
  int iss_item = -1, pf_item = -1;
  Item iss{}, pf{};
  __amdgpu_buffer_rsrc_t rw0 = ra, rw1 = ra, rs0 = ra, rs1 = ra;
  const int last_item = (u1 - 1) / nk;

  auto set_item = [&](int item) {
    iss = (item == pf_item) ? pf : load_item<MODE>(a, item, NNB, wave);
    iss_item = item;
    // one expert's matrix: N rows (F for gate/up, D for down)
    const size_t mat_b = (size_t)N * wrow_b;
    const size_t smat_b = (size_t)N * srow_b;
    rw0 = make_rsrc((const char*)a.B0 + (size_t)iss.e * mat_b, (uint32_t)mat_b);
    rw1 = MODE == 0 ? make_rsrc((const char*)a.B1 + (size_t)iss.e * mat_b, (uint32_t)mat_b) : rw0;
    if (WQ) {
      rs0 = make_rsrc((const char*)a.B0s + (size_t)iss.e * smat_b, (uint32_t)smat_b);
      rs1 = MODE == 0 ? make_rsrc((const char*)a.B1s + (size_t)iss.e * smat_b, (uint32_t)smat_b) : rs0;
    }
    if (item + 1 <= last_item) {
      pf = load_item<MODE>(a, item + 1, NNB, wave);
      pf_item = item + 1;
    }
  };

  // DMA of unit v into ring slot sl
  auto issue = [&](int v, int sl) {
    const int item = v / nk;
    const int kt = v - item * nk;
    if (item != iss_item) set_item(item);
    char* st = smem + sl * kStage;
    // weights: 8 x 1 KB (4 rows of 256 B each)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      int rowbase;
      if (MODE == 0) rowbase = iss.nb * 64 + wave * 16 + (jj & 3) * 4;
      else rowbase = iss.nb * 128 + wave * 32 + jj * 4;
      const __amdgpu_buffer_rsrc_t r = (MODE == 0 && jj >= 4) ? rw1 : rw0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(st + wave * 8192 + jj * 1024), 16, (int)vw[jj],
          (int)((uint32_t)rowbase * wrow_b + (uint32_t)kt * 256u), 0, 0);
    }
    if (WQ) {
      // scales: 4 x 256 B (8 rows of 32 B each), 4-byte lanes
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        int rowbase;
        if (MODE == 0) rowbase = iss.nb * 64 + wave * 16 + (m & 1) * 8;
        else rowbase = iss.nb * 128 + wave * 32 + m * 8;
        const __amdgpu_buffer_rsrc_t r = (MODE == 0 && m >= 2) ? rs1 : rs0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_ptr_t)(st + Gm::kW + wave * 1024 + m * 256), 4, (int)vs,
            (int)((uint32_t)rowbase * srow_b + (uint32_t)kt * 32u), 0, 0);
      }
    }
    // token rows 4 wave .. 4 wave + 3
#pragma unroll
    for (int pl = 0; pl < Gm::kAPlanes; ++pl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * wave + i;
        char* dst = st + Gm::kW + Gm::kSc + pl * Gm::kA + t * (WQ ? 1024 : 256);
        const int so = (int)((uint32_t)iss.tok[i] * a_row_b +
                             (uint32_t)kt * (WQ ? 1024u : 256u));
        if constexpr (WQ)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)dst, 16,
                                                   (int)va[i], so, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(pl ? ra2 : ra, (lds_ptr_t)dst,
                                                   4, (int)va[i], so, 0, 0);
      }
    }
  };

  const int r16 = lane & 15, q = lane >> 4;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int sl) {
    const char* Ws = smem + sl * kStage;
    const char* Ss = Ws + Gm::kW;
    const char* As = Ws + Gm::kW + Gm::kSc;
    const char* w0 = Ws + (wave * 32 + r16) * 256;
    const char* w1 = w0 + 16 * 256;
    if (!WQ) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int pc = ((4 * s + q) ^ r16) * 16;
        const V8 wa = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(w0 + pc));
        const V8 wb = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(w1 + pc));
        const V8 bt = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(As + r16 * 256 + pc));
        acc0 = mfma16(wa, bt, acc0);
        acc1 = mfma16(wb, bt, acc1);
        if (LO) {
          const V8 bl = __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(As + Gm::kA + r16 * 256 + pc));
          acc0 = mfma16(wa, bl, acc0);
          acc1 = mfma16(wb, bl, acc1);
        }
      }
    } else {
      const char* s0 = Ss + (wave * 32 + r16) * 32;
      const char* s1 = s0 + 16 * 32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 4 * g + q;
        const int pc = (c ^ r16) * 16;
        const uint4 qa = *reinterpret_cast<const uint4*>(w0 + pc);
        const uint4 qb = *reinterpret_cast<const uint4*>(w1 + pc);
        const _Float16 sa = *reinterpret_cast<const _Float16*>(s0 + c * 2);
        const _Float16 sb = *reinterpret_cast<const _Float16*>(s1 + c * 2);
        half8 ha[4], hb[4];
        dequant32(qa, sa, ha);
        dequant32(qb, sb, hb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tc = ((16 * g + 4 * q + i) ^ r16) * 16;
          const half8 bt = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(As + r16 * 1024 + tc));
          acc0 = mfma16(ha[i], bt, acc0);
          acc1 = mfma16(hb[i], bt, acc1);
        }
      }
    }
  };

  // prologue: NS - 1 units in flight
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(min(u0 + p, u1 - 1), p);

  int cmp_item = -1, c_nb = 0, c_nrows = 0, c_pstart = 0;
  for (int u = u0; u < u1; ++u) {
    const int j = u - u0;
    wait_vmcnt<(NS - 2) * nI>();       // unit u landed (this wave's share)
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
        stream_store<S, MODE>(a, acc0, acc1, c_nb, c_nrows, c_pstart, wave, lane);
      } else {
        float* pp = a.part + ((size_t)b * 2 + (item == first_item ? 0 : 1)) * 2048;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pp[r * 256 + tid] = acc0[r];
          pp[(4 + r) * 256 + tid] = acc1[r];
        }
      }
      acc0 = floatx4{0.f, 0.f, 0.f, 0.f};
      acc1 = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();   // no direct-to-LDS write outlives the workgroup
}

// Items cut by run boundaries: the partial sums of their runs, added in run
// order, then the same epilogue. Block j looks at the boundary after run j
// and handles the item only if j is the item's first run.
template <class TT, int WQ, int MODE>
__global__ __launch_bounds__(256) void gemm_stream_fixup_kernel(GemmArgs a, int G) {
  using S = typename TT::S;
  using Gm = Geo<WQ, 0>;
  const int nk = a.K / Gm::BK;
  const int NNB = MODE == 0 ? a.N / 64 : a.N / 128;
  const int U = a.meta[a.meta_index] * NNB * nk;
  const int j = blockIdx.x;
  if (j + 1 >= G || U == 0) return;
  const int v = run_start(U, j + 1, G);
  if (v >= U || v % nk == 0) return;
  const int item = v / nk;
  const int fu = item * nk;
  if (run_of(U, fu, G) != j) return;
  const int bl = run_of(U, fu + nk - 1, G);
  const int tid = threadIdx.x;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int rb = j; rb <= bl; ++rb) {
    const int s0 = run_start(U, rb, G);
    if (s0 == run_start(U, rb + 1, G)) continue;   // empty run
    const int slot = s0 / nk == item ? 0 : 1;
    const float* pp = a.part + ((size_t)rb * 2 + slot) * 2048;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc0[r] += pp[r * 256 + tid];
      acc1[r] += pp[(4 + r) * 256 + tid];
    }
  }
  const int g = item / NNB;
  stream_store<S, MODE>(a, acc0, acc1, item - g * NNB, a.list[4 * g + 2],
                        a.list[4 * g + 3], tid >> 6, tid & 63);
}

bool stream_supported(int mode, int K, int N, int wdt) {
  const int bk = wdt == MOE_Q4B32 ? 512 : 128;
  if (K <= 0 || K % bk) return false;
  return mode == 0 ? (N % 64 == 0) : (N % 128 == 0);
}

template <class TT, int WQ>
static hipError_t stream_launch(const GemmArgs& a, int grid, hipStream_t s) {
  if (a.mode == 0) {
    hipLaunchKernelGGL((gemm_stream_kernel<TT, WQ, 0, 0>), dim3(grid), dim3(256), 0, s, a);
    hipLaunchKernelGGL((gemm_stream_fixup_kernel<TT, WQ, 0>), dim3(grid), dim3(256), 0, s, a, grid);
  } else {
    if (!WQ && a.A2)
      hipLaunchKernelGGL((gemm_stream_kernel<TT, WQ, 1, 1>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_stream_kernel<TT, WQ, 1, 0>), dim3(grid), dim3(256), 0, s, a);
    hipLaunchKernelGGL((gemm_stream_fixup_kernel<TT, WQ, 1>), dim3(grid), dim3(256), 0, s, a, grid);
  }
  return hipGetLastError();
}

struct SF16 { using S = _Float16; using V8 = half8; };
struct SBF16 { using S = __bf16; using V8 = bf16x8; };

hipError_t launch_gemm_stream(const GemmArgs& a, int xdt, int wdt, int grid,
                              hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > kStreamMaxRuns) return hipErrorInvalidValue;
  if (xdt == MOE_BF16 && wdt == MOE_BF16) return stream_launch<SBF16, 0>(a, grid, s);
  if (xdt == MOE_F16 && wdt == MOE_F16) return stream_launch<SF16, 0>(a, grid, s);
  if (xdt == MOE_F16 && wdt == MOE_Q4B32) return stream_launch<SF16, 1>(a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
