// Internal declarations shared by the HIP sources of the MI355X MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- vector types for gfx950 MFMA operands ------------------------------
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Plan chunking: tokens per chunk of the permute (one 64-bit mask per
// expert and chunk gives the in-chunk stable rank by popcount). The route
// kernel writes one histogram row per 16 x tpw tokens (16 waves, tpw tokens
// each): tpw = 4 (one row per chunk) for long prompts over at most 256
// experts, else 1 (up to kRouteShortT tokens a 64-token block would leave
// most CUs idle; above 256 experts four tokens' logits do not fit a lane's
// registers). With tpw = 4, k <= 16 and at most 256 experts a wave ranks its
// four tokens at once, 16 lanes each; otherwise one after another on all
// 64 lanes (fewer instructions per token, more per wave).
constexpr int kChunk = 64;
constexpr int kRouteShortT = 2048;
constexpr int kRouteGroupK = 16;
inline bool route_grouped(int E, int k) { return E <= 256 && k <= kRouteGroupK; }
inline int route_tpw(int T, int E) { return (T <= kRouteShortT || E > 256) ? 1 : 4; }
// The single-block plan kernel takes prompts of at most kChunk tokens and
// kPlanSmallPairs (token, choice) pairs, held in LDS, over at most 256
// experts.
constexpr int kPlanSmallPairs = 4096;
constexpr int kPlanSmallE = 256;
constexpr int kMaxExperts = 1024;

// Token rows per full-tile work item (the classify kernel's tile list).
constexpr int kFullBM = 256;
// Row padding of the SwiGLU output H: 256 bytes, so rows whose unpadded
// stride is a large power of two do not all start on the same L2 channel.
constexpr int kPadBytes = 256;
// Split-K tile: output columns per item and rows per row block.
constexpr int kSkNB = 64;
constexpr int kSkRows = 64;   // rows per split-K group (4 blocks of 16)
// Stream tile: each run (workgroup) of a launch owns two fp32 partial-sum
// slots of 256 threads x 8 RB values (RB = 16-row token blocks of its
// groups) in a workspace buffer of kStreamPartFloats, so a launch takes at
// most kStreamPartFloats / (2 x 2048 RB) runs. Its groups hold at most
// kStreamTokRows pairs (the classify kernel's token table has that many
// entries per group).
constexpr int kStreamSlotFloats1 = 2048;          // per 16-row block
constexpr int kStreamPartFloats = 2 * 2048 * 2048;
constexpr int kStreamTokRows = 64;
// At most this many runs a launch: the arrival counters of the items cut by
// run boundaries are kept per (run, wave).
constexpr int kStreamMaxRuns = 512;
inline int stream_max_runs(int rb) {
  const int by_part = kStreamPartFloats / (2 * kStreamSlotFloats1 * rb);
  return by_part < kStreamMaxRuns ? by_part : kStreamMaxRuns;
}

// The format of a 4-bit weight dtype: 0 signed with an fp16 scale per 32
// K values, 1 / 2 affine with an fp16 (scale, bias) pair per 32 / 64; -1 if
// the dtype is not a 4-bit one.
inline int q4_fmt(int wdt) {
  return wdt == MOE_Q4B32 ? 0 : wdt == MOE_Q4A32 ? 1 : wdt == MOE_Q4A64 ? 2 : -1;
}

// Forward route tags per expert.
enum Route : int32_t { kRouteNone = 0, kRouteSplitK = 1, kRouteFull = 2,
                       kRouteFat = 3 };

// Forward meta counters written by the classify kernel (or, for a
// decode-shaped plan, by the plan kernel). Counters 8..15 and 16..23 are the
// full tile's work queues (one per XCD) of the gate/up and the down launch;
// from 32 on, the stream tile's arrival counters, 4 per run; the classify
// (plan) kernel zeroes them all, and the stream tile leaves its own at zero.
enum Meta : int32_t { kMetaFullTiles = 0, kMetaSk1 = 1, kMetaSk4 = 2,
                      kMetaFat = 3, kMetaQueueGateUp = 8, kMetaQueueDown = 16,
                      kMetaFix = 32, kMetaCount = kMetaFix + 4 * kStreamMaxRuns };

// Router GEMM: prompts of at most kRouterDotT tokens (and fp32 inputs) take
// the dot-product kernel; longer ones the MFMA tile, 128 x 128 when that
// gives at least kRouterBigTiles blocks, else 64 x 64.
constexpr int kRouterDotT = 64;
constexpr int kRouterBigTiles = 128;
// d_model bound of the router: a 128-row tile's bytes stay below 2^31.
constexpr int kRouterMaxD = 1 << 20;

// Sets this thread's last-error message (moe_last_error) and returns st.
moe_status set_error(moe_status st, const char* fmt, ...);

// ---- launchers (plan_kernels.hip) ---------------------------------------
hipError_t launch_route_hist(const float* logits, int T, int E, int k,
                             int32_t* ids, float* w, int32_t* hist, int tpw,
                             hipStream_t s);
hipError_t launch_scan(int32_t* hist, int NC, int T, int E, int k,
                       int n_shared, int64_t limit, int32_t* total,
                       int32_t* counts, int32_t* offsets, int64_t* stats,
                       hipStream_t s);
hipError_t launch_permute(const int32_t* ids, const float* w,
                          const int32_t* base, int rows_per_chunk,
                          const int32_t* offsets, int T, int E, int k,
                          int n_shared, int64_t limit, int32_t* slot,
                          int32_t* tok2pair, int32_t* pair_token,
                          float* pair_w, hipStream_t s);

// A decode-shaped plan (at most kDecodeT tokens: every expert holds at most
// that many pairs, one thin group each) also carries the thin-group list
// the classify kernel would build: (expert, 0, rows, first pair) per touched
// expert in expert order, each group's x rows (kStreamTokRows entries,
// clamped to its last row) and the group count at dmeta[kMetaSk1].
constexpr int kDecodeT = 16;
struct DecodeGroups {
  int32_t* list;   // [E + n_shared, 4]
  int32_t* tok;    // [E + n_shared, kStreamTokRows]
  int32_t* meta;   // [kMetaCount]
};
hipError_t launch_plan_small(const float* logits, int T, int E, int k,
                             int n_shared, int64_t limit, int32_t* ids,
                             float* w, int32_t* total, int32_t* counts,
                             int32_t* offsets, int64_t* stats, int32_t* slot,
                             int32_t* tok2pair, int32_t* pair_token,
                             float* pair_w, const DecodeGroups* dg,
                             hipStream_t s);

// ---- forward (forward_kernels.hip) --------------------------------------
struct ClassifyArgs {
  const int32_t* counts;   // [n_exp]
  int n_exp;               // E + n_shared
  int mode;                // 0: all split-K (f32), 1: by S (bf16/f16), 2: q4
  double S;                // split-K bound in pairs per expert (f32 value)
  int full_nnb;            // mode 1: gate/up column blocks per full tile
  int full_fill;           // mode 1: work-groups that one round of the full
                           // tile occupies; when its tiles x full_nnb fall
                           // short of that, experts of <= kFullBM rows move
                           // to split-K. 0: the S rule alone
  int fat_rows;            // q4: >= fat_rows -> fat; <= 0 off
  int32_t* full_tiles;     // [cap] (expert, row0) pairs as int2
  int32_t* sk1;            // [cap] (expert, row0, nrows, pstart) as int4,
                           // groups of <= 16 rows
  int32_t* sk4;            // [cap] same, groups of 17..64 rows
  const int32_t* offsets;  // [n_exp + 1]: pstart = offsets[e] + row0
  const int32_t* pair_token;   // [P]
  int32_t* sk1_tok;        // [cap, kStreamTokRows]: x rows of each sk1
                           // group, clamped to its last row; or null
  int32_t* sk4_tok;        // the same for sk4 (stream tile, wide 4-bit
                           // tile); or null
  int32_t* fat_slot;       // [n_exp]
  int32_t* fat_list;       // [n_exp]
  int32_t* meta;           // [kMetaCount]
};
hipError_t launch_classify(const ClassifyArgs& a, hipStream_t s);

// Operand set of one GEMM stage (gate/up or down).
struct GemmArgs {
  int mode;                 // 0: gate/up (+ clamped SwiGLU), 1: down; the
                            // full tile's backward modes: 2 gate/up raw f32
                            // [G | U], 4 dH' (A per-pair rows, B0 = W_down
                            // as [K, N]), 5 dX (A per-pair rows, B0 / B1 =
                            // W_gate / W_up as the two halves of K)
  int K, N;                 // K: reduction; N: output width (F or D)
  const void* A;            // gate/up: x [T, D]; down: H [P, F]
  const void* A2;           // down, bf16 split H: the low plane; else null
  uint32_t a_bytes;         // bytes of A (and of A2): below 2^31
  int a_ld;                 // A row stride, elements
  int out_ld;               // output row stride, elements
  const int32_t* pair_token;// gather map for gate/up
  const int32_t* offsets;   // [n_exp + 1]
  const float* pair_w;      // [P] (the combine applies the weights)
  // B operands, [n_exp, rows, K]: gate/up use B0 = W_gate, B1 = W_up; down
  // uses B0 = W_down. q4: data + scales.
  const void* B0; const void* B0s;
  const void* B1; const void* B1s;
  // Dequantised fp16 copies of fat experts, k-block-major: [slot][K / 32]
  // [rows][32]; nullptr if none.
  const void* S0; const void* S1;
  const int32_t* fat_slot;
  void* out;                // H [P, F] (x's dtype) or Ypair [P, D] (unweighted;
                            // fp16 in an fp16 layer, else f32)
  void* out2;               // gate/up, bf16 split H: low plane; else null
  float clamp;              // SwiGLU limit, <= 0 off
  const int32_t* list;      // work list (full tiles or split-K groups)
  const int32_t* meta;      // counts of the work lists
  int meta_index;           // which meta counter holds this list's length
  int32_t* queue;           // full tile: 8 zeroed work-queue counters
  int h_rows;               // full tile: rows of the k-block-major H
                            // ([F / 32][h_rows][32]) it writes (gate/up) or
                            // reads (down)
  const int32_t* tok;       // gate/up of the stream tile and the wide 4-bit
                            // tile: the listed groups' x rows
                            // (kStreamTokRows a group)
  float* part;              // stream tile: [runs, 2, 2048 RB] floats
  int32_t* fix;             // stream tile: [runs, 4] arrival counters of the
                            // items cut by run boundaries (zero on entry,
                            // left at zero)
};
hipError_t launch_gemm_full(const GemmArgs& a, int xdt, int grid,
                            hipStream_t s);

// Weight gradients (gemm_wgrad.hip): for every expert e (heaviest first in
// eord), C_e = A_e^T B_e over its kept pairs offsets[e] .. offsets[e + 1] of
// the per-pair A [P, M] (a_ld = M) and B [P, N] (b_ld = N), f32; rows below
// row_split to out + e out_estride, the rest to out2 + e out_estride (rows
// of N values); zeros for an expert without pairs.
struct WgradArgs {
  const void* A; uint32_t a_bytes; int a_ld; int M;   // bytes below 2^31
  const void* B; uint32_t b_bytes; int b_ld; int N;
  const int32_t* offsets;
  const int32_t* eord;
  int n_exp;
  float* out; float* out2; int row_split;
  int64_t out_estride;
};
hipError_t launch_wgrad(const WgradArgs& a, int xdt, hipStream_t s);
hipError_t launch_gemm_splitk(const GemmArgs& a, int xdt, int wdt, int rb,
                              int grid, hipStream_t s);
bool stream_supported(int mode, int K, int N, int wdt);
hipError_t launch_gemm_stream(const GemmArgs& a, int xdt, int wdt, int rows,
                              int grid, hipStream_t s);
hipError_t launch_gemm_wide(const GemmArgs& a, int xdt, int wdt, int grid,
                            hipStream_t s);
// fmt: the 4-bit format (q4_fmt in device_common.h): 0 signed with a scale
// per 32 values, 1 / 2 affine with a (scale, bias) word per 32 / 64 values
hipError_t launch_dequant_fat(const void* const q[3], const void* const sc[3],
                              void* const out[3], const int rows[3],
                              const int K[3], int n, const int32_t* fat_list,
                              const int32_t* meta, int grid, int fmt,
                              hipStream_t s);
hipError_t launch_dequant_rows(const void* q, const void* sc, void* out,
                               int64_t rows, int K, int fmt, hipStream_t s);
hipError_t launch_combine(const void* ypair, int ypair_f16,
                          const int32_t* tok2pair, const float* topk_w,
                          const int32_t* offsets, int T, int D, int k,
                          int n_shared, int E, int ydt, void* y, hipStream_t s);

// One-token calls on bf16 / fp16 layers (gemv_decode.hip): gate/up and
// SwiGLU, then down with the combine, one matrix-vector product per weight
// row of the token's experts.
struct GemvArgs {
  const void* x;            // [D] the token's row (x's dtype)
  const void* wg;           // W_gate [E + n_shared, F, D]
  const void* wu;           // W_up   [E + n_shared, F, D]
  const void* wd;           // W_down [E + n_shared, D, F]
  const void* wgs;          // 4-bit weights: the parameters of W_gate,
  const void* wus;          // W_up and W_down ([.., N, K / group] fp16
  const void* wds;          // scales or (scale, bias) words); else null
  int fmt;                  // 4-bit format (q4_fmt), or -1
  const int32_t* ids;       // [k] the token's experts (plan)
  const int32_t* tok2pair;  // [k] their pair rows, -1 if dropped (plan)
  const float* w;           // [k] routing weights (plan)
  const int32_t* offsets;   // [E + n_shared + 1] (plan): the shared row
  void* h;                  // H [P, h_ld], x's dtype
  void* h2;                 // bf16 low plane of H, or null
  int h_ld;
  void* ypair;              // [P, D] unweighted expert outputs (fp16 in an
                            // fp16 layer, else f32)
  void* y;                  // [D] the output, y's dtype
  int D, F, k, E, n_shared;
  float clamp;
};
bool gemv_supported(int D, int F, int k, int n_shared);
bool gemv_q4_supported(int D, int F, int k, int n_shared, int fmt);
hipError_t launch_gemv_gateup(const GemvArgs& a, int xdt, hipStream_t s);
hipError_t launch_gemv_down(const GemvArgs& a, int xdt, int ydt, hipStream_t s);

// ---- backward (backward.hip) --------------------------------------------
struct BwdArgs {
  int xdt;                      // MOE_BF16 or MOE_F16 (x and the weights)
  int T, D, F, E, k, n_shared, n_exp;
  int64_t Pmax;                 // most pairs the plan can hold
  int ncu;
  const void* x;                // [T, D]
  const float* dy;              // [T, D]
  const void* wg; const void* wu; const void* wd;
  float clamp;
  const int32_t* offsets; const int32_t* pair_token; const float* pair_w;
  const int32_t* tok2pair; const int32_t* ids; const float* topk_w;
  float* dx; float* dwg; float* dwu; float* dwd;   // outputs (f32)
  float* dtw; float* dlogits;   // optional outputs
  float* dtw_scratch;           // [T, k] when dlogits is wanted without dtw
  void* ws;                     // bwd_workspace_bytes
};
size_t bwd_workspace_bytes(int64_t Pmax, int n_exp, int D, int F);
// stage 0: recompute (gather, [G | U], H); 1: data gradients (dH', dG / dU
// with the per-pair routing-weight dots, dXp, dx); 2: weight gradients; 3:
// routing-weight and logit gradients
hipError_t launch_backward(const BwdArgs& a, int stage, hipStream_t s);

// ---- router (router.hip) ---------------------------------------------------
size_t router_scratch_bytes(int T, int E);
// scratch: the statistics scratch (its accumulators are cleared by the
// router kernel), or null when no statistics follow
hipError_t launch_router_gemm(const void* x, int xdt, const void* w,
                              float* logits, int T, int D, int E,
                              void* scratch, hipStream_t s);
hipError_t launch_router_stats(const float* logits, const int32_t* ids, int T,
                               int E, int k, int32_t* want_out, void* scratch,
                               float* stats, float z_weight, hipStream_t s);

}  // namespace moe
