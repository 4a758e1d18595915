// C ABI of the routed MoE layer: host-side validation, workspace layouts
// and launch sequencing. Every argument is checked before the first launch;
// every launch goes to the caller's stream; nothing here synchronises except
// moe_plan_stats_get and moe_phase_times.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

}  // namespace

moe_status moe::set_error(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

namespace {

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_EHIP, "%s: %s (%s)", where, hipGetErrorName(e),
              hipGetErrorString(e));
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline int xbytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

struct PlanLayout {
  size_t ids, w, slot, tok2pair, hist, total, counts, offsets, pair_token,
      pair_w, stats, dlist, dtok, dmeta, bytes;
  int NC;     // 64-token permute chunks
  int NR;     // histogram rows (16 x tpw tokens each)
  int tpw;    // route tokens per wave
  bool small; // one-block plan kernel
  bool decode;// ... which also writes the decode-shaped thin-group list
};

// The one-block plan kernel takes prompts of at most kChunk tokens over at
// most kPlanSmallE experts; for at most kDecodeT tokens it also writes the
// thin-group list (every expert then holds at most kDecodeT pairs).
inline bool plan_is_small(const moe_plan_desc& d) {
  return d.T >= 1 && d.T <= kChunk && (int64_t)d.T * d.k <= kPlanSmallPairs &&
         d.E <= kPlanSmallE;
}

bool desc_ok(const moe_plan_desc* d, std::string* why) {
  char buf[256];
  if (!d) { *why = "desc is NULL"; return false; }
  if (d->E < 1 || d->E > kMaxExperts) {
    snprintf(buf, sizeof buf, "E=%d outside 1..%d", d->E, kMaxExperts);
    *why = buf; return false;
  }
  if (d->k < 1 || d->k > d->E) {
    snprintf(buf, sizeof buf, "k=%d outside 1..E=%d", d->k, d->E);
    *why = buf; return false;
  }
  if (d->T < 0) { *why = "T < 0"; return false; }
  if (d->n_shared != 0 && d->n_shared != 1) { *why = "n_shared not 0 or 1"; return false; }
  if (!std::isfinite(d->capacity_factor) || d->capacity_factor < 0.f) {
    snprintf(buf, sizeof buf, "capacity_factor=%g must be finite and >= 0",
             (double)d->capacity_factor);
    *why = buf; return false;
  }
  if ((int64_t)d->T * (d->k + 1) >= ((int64_t)1 << 31)) {
    *why = "T*(k+1) must be below 2^31"; return false;
  }
  return true;
}

PlanLayout plan_layout(const moe_plan_desc& d) {
  PlanLayout L{};
  const size_t Tk = (size_t)d.T * d.k;
  const size_t P = Tk + (size_t)d.n_shared * d.T;
  L.NC = (d.T + kChunk - 1) / kChunk;
  L.tpw = route_tpw(d.T, d.E);
  L.NR = (d.T + 16 * L.tpw - 1) / (16 * L.tpw);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  L.ids = take(Tk * 4);
  L.w = take(Tk * 4);
  L.slot = take(Tk * 4);
  L.tok2pair = take(Tk * 4);
  L.hist = take((size_t)L.NR * (d.E + 1) * 4);
  L.total = take((size_t)(d.E + 1) * 4);
  L.counts = take((size_t)(d.E + 1) * 4);
  L.offsets = take((size_t)(d.E + 2) * 4);
  L.pair_token = take(P * 4 + 4);
  L.pair_w = take(P * 4 + 4);
  L.stats = take(8 * 8);
  L.small = plan_is_small(d);
  L.decode = L.small && d.T <= kDecodeT;
  const size_t ng = L.decode ? (size_t)(d.E + d.n_shared) : 0;
  L.dlist = take(ng * 16);
  L.dtok = take(ng * kStreamTokRows * 4);
  L.dmeta = take(L.decode ? kMetaCount * 4 : 0);
  L.bytes = o;
  return L;
}

int64_t capacity_limit(const moe_plan_desc& d) {
  if (d.capacity_factor == 0.f) return -1;
  const double fair = (double)d.capacity_factor * (double)d.T * d.k / d.E;
  const double f = std::floor(fair);
  if (f < 1.0) return 1;
  if (f > 2e9) return -1;   // beyond any count: same as no cap
  return (int64_t)f;
}

struct DevInfo { int ncu = 0; };

moe_status device_info(int* dev, DevInfo* info) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::mutex mu;
  static std::vector<int> ncu_cache;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ncu_cache.size() <= *dev) ncu_cache.resize(*dev + 1, 0);
  if (ncu_cache[*dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, *dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    ncu_cache[*dev] = n > 0 ? n : 1;
  }
  info->ncu = ncu_cache[*dev];
  return MOE_OK;
}

// ---- the forward's second stream ------------------------------------------
//
// Per device: a non-blocking stream at the default priority and the two
// events that fork it from the caller's stream and join it back. The mutex
// is held from the fork to the join of one call, so calls from several
// host threads do not interleave their records of the events.
constexpr double kForkMinWork = 8589934592.0;   // T k D F, 2^33

struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
std::mutex g_side_mu;
std::vector<SideStream*> g_side;   // never freed: lives as long as the process

SideStream* side_stream(int dev, moe_status* st) {
  std::lock_guard<std::mutex> lock(g_side_mu);
  if ((int)g_side.size() <= dev) g_side.resize(dev + 1, nullptr);
  if (!g_side[dev]) {
    SideStream* ss = new SideStream;
    hipError_t e = hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss->join, hipEventDisableTiming);
    if (e != hipSuccess) {
      *st = hip_fail(e, "second stream");
      if (ss->join) hipEventDestroy(ss->join);
      if (ss->fork) hipEventDestroy(ss->fork);
      if (ss->s) hipStreamDestroy(ss->s);
      delete ss;
      return nullptr;
    }
    g_side[dev] = ss;
  }
  return g_side[dev];
}

// ---- phase events ---------------------------------------------------------

struct PhaseRecord {
  hipEvent_t ev[2 * MOE_N_PHASES];
  bool used[MOE_N_PHASES];
  uint32_t mask;   // the phases this call records
};
std::mutex g_ev_mu;
std::vector<PhaseRecord> g_records;
size_t g_records_used = 0;

// flags: the call's option flags; bits 16 + p select phase p (none: all)
PhaseRecord* acquire_record(int32_t flags, moe_status* st) {
  std::lock_guard<std::mutex> lock(g_ev_mu);
  if (g_records_used == g_records.size()) {
    PhaseRecord r{};
    for (int i = 0; i < 2 * MOE_N_PHASES; ++i) {
      hipError_t e = hipEventCreate(&r.ev[i]);
      if (e != hipSuccess) {
        *st = hip_fail(e, "hipEventCreate");
        return nullptr;
      }
    }
    g_records.push_back(r);
  }
  PhaseRecord* r = &g_records[g_records_used++];
  for (int i = 0; i < MOE_N_PHASES; ++i) r->used[i] = false;
  const uint32_t sel = (uint32_t)flags >> MOE_OPT_PHASE_SHIFT;
  r->mask = sel ? sel : 0xFFFFu;
  return r;
}

struct PhaseScope {
  PhaseRecord* rec;
  int phase;
  hipStream_t s;
  PhaseScope(PhaseRecord* r, int p, hipStream_t st)
      : rec(r && ((r->mask >> p) & 1u) ? r : nullptr), phase(p), s(st) {
    if (rec) hipEventRecord(rec->ev[2 * phase], s);
  }
  ~PhaseScope() {
    if (rec) {
      hipEventRecord(rec->ev[2 * phase + 1], s);
      rec->used[phase] = true;
    }
  }
};

struct FwdLayout {
  size_t H, H2, Ht, Ht2, Y, full_tiles, sk1, sk4, sk1_tok, sk4_tok, part,
      fat_slot, fat_list, meta, stg_g, stg_u, stg_d, bytes;
  int cap_tiles, cap_sk1, cap_sk4, max_fat, fat_rows;
  bool stream;       // split-K groups on the stream tile
  bool can_full, can_sk1, can_sk4, can_fat;
  bool split_h;   // bf16: SwiGLU output as a hi + lo bf16 pair
  int h_ld;                 // padded row stride of H (elements)
};

bool dtypes_ok(int xdt, int wdt) {
  return (xdt == MOE_F32 && wdt == MOE_F32) ||
         (xdt == MOE_BF16 && wdt == MOE_BF16) ||
         (xdt == MOE_F16 && wdt == MOE_F16) ||
         (xdt == MOE_F16 && q4_fmt(wdt) >= 0);
}

int effective_fat_rows(const moe_options& o) {
  if (o.fat_rows <= 0) return 0;
  return std::max(o.fat_rows, 17);
}

FwdLayout fwd_layout(const moe_plan_desc& d, int D, int F, int xdt, int wdt,
                     const moe_options& o) {
  FwdLayout L{};
  const int64_t Pmax = (int64_t)d.T * d.k + (int64_t)d.n_shared * d.T;
  const int n_exp = d.E + d.n_shared;
  L.cap_tiles = n_exp + (int)(Pmax / kFullBM) + 1;
  L.cap_sk1 = n_exp;
  L.cap_sk4 = n_exp + (int)(Pmax / kSkRows) + 1;
  L.fat_rows = q4_fmt(wdt) >= 0 ? effective_fat_rows(o) : 0;
  // an expert holds at most T pairs (k distinct experts per token; the
  // shared one takes each token once), so a prompt of fewer than fat_rows
  // tokens has no fat expert
  L.max_fat = 0;
  if (L.fat_rows > 0 && d.T >= L.fat_rows)
    L.max_fat = (int)std::min<int64_t>(n_exp, Pmax / L.fat_rows);
  // the stream tile takes the split-K groups of a bf16/f16/q4 layer whose
  // sizes it tiles
  L.stream = wdt != MOE_F32 && stream_supported(0, D, F, wdt) &&
             stream_supported(1, F, D, wdt);
  if (wdt == MOE_F32) {
    L.can_full = false; L.can_sk1 = true; L.can_sk4 = true; L.can_fat = false;
  } else if (q4_fmt(wdt) >= 0) {
    L.can_fat = L.max_fat > 0;
    L.can_full = L.can_fat;
    L.can_sk1 = true;
    L.can_sk4 = L.fat_rows == 0 || L.fat_rows > 17;
  } else {
    const double S = (double)o.splitk_max_pairs;
    // without MOE_OPT_EXACT_ROUTES an underfilled full route hands experts
    // of up to kFullBM rows to split-K, in groups of both sizes
    const bool moves = !(o.flags & MOE_OPT_EXACT_ROUTES) && S < (double)Pmax;
    L.can_fat = false;
    L.can_full = S < (double)Pmax;
    L.can_sk1 = S >= 1.0 || moves;
    L.can_sk4 = S > 16.0 || moves;
  }
  const int xb = xbytes(xdt);
  L.h_ld = F + kPadBytes / xb;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  L.H = take((size_t)Pmax * L.h_ld * xb + 16);
  // bf16 H: the low plane by default only for capped plans (their dropped
  // pairs leave rows of y at zero, which lowers RMS(y) against the rounding
  // error of the rows that are not); an explicit flag decides otherwise
  L.split_h = xdt == MOE_BF16 &&
              ((o.flags & MOE_OPT_BF16_SPLIT_H) ||
               (!(o.flags & MOE_OPT_BF16_PLAIN_H) && d.capacity_factor > 0.f));
  L.H2 = take(L.split_h ? (size_t)Pmax * L.h_ld * 2 + 16 : 0);
  // H of full-tile experts, k-block-major [F / 32][Pmax][32]
  L.Ht = take(L.can_full ? (size_t)Pmax * F * xb + 16 : 0);
  L.Ht2 = take(L.can_full && L.split_h ? (size_t)Pmax * F * 2 + 16 : 0);
  L.Y = take((size_t)Pmax * D * (xdt == MOE_F16 ? 2 : 4) + 16);   // Ypair
  L.full_tiles = take((size_t)L.cap_tiles * 8);
  L.sk1 = take((size_t)L.cap_sk1 * 16);
  L.sk4 = take((size_t)L.cap_sk4 * 16);
  // the groups' x rows: read by the stream tile and (17..64-row groups)
  // by the wide 4-bit tile
  L.sk1_tok = take(L.stream ? (size_t)L.cap_sk1 * kStreamTokRows * 4 : 0);
  L.sk4_tok = take(L.stream || q4_fmt(wdt) >= 0
                       ? (size_t)L.cap_sk4 * kStreamTokRows * 4 : 0);
  L.part = take(L.stream ? (size_t)kStreamPartFloats * 4 : 0);
  L.fat_slot = take((size_t)n_exp * 4);
  L.fat_list = take((size_t)n_exp * 4);
  L.meta = take(kMetaCount * 4);
  // fp16 copies of fat experts, k-block-major [K / 32][rows][32]
  L.stg_g = take((size_t)L.max_fat * F * D * 2);
  L.stg_u = take((size_t)L.max_fat * F * D * 2);
  L.stg_d = take((size_t)L.max_fat * D * F * 2);
  L.bytes = off;
  return L;
}

moe_options defaults() {
  moe_options o;
  o.swiglu_limit = 7.0f;
  o.splitk_max_pairs = 16.0f;
  o.fat_rows = 64;
  o.flags = 0;
  return o;
}

bool weight_ok(const moe_weight& w, int wdt, std::string* why, const char* name) {
  char buf[200];
  if (w.dtype != wdt) {
    snprintf(buf, sizeof buf, "%s dtype %d differs from w_gate's %d", name, w.dtype, wdt);
    *why = buf; return false;
  }
  if (!w.data) { snprintf(buf, sizeof buf, "%s data is NULL", name); *why = buf; return false; }
  if (!aligned16(w.data)) { snprintf(buf, sizeof buf, "%s data not 16-byte aligned", name); *why = buf; return false; }
  if (q4_fmt(wdt) >= 0) {
    if (!w.scales) { snprintf(buf, sizeof buf, "%s scales NULL for 4-bit weights", name); *why = buf; return false; }
    // a lane reads two adjacent parameters as one load
    const uintptr_t al = wdt == MOE_Q4B32 ? 3u : 7u;
    if ((reinterpret_cast<uintptr_t>(w.scales) & al) != 0) {
      snprintf(buf, sizeof buf, "%s scales not %d-byte aligned", name, (int)al + 1);
      *why = buf; return false;
    }
  }
  return true;
}

}  // namespace

// The plan's kernels over `logits` into the workspace at b.
moe_status launch_plan(const moe_plan_desc& d, const float* logits,
                       const PlanLayout& L, char* b, int64_t limit,
                       hipStream_t s) {
  hipError_t e;
  if (L.small) {
    // one chunk: route, scan and permute in one block
    const DecodeGroups dg{(int32_t*)(b + L.dlist), (int32_t*)(b + L.dtok),
                          (int32_t*)(b + L.dmeta)};
    e = launch_plan_small(logits, d.T, d.E, d.k, d.n_shared, limit,
                          (int32_t*)(b + L.ids), (float*)(b + L.w),
                          (int32_t*)(b + L.total), (int32_t*)(b + L.counts),
                          (int32_t*)(b + L.offsets), (int64_t*)(b + L.stats),
                          (int32_t*)(b + L.slot), (int32_t*)(b + L.tok2pair),
                          (int32_t*)(b + L.pair_token), (float*)(b + L.pair_w),
                          L.decode ? &dg : nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "plan kernel");
  } else {
    if (L.NC > 0) {
      e = launch_route_hist(logits, d.T, d.E, d.k, (int32_t*)(b + L.ids),
                            (float*)(b + L.w), (int32_t*)(b + L.hist), L.tpw, s);
      if (e != hipSuccess) return hip_fail(e, "route kernel");
    }
    e = launch_scan((int32_t*)(b + L.hist), L.NR, d.T, d.E, d.k, d.n_shared,
                    limit, (int32_t*)(b + L.total), (int32_t*)(b + L.counts),
                    (int32_t*)(b + L.offsets), (int64_t*)(b + L.stats), s);
    if (e != hipSuccess) return hip_fail(e, "scan kernel");
    if (L.NC > 0) {
      e = launch_permute((const int32_t*)(b + L.ids), (const float*)(b + L.w),
                         (const int32_t*)(b + L.hist), 4 / L.tpw,
                         (const int32_t*)(b + L.offsets), d.T, d.E, d.k,
                         d.n_shared, limit, (int32_t*)(b + L.slot),
                         (int32_t*)(b + L.tok2pair), (int32_t*)(b + L.pair_token),
                         (float*)(b + L.pair_w), s);
      if (e != hipSuccess) return hip_fail(e, "permute kernel");
    }
  }
  return MOE_OK;
}

struct moe_plan {
  moe_plan_desc desc;
  int64_t limit;
  char* ws;
  PlanLayout L;
};

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

void moe_options_default(moe_options* opt) {
  if (opt) *opt = defaults();
}

size_t moe_plan_workspace_bytes(const moe_plan_desc* desc) {
  std::string why;
  if (!desc_ok(desc, &why)) { fail(MOE_EINVAL, "%s", why.c_str()); return 0; }
  return plan_layout(*desc).bytes;
}

moe_status moe_plan_create(const moe_plan_desc* desc, const float* logits,
                           void* ws, size_t ws_bytes, void* stream,
                           moe_plan** out) {
  std::string why;
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!desc_ok(desc, &why)) return fail(MOE_EINVAL, "%s", why.c_str());
  if (desc->T > 0 && !logits) return fail(MOE_EINVAL, "logits is NULL");
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (!aligned16(logits) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(MOE_EINVAL, "logits must be 16-byte and ws 256-byte aligned");
  const PlanLayout L = plan_layout(*desc);
  if (ws_bytes < L.bytes)
    return fail(MOE_EWORKSPACE, "plan workspace %zu bytes < %zu needed",
                ws_bytes, L.bytes);
  int dev;
  DevInfo info;
  moe_status st = device_info(&dev, &info);
  if (st != MOE_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* b = static_cast<char*>(ws);
  const moe_plan_desc& d = *desc;
  const int64_t limit = capacity_limit(d);
  st = launch_plan(d, logits, L, b, limit, s);
  if (st != MOE_OK) return st;
  moe_plan* p = new (std::nothrow) moe_plan;
  if (!p) return fail(MOE_EINVAL, "out of host memory");
  p->desc = d;
  p->limit = limit;
  p->ws = b;
  p->L = L;
  *out = p;
  return MOE_OK;
}

size_t moe_route_workspace_bytes(const moe_plan_desc* desc, int32_t D) {
  std::string why;
  if (!desc_ok(desc, &why)) { fail(MOE_EINVAL, "%s", why.c_str()); return 0; }
  if (D < 8 || D % 8 || D > kRouterMaxD) {
    fail(MOE_EINVAL, "D=%d must be a multiple of 8 in 8..%d", D, kRouterMaxD);
    return 0;
  }
  return plan_layout(*desc).bytes + router_scratch_bytes(desc->T, desc->E);
}

moe_status moe_route(const moe_plan_desc* desc, const void* x, int32_t x_dtype,
                     const void* w_router, int32_t D, float z_weight,
                     float* logits, moe_route_stats* stats,
                     int32_t* token_want, void* ws, size_t ws_bytes,
                     int32_t flags, void* stream, moe_plan** out) {
  std::string why;
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!desc_ok(desc, &why)) return fail(MOE_EINVAL, "%s", why.c_str());
  const moe_plan_desc& d = *desc;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16 && x_dtype != MOE_F16)
    return fail(MOE_EUNSUPPORTED, "router dtype %d: f32, bf16 or f16 only", x_dtype);
  if (D < 8 || D % 8 || D > kRouterMaxD)
    return fail(MOE_EINVAL, "D=%d must be a multiple of 8 in 8..%d", D, kRouterMaxD);
  if (!std::isfinite(z_weight)) return fail(MOE_EINVAL, "z_weight must be finite");
  if (d.T > 0 && (!x || !w_router || !logits))
    return fail(MOE_EINVAL, "x, w_router and logits must be non-NULL");
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits) ||
      !aligned16(stats) || !aligned16(token_want) ||
      (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(MOE_EINVAL, "pointers must be 16-byte and ws 256-byte aligned");
  const PlanLayout L = plan_layout(d);
  const size_t need = L.bytes + router_scratch_bytes(d.T, d.E);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "route workspace %zu bytes < %zu needed",
                ws_bytes, need);
  int dev;
  DevInfo info;
  moe_status st = device_info(&dev, &info);
  if (st != MOE_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* b = static_cast<char*>(ws);
  const int64_t limit = capacity_limit(d);
  PhaseRecord* rec = nullptr;
  if (flags & MOE_OPT_PHASE_EVENTS) {
    rec = acquire_record(flags, &st);
    if (!rec) return st;
  }
  hipError_t e;
  {
    PhaseScope ps(rec, 7, s);
    e = launch_router_gemm(x, x_dtype, w_router, logits, d.T, D, d.E,
                           (stats || token_want) ? b + L.bytes : nullptr, s);
  }
  if (e != hipSuccess) return hip_fail(e, "router kernel");
  {
    PhaseScope ps(rec, 8, s);
    st = launch_plan(d, logits, L, b, limit, s);
  }
  if (st != MOE_OK) return st;
  if (stats || token_want) {
    PhaseScope ps(rec, 9, s);
    e = launch_router_stats(logits, (const int32_t*)(b + L.ids), d.T, d.E,
                            d.k, token_want, b + L.bytes,
                            reinterpret_cast<float*>(stats), z_weight, s);
    if (e != hipSuccess) return hip_fail(e, "router statistics kernel");
  }
  moe_plan* p = new (std::nothrow) moe_plan;
  if (!p) return fail(MOE_EINVAL, "out of host memory");
  p->desc = d;
  p->limit = limit;
  p->ws = b;
  p->L = L;
  *out = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan* plan) { delete plan; }

moe_status moe_plan_get_views(const moe_plan* p, moe_plan_views* v) {
  if (!p || !v) return fail(MOE_EINVAL, "NULL plan or views");
  char* b = p->ws;
  v->topk_id = (const int32_t*)(b + p->L.ids);
  v->topk_w = (const float*)(b + p->L.w);
  v->slot = (const int32_t*)(b + p->L.slot);
  v->tok2pair = (const int32_t*)(b + p->L.tok2pair);
  v->counts = (const int32_t*)(b + p->L.counts);
  v->offsets = (const int32_t*)(b + p->L.offsets);
  v->pair_token = (const int32_t*)(b + p->L.pair_token);
  v->pair_w = (const float*)(b + p->L.pair_w);
  v->stats = (const int64_t*)(b + p->L.stats);
  return MOE_OK;
}

moe_status moe_plan_stats_get(const moe_plan* p, const moe_options* opt,
                              moe_plan_stats* out, void* stream) {
  if (!p || !out) return fail(MOE_EINVAL, "NULL plan or stats");
  const moe_options o = opt ? *opt : defaults();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const moe_plan_desc& d = p->desc;
  int64_t st[8];
  std::vector<int32_t> counts((size_t)d.E + d.n_shared);
  hipError_t e = hipMemcpyAsync(st, p->ws + p->L.stats, sizeof st,
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(counts.data(), p->ws + p->L.counts,
                       counts.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "moe_plan_stats_get");
  moe_plan_stats r{};
  r.T = d.T; r.E = d.E; r.k = d.k; r.n_shared = d.n_shared;
  r.limit = p->limit;
  r.pairs = (int64_t)d.T * d.k;
  r.dropped = st[0];
  r.kept = st[1];
  r.nonfinite = st[2];
  r.touched = st[3];
  r.max_rows = st[4];
  r.drop_fraction = r.pairs ? (double)r.dropped / (double)r.pairs : 0.0;
  const int fr = effective_fat_rows(o);
  for (int e2 = 0; e2 < d.E; ++e2) {
    const int c = counts[e2];
    if (c <= 0) continue;
    // route counts for 4-bit weights (fat_rows) and for dense bf16/f16 (S)
    if (fr > 0 && c >= fr) r.fat++;
    if ((double)c <= (double)o.splitk_max_pairs) r.thin++;
    else r.full++;
  }
  *out = r;
  return MOE_OK;
}

size_t moe_forward_workspace_bytes(const moe_plan* p, int32_t D, int32_t F,
                                   int32_t x_dtype, int32_t w_dtype,
                                   const moe_options* opt) {
  if (!p || D <= 0 || F <= 0 || D % 128 || F % 128 || !dtypes_ok(x_dtype, w_dtype)) {
    fail(MOE_EINVAL, "bad plan, sizes or dtypes for the workspace query");
    return 0;
  }
  const moe_options o = opt ? *opt : defaults();
  return fwd_layout(p->desc, D, F, x_dtype, w_dtype, o).bytes;
}

moe_status moe_forward(const moe_plan* p, const void* x, int32_t x_dtype,
                       moe_weight w_gate, moe_weight w_up, moe_weight w_down,
                       int32_t D, int32_t F, void* y, int32_t y_dtype,
                       void* ws, size_t ws_bytes, const moe_options* opt,
                       void* stream) {
  std::string why;
  if (!p) return fail(MOE_EINVAL, "plan is NULL");
  const moe_plan_desc& d = p->desc;
  const moe_options o = opt ? *opt : defaults();
  if (D <= 0 || F <= 0 || D % 128 || F % 128)
    return fail(MOE_EUNSUPPORTED, "D=%d and F=%d must be positive multiples of 128", D, F);
  const int wdt = w_gate.dtype;
  if (!dtypes_ok(x_dtype, wdt))
    return fail(MOE_EUNSUPPORTED, "dtype pair (x=%d, W=%d) not supported", x_dtype, wdt);
  if (!weight_ok(w_gate, wdt, &why, "w_gate") || !weight_ok(w_up, wdt, &why, "w_up") ||
      !weight_ok(w_down, wdt, &why, "w_down"))
    return fail(MOE_EINVAL, "%s", why.c_str());
  if (y_dtype != MOE_F32 && y_dtype != x_dtype)
    return fail(MOE_EUNSUPPORTED, "y dtype %d must be F32 or x's dtype", y_dtype);
  if (std::isnan(o.swiglu_limit) || std::isnan(o.splitk_max_pairs))
    return fail(MOE_EINVAL, "NaN option");
  if (d.T > 0 && (!x || !y)) return fail(MOE_EINVAL, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y))
    return fail(MOE_EINVAL, "x and y must be 16-byte aligned");
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(MOE_EINVAL, "workspace NULL or not 256-byte aligned");
  const FwdLayout L = fwd_layout(d, D, F, x_dtype, wdt, o);
  const size_t Pmax_rows = (size_t)d.T * d.k + (size_t)d.n_shared * d.T;
  const size_t lim31 = ((size_t)1 << 31) - 1;
  if ((size_t)d.T * D * xbytes(x_dtype) > lim31 ||
      Pmax_rows * (F * xbytes(x_dtype) + kPadBytes) > lim31 ||
      (size_t)D * F * 4 > lim31)
    return fail(MOE_EUNSUPPORTED, "x, the SwiGLU buffer and each weight "
                "matrix must each stay below 2 GiB");
  if (ws_bytes < L.bytes)
    return fail(MOE_EWORKSPACE, "forward workspace %zu bytes < %zu needed",
                ws_bytes, L.bytes);
  if (d.T == 0) return MOE_OK;
  int dev;
  DevInfo info;
  moe_status st = device_info(&dev, &info);
  if (st != MOE_OK) return st;
  PhaseRecord* rec = nullptr;
  if (o.flags & MOE_OPT_PHASE_EVENTS) {
    rec = acquire_record(o.flags, &st);
    if (!rec) return st;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* b = static_cast<char*>(ws);
  char* pb = p->ws;
  const int n_exp = d.E + d.n_shared;
  int32_t* meta = (int32_t*)(b + L.meta);
  hipError_t e;
  // A decode-shaped plan holds at most kDecodeT pairs an expert, so every
  // expert is one thin group unless the S rule sends experts of that size
  // to the full tile; then the plan's own group list stands in for the
  // classify kernel's.
  const bool decode = p->L.decode &&
      (wdt == MOE_F32 || q4_fmt(wdt) >= 0 ||
       (double)o.splitk_max_pairs >= (double)d.T);

  // One token on a 16-bit layer, or on a 4-bit layer with fp16 x: each of
  // its experts holds one pair, so every product is a matrix-vector
  // product; two launches read the chosen experts' weights across all
  // compute units, the second also summing the pairs into y (no combine
  // launch).
  const int fmt = q4_fmt(wdt);
  const bool gemv16 = L.stream && x_dtype == wdt && gemv_supported(D, F, d.k, d.n_shared);
  const bool gemv4 = fmt >= 0 && x_dtype == MOE_F16 &&
                     gemv_q4_supported(D, F, d.k, d.n_shared, fmt);
  if (decode && d.T == 1 && (gemv16 || gemv4) && !(o.flags & MOE_OPT_TILED_DECODE)) {
    GemvArgs ga{};
    ga.x = x;
    ga.wg = w_gate.data; ga.wu = w_up.data; ga.wd = w_down.data;
    ga.wgs = w_gate.scales; ga.wus = w_up.scales; ga.wds = w_down.scales;
    ga.fmt = fmt;
    ga.ids = (const int32_t*)(pb + p->L.ids);
    ga.tok2pair = (const int32_t*)(pb + p->L.tok2pair);
    ga.w = (const float*)(pb + p->L.w);
    ga.offsets = (const int32_t*)(pb + p->L.offsets);
    ga.h = b + L.H;
    ga.h2 = L.split_h ? b + L.H2 : nullptr;
    ga.h_ld = L.h_ld;
    ga.ypair = b + L.Y;
    ga.y = y;
    ga.D = D; ga.F = F; ga.k = d.k; ga.E = d.E; ga.n_shared = d.n_shared;
    ga.clamp = o.swiglu_limit;
    {
      PhaseScope ps(rec, 3, s);
      e = launch_gemv_gateup(ga, x_dtype, s);
      if (e != hipSuccess) return hip_fail(e, "one-token gate/up kernel");
    }
    PhaseScope ps(rec, 5, s);
    e = launch_gemv_down(ga, x_dtype, y_dtype, s);
    if (e != hipSuccess) return hip_fail(e, "one-token down kernel");
    return MOE_OK;
  }

  if (decode) {
    meta = (int32_t*)(pb + p->L.dmeta);
  } else {
    PhaseScope ps(rec, 0, s);
    ClassifyArgs ca{};
    ca.counts = (const int32_t*)(pb + p->L.counts);
    ca.n_exp = n_exp;
    ca.mode = wdt == MOE_F32 ? 0 : (q4_fmt(wdt) >= 0 ? 2 : 1);
    ca.S = (double)o.splitk_max_pairs;
    ca.full_nnb = F / 128;
    ca.full_fill = (ca.mode == 1 && !(o.flags & MOE_OPT_EXACT_ROUTES)) ? info.ncu : 0;
    ca.fat_rows = L.fat_rows;
    ca.full_tiles = (int32_t*)(b + L.full_tiles);
    ca.sk1 = (int32_t*)(b + L.sk1);
    ca.sk4 = (int32_t*)(b + L.sk4);
    ca.offsets = (const int32_t*)(pb + p->L.offsets);
    ca.pair_token = (const int32_t*)(pb + p->L.pair_token);
    ca.sk1_tok = L.stream ? (int32_t*)(b + L.sk1_tok) : nullptr;
    ca.sk4_tok = L.stream || ca.mode == 2 ? (int32_t*)(b + L.sk4_tok) : nullptr;
    ca.fat_slot = (int32_t*)(b + L.fat_slot);
    ca.fat_list = (int32_t*)(b + L.fat_list);
    ca.meta = meta;
    e = launch_classify(ca, s);
    if (e != hipSuccess) return hip_fail(e, "classify kernel");
  }
  // Routes that this prompt cannot use are not launched: an expert holds at
  // most T pairs (a token picks k distinct experts; the shared expert takes
  // every token), so with T <= S no expert leaves the split-K side, with
  // T < fat_rows none is fat, and with T <= 16 every split-K group is one
  // group of <= 16 rows (decode-shaped calls).
  const int64_t row_bound = d.T;
  const bool run_fat = !decode && L.can_fat && row_bound >= L.fat_rows;
  const bool run_full = !decode && L.can_full &&
      (q4_fmt(wdt) >= 0 ? run_fat : (double)row_bound > (double)o.splitk_max_pairs);
  const bool run_sk1 = L.can_sk1 || decode;
  const bool run_sk4 = !decode && L.can_sk4 && row_bound > 16;
  // Thin groups beside fat / full ones: their launches (weight-stream or
  // decode bound) run on the second stream, overlapping the dequantisation
  // and the full tiles, whose buffers they do not touch (they write H and
  // Ypair rows of their own pairs only). The fork and the join cost about
  // 20 us of dependency latency, so small layers stay on one stream: at
  // most T k D F = 2^33 multiply-adds a product (the skewed 2048-token
  // layer, 2^31, lost 23 us; the 4096-token prefill layer, 2^35.6, gained
  // 24 us; a short prompt whose full route the classify kernel empties
  // pays the fork for nothing).
  const bool fork = !(o.flags & MOE_OPT_ONE_STREAM) && (run_fat || run_full) &&
                    (run_sk1 || run_sk4) &&
                    (double)d.T * d.k * D * F > kForkMinWork;
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_lock;
  hipStream_t ts = s;   // the thin launches' stream
  // joins the second stream back into `stream` on every way out, errors
  // included, so nothing the call launched outlives it on `stream`'s order
  struct Join {
    SideStream* side = nullptr;
    hipStream_t s = nullptr;
    hipError_t run() {
      if (!side) return hipSuccess;
      hipError_t e = hipEventRecord(side->join, side->s);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
      side = nullptr;
      return e;
    }
    ~Join() { run(); }
  } join;
  if (fork) {
    side = side_stream(dev, &st);
    if (!side) return st;
    side_lock = std::unique_lock<std::mutex>(side->mu);
    e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return hip_fail(e, "fork of the second stream");
    ts = side->s;
    join.side = side;
    join.s = s;
  }
  const int32_t* sk1_list = decode ? (const int32_t*)(pb + p->L.dlist)
                                   : (const int32_t*)(b + L.sk1);
  const int32_t* sk1_tok = decode ? (const int32_t*)(pb + p->L.dtok)
                                  : (const int32_t*)(b + L.sk1_tok);
  if (run_fat) {
    PhaseScope ps(rec, 1, s);
    const int grid = info.ncu * 8;
    // one launch for the three matrices
    const void* const q[3] = {w_gate.data, w_up.data, w_down.data};
    const void* const sc[3] = {w_gate.scales, w_up.scales, w_down.scales};
    void* const out[3] = {b + L.stg_g, b + L.stg_u, b + L.stg_d};
    const int rows[3] = {F, F, D};
    const int Ks[3] = {D, D, F};
    e = launch_dequant_fat(q, sc, out, rows, Ks, 3,
                           (const int32_t*)(b + L.fat_list), meta, grid,
                           q4_fmt(wdt), s);
    if (e != hipSuccess) return hip_fail(e, "dequant kernel");
  }

  GemmArgs g{};
  g.offsets = (const int32_t*)(pb + p->L.offsets);
  g.pair_token = (const int32_t*)(pb + p->L.pair_token);
  g.pair_w = (const float*)(pb + p->L.pair_w);
  g.meta = meta;
  g.clamp = o.swiglu_limit;
  g.fat_slot = L.can_fat ? (const int32_t*)(b + L.fat_slot) : nullptr;
  void* H = b + L.H;
  void* H2 = L.split_h ? b + L.H2 : nullptr;
  void* Y = b + L.Y;
  const int sk_rb1_grid_cap = info.ncu * 8;
  const int sk_rb4_grid_cap = info.ncu * 4;
  const int full_grid_cap = info.ncu;      // one 128 KB-LDS block per CU

  for (int stage = 0; stage < 2; ++stage) {
    g.mode = stage;
    if (stage == 0) {
      g.K = D; g.N = F; g.A = x; g.A2 = nullptr; g.out = H; g.out2 = H2;
      g.a_bytes = (uint32_t)((size_t)d.T * D * xbytes(x_dtype));
      g.a_ld = D; g.out_ld = L.h_ld;
      g.B0 = w_gate.data; g.B0s = w_gate.scales;
      g.B1 = w_up.data; g.B1s = w_up.scales;
      g.S0 = b + L.stg_g; g.S1 = b + L.stg_u;
    } else {
      g.K = F; g.N = D; g.A = H; g.A2 = H2; g.out = Y; g.out2 = nullptr;
      g.a_bytes = (uint32_t)(Pmax_rows * L.h_ld * xbytes(x_dtype));
      g.a_ld = L.h_ld; g.out_ld = D;
      g.B0 = w_down.data; g.B0s = w_down.scales;
      g.B1 = nullptr; g.B1s = nullptr;
      g.S0 = b + L.stg_d; g.S1 = nullptr;
    }
    if (run_full) {
      PhaseScope ps(rec, stage == 0 ? 2 : 4, s);
      const int nnb = stage == 0 ? F / 128 : (D + 255) / 256;
      GemmArgs gf = g;
      gf.h_rows = (int)Pmax_rows;
      void* Ht = b + L.Ht;
      void* Ht2 = L.split_h ? b + L.Ht2 : nullptr;
      if (stage == 0) {
        gf.out = Ht; gf.out2 = Ht2;
      } else {
        gf.A = Ht; gf.A2 = Ht2;
        gf.a_bytes = (uint32_t)(Pmax_rows * F * xbytes(x_dtype));
      }
      gf.list = (const int32_t*)(b + L.full_tiles);
      gf.meta_index = kMetaFullTiles;
      gf.queue = meta + (stage == 0 ? kMetaQueueGateUp : kMetaQueueDown);
      const int grid = (int)std::min<int64_t>((int64_t)L.cap_tiles * nnb, full_grid_cap);
      e = launch_gemm_full(gf, x_dtype, grid, s);
      if (e != hipSuccess) return hip_fail(e, "full tile kernel");
    }
    {
      const int nnb = stage == 0 ? F / 32 : D / 64;
      if (L.stream) {
        g.part = (float*)(b + L.part);
        g.fix = meta + kMetaFix;
      }
      const int stream_grid1 = std::min(info.ncu, stream_max_runs(1));
      const int stream_grid4 = std::min(info.ncu, stream_max_runs(4));
      if (run_sk1) {
        // groups of <= 16 rows
        PhaseScope ps(rec, stage == 0 ? 3 : 5, ts);
        g.list = sk1_list;
        g.meta_index = kMetaSk1;
        if (L.stream) {
          g.tok = sk1_tok;
          // a decode-shaped call has at most T k + n_shared groups: when
          // their items fit one workgroup each on the GPU, the launch takes
          // them whole (no partial sums, no fix-up)
          const int64_t max_items =
              (int64_t)std::min<int64_t>(n_exp, (int64_t)d.T * d.k + d.n_shared) *
              (stage == 0 ? F / 64 : D / 128);
          GemmArgs gs = g;
          int grid = stream_grid1;
          if (decode && max_items <= info.ncu) {
            gs.part = nullptr;
            grid = (int)max_items;
          }
          e = launch_gemm_stream(gs, x_dtype, wdt, 16, grid, ts);
        } else {
          // the 4-bit tile: four times the workgroups that fit the GPU at
          // once, one or two items each, so the hardware's dispatch evens
          // out the end of the launch (down 148 -> 141 us at the 13K-token
          // layer; with only the resident four per CU, 5 % slower)
          const int cap = q4_fmt(wdt) >= 0 ? info.ncu * 16 : sk_rb1_grid_cap;
          // each group holds a pair: at most T k + n_shared groups
          const int64_t groups = std::min<int64_t>(L.cap_sk1, (int64_t)d.T * d.k + d.n_shared);
          const int grid = (int)std::min<int64_t>(groups * nnb, cap);
          e = launch_gemm_splitk(g, x_dtype, wdt, 1, grid, ts);
        }
        if (e != hipSuccess) return hip_fail(e, "split-K kernel");
      }
      if (run_sk4) {
        // groups of 17..64 rows
        PhaseScope ps(rec, stage == 0 ? 14 : 15, ts);
        g.list = (const int32_t*)(b + L.sk4);
        g.meta_index = kMetaSk4;
        if (x_dtype == MOE_F32) {
          const int grid = (int)std::min<int64_t>((int64_t)L.cap_sk4 * nnb, sk_rb4_grid_cap);
          e = launch_gemm_splitk(g, x_dtype, wdt, 4, grid, ts);
        } else if (L.stream) {
          g.tok = (const int32_t*)(b + L.sk4_tok);
          e = launch_gemm_stream(g, x_dtype, wdt, kStreamTokRows, stream_grid4, ts);
        } else {
          // wide fused-dequant tile, 256 columns per item
          g.tok = (const int32_t*)(b + L.sk4_tok);
          const int wnb = stage == 0 ? (F + 127) / 128 : (D + 255) / 256;
          const int grid = (int)std::min<int64_t>((int64_t)L.cap_sk4 * wnb, info.ncu * 2);
          e = launch_gemm_wide(g, x_dtype, wdt, grid, ts);
        }
        if (e != hipSuccess) return hip_fail(e, "split-K kernel");
      }
    }
  }
  {
    e = join.run();
    if (e != hipSuccess) return hip_fail(e, "join of the second stream");
    PhaseScope ps(rec, 6, s);
    e = launch_combine(Y, x_dtype == MOE_F16, (const int32_t*)(pb + p->L.tok2pair),
                       (const float*)(pb + p->L.w),
                       (const int32_t*)(pb + p->L.offsets), d.T, D, d.k,
                       d.n_shared, d.E, y_dtype, y, s);
    if (e != hipSuccess) return hip_fail(e, "combine kernel");
  }
  return MOE_OK;
}

moe_status moe_forward_get_views(const moe_plan* p, int32_t D, int32_t F,
                                 int32_t x_dtype, int32_t w_dtype,
                                 const moe_options* opt, const void* ws,
                                 moe_forward_views* v) {
  if (!p || !ws || !v) return fail(MOE_EINVAL, "NULL plan, workspace or views");
  if (D <= 0 || F <= 0 || D % 128 || F % 128 || !dtypes_ok(x_dtype, w_dtype))
    return fail(MOE_EINVAL, "bad sizes or dtypes for the forward views");
  const moe_options o = opt ? *opt : defaults();
  const FwdLayout L = fwd_layout(p->desc, D, F, x_dtype, w_dtype, o);
  const char* b = static_cast<const char*>(ws);
  const bool fat = L.max_fat > 0;
  v->h = b + L.H;
  v->h_lo = L.split_h ? b + L.H2 : nullptr;
  v->h_ld = L.h_ld;
  v->ht = L.can_full ? b + L.Ht : nullptr;
  v->ht_lo = L.can_full && L.split_h ? b + L.Ht2 : nullptr;
  v->pairs_max = (int64_t)p->desc.T * p->desc.k + (int64_t)p->desc.n_shared * p->desc.T;
  v->ypair = b + L.Y;
  v->ypair_dtype = x_dtype == MOE_F16 ? MOE_F16 : MOE_F32;
  v->fat_slot = L.can_fat ? reinterpret_cast<const int32_t*>(b + L.fat_slot) : nullptr;
  v->fat_copy[0] = fat ? b + L.stg_g : nullptr;
  v->fat_copy[1] = fat ? b + L.stg_u : nullptr;
  v->fat_copy[2] = fat ? b + L.stg_d : nullptr;
  v->fat_slots = L.max_fat;
  return MOE_OK;
}

size_t moe_backward_workspace_bytes(const moe_plan* p, int32_t D, int32_t F,
                                    int32_t x_dtype) {
  if (!p) { fail(MOE_EINVAL, "plan is NULL"); return 0; }
  if (x_dtype != MOE_BF16 && x_dtype != MOE_F16) {
    fail(MOE_EUNSUPPORTED, "backward supports bf16 and f16 layers"); return 0;
  }
  if (D <= 0 || F <= 0 || D % 128 || F % 128) {
    fail(MOE_EINVAL, "D and F must be positive multiples of 128"); return 0;
  }
  const moe_plan_desc& d = p->desc;
  const int64_t Pmax = (int64_t)d.T * d.k + (int64_t)d.n_shared * d.T;
  return bwd_workspace_bytes(Pmax, d.E + d.n_shared, D, F) +
         align256((size_t)d.T * d.k * 4);
}

moe_status moe_backward(const moe_plan* p, const void* x, int32_t x_dtype,
                        moe_weight w_gate, moe_weight w_up, moe_weight w_down,
                        int32_t D, int32_t F, const float* dy, float* dx,
                        float* dw_gate, float* dw_up, float* dw_down,
                        float* d_topk_w, float* d_logits, void* ws,
                        size_t ws_bytes, const moe_options* opt, void* stream) {
  if (!p) return fail(MOE_EINVAL, "plan is NULL");
  const moe_plan_desc& d = p->desc;
  const size_t need = moe_backward_workspace_bytes(p, D, F, x_dtype);
  if (need == 0) return x_dtype != MOE_BF16 && x_dtype != MOE_F16 ? MOE_EUNSUPPORTED : MOE_EINVAL;
  std::string why;
  if (w_gate.dtype != x_dtype)
    return fail(MOE_EUNSUPPORTED, "backward needs weights in x's dtype (16-bit)");
  if (!weight_ok(w_gate, x_dtype, &why, "w_gate") ||
      !weight_ok(w_up, x_dtype, &why, "w_up") ||
      !weight_ok(w_down, x_dtype, &why, "w_down"))
    return fail(MOE_EINVAL, "%s", why.c_str());
  if (!dw_gate || !dw_up || !dw_down || (d.T > 0 && (!x || !dy || !dx)))
    return fail(MOE_EINVAL, "x, dy, dx and the three weight gradients must be non-NULL");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(dw_gate) ||
      !aligned16(dw_up) || !aligned16(dw_down) || !aligned16(d_topk_w) ||
      !aligned16(d_logits) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(MOE_EINVAL, "pointers must be 16-byte and ws 256-byte aligned");
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "backward workspace %zu bytes < %zu needed", ws_bytes, need);
  {
    // the products address x and the per-pair 16-bit operands with 31-bit
    // buffer offsets
    const size_t Pmax = (size_t)d.T * d.k + (size_t)d.n_shared * d.T;
    const size_t lim31 = ((size_t)1 << 31) - 1;
    if ((size_t)d.T * D * 2 > lim31 || Pmax * std::max(2 * F, D) * 2 > lim31 ||
        (size_t)D * F * 2 > lim31)
      return fail(MOE_EUNSUPPORTED, "x, each per-pair operand (pairs x max(2F, D) "
                  "16-bit values) and each weight matrix must stay below 2 GiB");
  }
  const moe_options o = opt ? *opt : defaults();
  int dev;
  DevInfo info;
  moe_status st = device_info(&dev, &info);
  if (st != MOE_OK) return st;
  const char* pb = p->ws;
  BwdArgs a{};
  a.xdt = x_dtype; a.T = d.T; a.D = D; a.F = F; a.E = d.E; a.k = d.k;
  a.n_shared = d.n_shared; a.n_exp = d.E + d.n_shared;
  a.Pmax = (int64_t)d.T * d.k + (int64_t)d.n_shared * d.T;
  a.ncu = info.ncu;
  a.x = x; a.dy = dy; a.wg = w_gate.data; a.wu = w_up.data; a.wd = w_down.data;
  a.clamp = o.swiglu_limit;
  a.offsets = (const int32_t*)(pb + p->L.offsets);
  a.pair_token = (const int32_t*)(pb + p->L.pair_token);
  a.pair_w = (const float*)(pb + p->L.pair_w);
  a.tok2pair = (const int32_t*)(pb + p->L.tok2pair);
  a.ids = (const int32_t*)(pb + p->L.ids);
  a.topk_w = (const float*)(pb + p->L.w);
  a.dx = dx; a.dwg = dw_gate; a.dwu = dw_up; a.dwd = dw_down;
  a.dtw = d_topk_w; a.dlogits = d_logits;
  char* b = static_cast<char*>(ws);
  a.ws = b;
  a.dtw_scratch = reinterpret_cast<float*>(b + bwd_workspace_bytes(a.Pmax, a.n_exp, D, F));
  PhaseRecord* rec = nullptr;
  if (o.flags & MOE_OPT_PHASE_EVENTS) {
    rec = acquire_record(o.flags, &st);
    if (!rec) return st;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int stage = 0; stage < 4; ++stage) {
    hipError_t e;
    {
      PhaseScope ps(rec, 10 + stage, s);
      e = launch_backward(a, stage, s);
    }
    if (e != hipSuccess) return hip_fail(e, "backward kernels");
  }
  return MOE_OK;
}

moe_status moe_dequant_q4(const void* data, const void* scales, int64_t rows,
                          int64_t K, void* out_f16, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return fail(MOE_EINVAL, "rows >= 0 and K a positive multiple of 32");
  if (K > (1 << 30)) return fail(MOE_EUNSUPPORTED, "K too large");
  if (rows == 0) return MOE_OK;
  if (!data || !scales || !out_f16) return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned16(data) || !aligned16(out_f16) || (reinterpret_cast<uintptr_t>(scales) & 1u))
    return fail(MOE_EINVAL, "data/out must be 16-byte aligned, scales 2-byte");
  hipError_t e = launch_dequant_rows(data, scales, out_f16, rows, (int)K, 0,
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequant kernel");
  return MOE_OK;
}

moe_status moe_dequant_weights(int32_t dtype, const void* data,
                               const void* scales, int64_t rows, int64_t K,
                               void* out_f16, void* stream) {
  const int fmt = q4_fmt(dtype);
  if (fmt < 0) return fail(MOE_EUNSUPPORTED, "dtype %d is not a 4-bit format", dtype);
  const int G = dtype == MOE_Q4A64 ? 64 : 32;
  if (rows < 0 || K <= 0 || K % G)
    return fail(MOE_EINVAL, "rows >= 0 and K a positive multiple of %d", G);
  if (K > (1 << 30)) return fail(MOE_EUNSUPPORTED, "K too large");
  if (rows == 0) return MOE_OK;
  if (!data || !scales || !out_f16) return fail(MOE_EINVAL, "NULL pointer");
  const uintptr_t al = fmt == 0 ? 1u : 3u;
  if (!aligned16(data) || !aligned16(out_f16) ||
      (reinterpret_cast<uintptr_t>(scales) & al))
    return fail(MOE_EINVAL, "data/out must be 16-byte aligned, scales %d-byte", (int)al + 1);
  hipError_t e = launch_dequant_rows(data, scales, out_f16, rows, (int)K, fmt,
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequant kernel");
  return MOE_OK;
}

moe_status moe_phase_times(double* ms, int32_t n, int64_t* calls, int32_t reset) {
  std::lock_guard<std::mutex> lock(g_ev_mu);
  std::vector<double> acc(MOE_N_PHASES, 0.0);
  for (size_t i = 0; i < g_records_used; ++i) {
    PhaseRecord& r = g_records[i];
    for (int ph = 0; ph < MOE_N_PHASES; ++ph) {
      if (!r.used[ph]) continue;
      hipError_t e = hipEventSynchronize(r.ev[2 * ph + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      float t = 0.f;
      e = hipEventElapsedTime(&t, r.ev[2 * ph], r.ev[2 * ph + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      acc[ph] += t;
    }
  }
  if (ms)
    for (int i = 0; i < n && i < MOE_N_PHASES; ++i) ms[i] = acc[i];
  if (calls) *calls = (int64_t)g_records_used;
  if (reset) g_records_used = 0;
  return MOE_OK;
}

}  // extern "C"
