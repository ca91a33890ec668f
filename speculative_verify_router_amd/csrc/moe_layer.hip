// C-ABI entry points of the routed-MoE verify layer (declared in
// include/moe_layer.h): argument validation, workspace layout, kernel
// selection and the launch sequence on the caller's HIP stream.
//
// Two launch sequences:
//  * staged (up to 16 tokens), three stages, each one launch where a fused
//    instantiation exists:
//      1 route_shared_gateup  router GEMV + shared gate/up; the grid's last
//                             workgroup: top-k, weights, bucketing
//      2 gateup               routed gate/up + SwiGLU, shared down
//      3 down_combine         routed down; last workgroup per row tile
//                             combines
//    Shapes outside the fused instantiations take the same steps as
//    separate launches.
//  * batched (more than 16 tokens), three stages of several launches:
//      1 route          router GEMM (fp32 MFMA), top-k, bucketing, token
//                       tiles, bf16 hi/lo split of x
//      2 gateup         shared and routed gate/up + SwiGLU as grouped GEMMs
//                       (bf16 MFMA)
//      3 down_combine   shared and routed down GEMMs, combine
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <unordered_map>

#include "common.h"
#include "ffn.h"
#include "gemm.h"
#include "misc.h"
#include "phases.h"
#include "route.h"
#include "launch.h"

using namespace svr;
using namespace svr::host;

namespace {

constexpr int kVersion = 400;  // 0.4.0
constexpr int kFusedMaxTokens = 16;

enum Stage { kStPhase1 = 0, kStPhase2, kStPhase3, kNumStages };
const char* const kStageNames[kNumStages] = {"route_shared_gateup", "gateup", "down_combine"};

struct Plan {
  int H, E, k, F, Fs, et, st, dt, M, flags;  // dt: routed down type
  size_t ctr, keys, logits, ids, w, ptok, counts, offsets, slots, active, nactive, h, hs, o, s, xs,
      tiles, total;
  int tiles_cap;  // routed token tiles of the batched path, at most
};

int check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->ffn <= 0 || d->shared_ffn < 0)
    return MOE_ERR_SHAPE;
  if (d->flags != 0) return MOE_ERR_ARG;
  if (!routed_type(d->expert_type)) return MOE_ERR_DTYPE;
  if (d->down_type != 0 && !routed_type(d->down_type)) return MOE_ERR_DTYPE;
  if (d->shared_ffn > 0 && !quant_type(d->shared_type)) return MOE_ERR_DTYPE;
  if (d->n_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (d->top_k > d->n_experts || d->top_k > kMaxTopK) return MOE_ERR_SHAPE;
  FfnShape s;
  const int dt = d->down_type ? d->down_type : d->expert_type;
  if (!ffn_shape(d->expert_type, d->hidden, &s) || !ffn_shape(dt, d->ffn, &s))
    return MOE_ERR_SHAPE;
  if (d->shared_ffn > 0 &&
      (!ffn_shape(d->shared_type, d->hidden, &s) || !ffn_shape(d->shared_type, d->shared_ffn, &s)))
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

int make_plan(const moe_layer_desc* d, int M, Plan* p) {
  const int rc = check_desc(d);
  if (rc != MOE_OK) return rc;
  if (M < 0) return MOE_ERR_NULL;
  p->H = d->hidden;
  p->E = d->n_experts;
  p->k = d->top_k;
  p->F = d->ffn;
  p->Fs = d->shared_ffn;
  p->et = d->expert_type;
  p->dt = d->down_type ? d->down_type : d->expert_type;
  p->st = d->shared_type;
  p->flags = d->flags;
  p->M = M;
  const size_t Mz = (size_t)M, P = Mz * p->k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  // Hand-off areas, zero between calls, at offsets that depend on E only
  // (so that calls of any batch size agree on them): counters, then the
  // routing keys of up to kFusedMaxTokens tokens.
  p->ctr = take(kCounterBytes);
  p->keys = take((size_t)p->E * kFusedMaxTokens * 4);
  p->logits = take(Mz * p->E * 4);
  p->ids = take(P * 4);
  p->w = take(P * 4);
  p->ptok = take(P * 8);
  p->counts = take((size_t)p->E * 4);
  p->offsets = take((size_t)(p->E + 1) * 4);
  p->slots = take(P * 4);
  p->active = take((size_t)p->E * 4);
  p->nactive = take(4);
  p->h = take(P * p->F * 4);
  p->hs = take(Mz * p->Fs * 4);
  p->o = take(P * p->H * 4);
  p->s = take(Mz * p->H * 4);
  // Batched path: x split into bf16 hi/lo terms, and the routed token tiles
  // (every active expert has at most one partial tile).
  p->xs = take(Mz * p->H * 4);
  p->tiles_cap = (int)(std::min<size_t>(P, (size_t)p->E) + P / 16);
  p->tiles = take((size_t)(3 * p->tiles_cap + 1) * 4);
  p->total = off;
  return MOE_OK;
}

// Phase 1: router rows (NC float4 per lane) + shared gate/up tiles in the
// rest of one resident round.
template <int NC>
bool launch_phase1_nc(int skey, hipStream_t st, const RouteArgs& r, FfnArgs s, int sdtype) {
  switch (skey) {
#define SVR_P1(F, C, L)                                                                  \
  case key(F, shape_code(C, L)): {                                                       \
    auto k = k_phase1<NC, F, shape_code(C, L)>;                                          \
    const int64_t cap = resident_blocks(k);                                              \
    size_shared_tiles(s, sdtype, std::max<int64_t>(cap - r.n_router_blocks - 1, cap / 4)); \
    hipLaunchKernelGGL(k, dim3(r.n_router_blocks + tiles_of(s) + 1), dim3(kBlock), 0, st, r, \
                       s);                                                               \
    return true;                                                                         \
  }
    case 0:
      hipLaunchKernelGGL((k_phase1<NC, 0, 1>), dim3(r.n_router_blocks + 1), dim3(kBlock), 0, st,
                         r, s);
      return true;
    SVR_P1(kQ8_0, 4, 64)
    SVR_P1(kQ8_0, 1, 0) SVR_P1(kQ8_0, 2, 0) SVR_P1(kQ8_0, 4, 0) SVR_P1(kQ8_0, 5, 0)
    SVR_P1(kQ4_K, 1, 0) SVR_P1(kQ4_K, 2, 0)
#undef SVR_P1
    default: return false;
  }
}

// NC: float4 chunks per lane in a quarter row (H/16 chunks per quarter).
bool launch_phase1_k(int H, int skey, hipStream_t st, const RouteArgs& r, const FfnArgs& s,
                     int sdtype) {
  if (H <= 1024) return launch_phase1_nc<1>(skey, st, r, s, sdtype);
  if (H <= 2048) return launch_phase1_nc<2>(skey, st, r, s, sdtype);
  if (H <= 4096) return launch_phase1_nc<4>(skey, st, r, s, sdtype);
  if (H <= 8192) return launch_phase1_nc<8>(skey, st, r, s, sdtype);
  return false;
}

// sshape: the shared gate/up lane shape (ignored without a shared expert).
bool launch_phase1(int H, bool shared, int sdtype, const FfnShape& sshape, hipStream_t st,
                   const RouteArgs& r, const FfnArgs& s) {
  if (!shared) return launch_phase1_k(H, 0, st, r, s, sdtype);
  return launch_phase1_k(H, exact_key(sdtype, sshape), st, r, s, sdtype) ||
         launch_phase1_k(H, generic_key(sdtype, sshape), st, r, s, sdtype);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Records stage event i if the caller asked for events; a failure shows up
// in the final hipGetLastError check.
inline void mark(hipEvent_t* ev, int i, hipStream_t st) {
  if (ev && ev[i]) (void)hipEventRecord(ev[i], st);
}

struct Buffers {
  Counters* ctr;
  uint32_t* keys;
  uint2* ptok;
  float *logits, *w, *h, *hs, *o, *s;
  int32_t *ids, *counts, *offsets, *slots, *active, *nactive, *tiles, *ntiles;
  uint4* xs;
};

Buffers carve(const Plan& p, void* ws, int32_t* ids, float* w) {
  uint8_t* b = (uint8_t*)ws;
  Buffers r;
  r.ctr = (Counters*)(b + p.ctr);
  r.keys = (uint32_t*)(b + p.keys);
  r.logits = (float*)(b + p.logits);
  r.ids = ids ? ids : (int32_t*)(b + p.ids);
  r.w = w ? w : (float*)(b + p.w);
  r.ptok = (uint2*)(b + p.ptok);
  r.counts = (int32_t*)(b + p.counts);
  r.offsets = (int32_t*)(b + p.offsets);
  r.slots = (int32_t*)(b + p.slots);
  r.active = (int32_t*)(b + p.active);
  r.nactive = (int32_t*)(b + p.nactive);
  r.h = (float*)(b + p.h);
  r.hs = (float*)(b + p.hs);
  r.o = (float*)(b + p.o);
  r.s = (float*)(b + p.s);
  r.xs = (uint4*)(b + p.xs);
  r.tiles = (int32_t*)(b + p.tiles);
  r.ntiles = r.tiles + 3 * p.tiles_cap;
  return r;
}

// Router logits of a batch: the fp32 MFMA GEMM above the fused batch
// sizes (H a multiple of 64), else a wave per expert row.
void enqueue_logits(const Plan& p, const float* router, const float* x, float* logits,
                    hipStream_t st) {
  if (p.M > kFusedMaxTokens && p.H % 64 == 0) {
    const dim3 grid((p.M + 31) / 32, (p.E + 31) / 32);
    if (p.H == 4096)
      hipLaunchKernelGGL(k_router_mfma<64>, grid, dim3(kBlock), 0, st, router, x, logits, p.H, p.E, p.M);
    else
      hipLaunchKernelGGL(k_router_mfma<0>, grid, dim3(kBlock), 0, st, router, x, logits, p.H, p.E, p.M);
    return;
  }
  hipLaunchKernelGGL(k_router_logits, dim3((p.E + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(kBlock), 0, st, router, x, logits, p.H, p.E, p.M);
}

// Router + top-k + bucketing as three launches (any batch size).
void enqueue_route_plain(const Plan& p, const float* router, const float* x, const Buffers& b,
                         const BucketOut& bo, hipStream_t st) {
  enqueue_logits(p, router, x, b.logits, st);
  hipLaunchKernelGGL(k_topk, dim3((p.M + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0,
                     st, b.logits, b.ids, b.w, p.E, p.k, p.M);
  if (p.M * p.k > 256)
    hipLaunchKernelGGL(k_bucket_wide, dim3(1), dim3(kWideBlock), 0, st, b.ids, p.M * p.k, p.E, bo);
  else
    hipLaunchKernelGGL(k_bucket, dim3(1), dim3(kBlock), 0, st, b.ids, p.M * p.k, p.E, bo);
}

FfnArgs shared_gateup_args(const Plan& p, const moe_layer_weights* wt, const float* x,
                           const Buffers& b) {
  FfnArgs a{};
  a.w0 = (const uint8_t*)wt->shared_gate;
  a.w1 = (const uint8_t*)wt->shared_up;
  a.total_rows = p.Fs;
  a.rows_per_expert = p.Fs;
  a.K = p.H;
  a.n_tokens = p.M;
  a.top_k = 1;
  a.act = x;
  a.act_by_pair = 0;
  a.out = b.hs;
  a.split_tokens = 1;
  return a;
}

FfnArgs shared_down_args(const Plan& p, const moe_layer_weights* wt, const Buffers& b) {
  FfnArgs a{};
  a.w0 = (const uint8_t*)wt->shared_down;
  a.total_rows = p.H;
  a.rows_per_expert = p.H;
  a.K = p.Fs;
  a.n_tokens = p.M;
  a.top_k = 1;
  a.act = b.hs;
  a.act_by_pair = 1;
  a.out = b.s;
  a.split_tokens = 1;
  return a;
}

FfnArgs routed_args(const Plan& p, const Buffers& b, bool gateup, const moe_layer_weights* wt,
                    const float* x, bool pairs) {
  FfnArgs a{};
  if (pairs) {
    a.pair_expert = b.ids;
    a.n_pairs = p.M * p.k;
    // gate/up of two or more tokens: one pass per expert over all of its
    // tokens
    if (gateup && p.M > 1) a.pair_info = b.ptok;
  } else {
    a.active = b.active;
    a.n_active = b.nactive;
    a.offsets = b.offsets;
    a.slots = b.slots;
  }
  a.top_k = p.k;
  a.split_tokens = 0;
  if (gateup) {
    a.w0 = (const uint8_t*)wt->gate;
    a.w1 = (const uint8_t*)wt->up;
    a.total_rows = (int64_t)p.E * p.F;
    a.rows_per_expert = p.F;
    a.K = p.H;
    a.act = x;
    a.act_by_pair = 0;
    a.out = b.h;
  } else {
    a.w0 = (const uint8_t*)wt->down;
    a.total_rows = (int64_t)p.E * p.H;
    a.rows_per_expert = p.H;
    a.K = p.F;
    a.act = b.h;
    a.act_by_pair = 1;
    a.out = b.o;
  }
  // Batches above the fused sizes (types without a matrix-core path) make
  // one token pass per token of an expert over the same rows: tiles of
  // about 64 KB of weights stay in L2 from pass to pass.
  if (p.M > kFusedMaxTokens) {
    const double rb = gateup ? 2.0 * row_bytes(p.et, p.H) : row_bytes(p.dt, p.F);
    a.max_rows = (int)std::max(1.0, 65536.0 / rb);
  }
  return a;
}

// ---- Batched path: grouped GEMMs on the matrix cores.
constexpr int kGemmGateUpRtr = 2;  // row tiles of 16 per wave and matrix
constexpr int kGemmDownRtr = 4;
constexpr int kGemmQ8Rtr = 1;
constexpr int kGemmQ8DenseDownRtr = 2;  // the shared down: one round of two per CU
// Stages of the batched path; the shared expert's GEMMs are stages of their
// own (empty without one), so that "gateup" is the routed gate/up GEMM alone.
constexpr int kGemmStages = 5;
const char* const kGemmStageNames[kGemmStages] = {"route", "shared_gateup", "gateup",
                                                   "shared_down", "down_combine"};

bool gemm_path(const Plan& p) {
  if (p.M <= kFusedMaxTokens) return false;
  // every routed type has a matrix-core decoder; gate/up and down may differ
  // Split activations and h are addressed with 32-bit byte offsets.
  const int64_t P = (int64_t)p.M * p.k;
  if (P * std::max(p.H, p.F) * 4 >= (1ll << 31)) return false;
  if ((int64_t)p.M * std::max(p.H, p.Fs) * 4 >= (1ll << 31)) return false;
  return true;
}

template <int FMT, bool GU, int RTR, int TT = 1>
void launch_gemm_t(GemmArgs a, int tiles_cap, hipStream_t st) {
  const int per = kWavesPerBlock * 16 * RTR;
  a.row_blocks = (a.rows + per - 1) / per;
  const int t8 = ((tiles_cap + TT - 1) / TT + 7) & ~7;  // work units, rounded up to 8
  hipLaunchKernelGGL((k_gemm<FMT, GU, RTR, TT>), dim3((unsigned)(t8 * a.row_blocks)),
                     dim3(kBlock), 0, st, a);
}

void launch_gemm(int dtype, bool gateup, const GemmArgs& a, int tiles_cap, hipStream_t st) {
  if (dtype == MOE_Q2_K) {
    if (gateup) launch_gemm_t<kQ2_K, true, kGemmGateUpRtr>(a, tiles_cap, st);
    else launch_gemm_t<kQ2_K, false, kGemmDownRtr>(a, tiles_cap, st);
  } else if (dtype == MOE_Q3_K) {
    // Q3_K and Q6_K keep two product tiles per row tile (one per half step)
    if (gateup) launch_gemm_t<kQ3_K, true, 1>(a, tiles_cap, st);
    else launch_gemm_t<kQ3_K, false, 2>(a, tiles_cap, st);
  } else if (dtype == MOE_Q6_K) {
    if (gateup) launch_gemm_t<kQ6_K, true, 1>(a, tiles_cap, st);
    else launch_gemm_t<kQ6_K, false, 2>(a, tiles_cap, st);
  } else if (dtype == MOE_Q4_K) {
    if (gateup) launch_gemm_t<kQ4_K, true, kGemmGateUpRtr>(a, tiles_cap, st);
    else launch_gemm_t<kQ4_K, false, kGemmDownRtr>(a, tiles_cap, st);
  } else if (!a.tiles) {
    // The dense token list (the shared expert): two token tiles per
    // workgroup share each weight operand it builds.  The down GEMM's waves
    // take two row tiles: at 512 tokens and H = 4096 its grid is then one
    // resident round (38 us against 52 us with one row tile: 1.33 rounds).
    if (gateup) launch_gemm_t<kQ8_0, true, kGemmQ8Rtr, 2>(a, tiles_cap, st);
    else launch_gemm_t<kQ8_0, false, kGemmQ8DenseDownRtr, 2>(a, tiles_cap, st);
  } else {
    // Q8_0 weight slabs are twice as long: fewer row tiles per wave keep
    // two workgroups per CU.
    if (gateup) launch_gemm_t<kQ8_0, true, kGemmQ8Rtr>(a, tiles_cap, st);
    else launch_gemm_t<kQ8_0, false, kGemmQ8Rtr>(a, tiles_cap, st);
  }
}

void forward_gemm(const Plan& p, const moe_layer_weights* wt, const float* x, float* y,
                  const Buffers& b, hipStream_t st, hipEvent_t* ev) {
  const bool shared = p.Fs > 0;
  const int P = p.M * p.k;
  const int dense_tiles = (p.M + 15) / 16;

  mark(ev, 0, st);
  const BucketOut bo{b.counts, b.offsets, b.slots, b.active, b.nactive};
  enqueue_route_plain(p, wt->router, x, b, bo, st);
  hipLaunchKernelGGL(k_tiles, dim3(1), dim3(kBlock), 0, st, b.offsets, p.E,
                     TileList{b.tiles, b.ntiles});
  const int64_t n8 = (int64_t)p.M * p.H / 8;
  hipLaunchKernelGGL(k_split_act, dim3((unsigned)((n8 + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                     st, x, n8, b.xs);

  mark(ev, 1, st);
  if (shared) {
    GemmArgs a{};
    a.w0 = (const uint8_t*)wt->shared_gate;
    a.w1 = (const uint8_t*)wt->shared_up;
    a.total_rows = p.Fs;
    a.rows = p.Fs;
    a.K = p.H;
    a.act = b.xs;
    a.act_rows = p.M;
    a.out = b.hs;
    a.dense_tokens = p.M;
    launch_gemm(p.st, true, a, dense_tiles, st);
  }
  mark(ev, 2, st);
  {
    GemmArgs a{};
    a.w0 = (const uint8_t*)wt->gate;
    a.w1 = (const uint8_t*)wt->up;
    a.total_rows = (int64_t)p.E * p.F;
    a.rows = p.F;
    a.K = p.H;
    a.act = b.xs;
    a.act_rows = p.M;
    a.out = b.h;
    a.tiles = b.tiles;
    a.n_tiles = b.ntiles;
    a.slots = b.slots;
    a.top_k = p.k;
    a.act_gather = 1;
    launch_gemm(p.et, true, a, p.tiles_cap, st);
  }

  mark(ev, 3, st);
  if (shared) {
    GemmArgs a{};
    a.w0 = (const uint8_t*)wt->shared_down;
    a.total_rows = p.H;
    a.rows = p.H;
    a.K = p.Fs;
    a.act = reinterpret_cast<const uint4*>(b.hs);
    a.act_rows = p.M;
    a.out = b.s;
    a.dense_tokens = p.M;
    launch_gemm(p.st, false, a, dense_tiles, st);
  }
  mark(ev, 4, st);
  {
    GemmArgs a{};
    a.w0 = (const uint8_t*)wt->down;
    a.total_rows = (int64_t)p.E * p.H;
    a.rows = p.H;
    a.K = p.F;
    a.act = reinterpret_cast<const uint4*>(b.h);
    a.act_rows = P;
    a.out = b.o;
    a.tiles = b.tiles;
    a.n_tiles = b.ntiles;
    a.slots = b.slots;
    a.top_k = p.k;
    a.out_scatter = 1;
    launch_gemm(p.dt, false, a, p.tiles_cap, st);
  }
  const int64_t n4 = (int64_t)p.M * (p.H / 4);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n4 + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                     b.o, shared ? b.s : nullptr, b.w, y, p.M, p.H, p.k);
  mark(ev, 5, st);
}

int forward_impl(const moe_layer_desc* desc, const moe_layer_weights* wt, const float* x,
                 int32_t n_tokens, float* y, int32_t* topk_ids, float* topk_w, void* workspace,
                 size_t workspace_bytes, void* hip_stream, void* const* events, int32_t n_events) {
  if (!desc || !wt) return MOE_ERR_NULL;
  Plan p;
  int rc = make_plan(desc, n_tokens, &p);
  if (rc != MOE_OK) return rc;
  const int n_stages = gemm_path(p) ? kGemmStages : kNumStages;
  if (events && n_events != n_stages + 1) return MOE_ERR_ARG;
  hipStream_t st = (hipStream_t)hip_stream;
  hipEvent_t* ev = events ? (hipEvent_t*)events : nullptr;
  if (n_tokens == 0) {
    for (int i = 0; i <= n_stages; ++i) mark(ev, i, st);
    return MOE_OK;
  }
  if (!x || !y || !wt->router || !wt->gate || !wt->up || !wt->down) return MOE_ERR_NULL;
  if (p.Fs > 0 && (!wt->shared_gate || !wt->shared_up || !wt->shared_down)) return MOE_ERR_NULL;
  if (!workspace) return MOE_ERR_NULL;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256) || !aligned(x, 16) || !aligned(y, 16) || !aligned(wt->router, 16) ||
      !aligned(wt->gate, 16) || !aligned(wt->up, 16) || !aligned(wt->down, 16))
    return MOE_ERR_ARG;
  if (p.Fs > 0 && (!aligned(wt->shared_gate, 16) || !aligned(wt->shared_up, 16) ||
                   !aligned(wt->shared_down, 16)))
    return MOE_ERR_ARG;

  const Buffers b = carve(p, workspace, topk_ids, topk_w);
  if (gemm_path(p)) {
    (void)hipGetLastError();
    forward_gemm(p, wt, x, y, b, st, ev);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
  }
  const BucketOut bo{b.counts, b.offsets, b.slots, b.active, b.nactive};
  const bool pairs = p.M <= kPairTokens;
  // Pairs of several tokens may share experts: the routing gives each pair
  // its expert and token word (one token shares nothing).
  const bool share = pairs && p.M > 1;
  const int slots_max = pairs ? p.M * p.k : ((p.M * p.k < p.E) ? p.M * p.k : p.E);
  const bool shared = p.Fs > 0;
  (void)hipGetLastError();  // clear a stale error from earlier, unrelated calls

  // ---- stage 1: routing and shared gate/up
  mark(ev, kStPhase1, st);
  FfnArgs sgu{};
  FfnShape ss{};
  if (shared) {
    sgu = shared_gateup_args(p, wt, x, b);
    ffn_shape(p.st, p.H, &ss);
  }
  bool fused1 = false;
  if (p.M <= kFusedMaxTokens) {
    RouteArgs r{wt->router, x, b.keys, share ? b.ptok : nullptr, b.ids, b.w, bo, p.H, p.E, p.k,
                p.M, p.E, b.ctr, !pairs};
    fused1 = launch_phase1(p.H, shared, p.st, ss, st, r, sgu);
    if (!fused1 && shared) {
      // No fused instantiation for this shared shape: route alone, then the
      // shared gate/up as its own launch.
      fused1 = launch_phase1(p.H, false, p.st, ss, st, r, sgu);
      if (fused1 && !launch_ffn(p.st, true, sgu, 1, st)) return MOE_ERR_SHAPE;
    }
  }
  if (!fused1) {
    enqueue_route_plain(p, wt->router, x, b, bo, st);
    if (share)
      hipLaunchKernelGGL(k_pair_infos, dim3(1), dim3(kWave), 0, st, b.ids, b.ptok, p.M, p.k);
    if (shared && !launch_ffn(p.st, true, sgu, 1, st)) return MOE_ERR_SHAPE;
  }

  // ---- stage 2: routed gate/up (+ shared down)
  mark(ev, kStPhase2, st);
  {
    FfnArgs rgu = routed_args(p, b, true, wt, x, pairs);
    bool done = false;
    if (shared) {
      FfnArgs sd = shared_down_args(p, wt, b);
      FfnShape rs, ds;
      ffn_shape(p.et, p.H, &rs);
      ffn_shape(p.st, p.Fs, &ds);
      DualPlan dp;
      dp.a_work = (int64_t)(row_bytes(p.et, p.H) * 2 * p.F * slots_max);
      dp.b_work = (int64_t)(row_bytes(p.st, p.Fs) * p.H * (p.M < kWavesPerBlock ? p.M : kWavesPerBlock));
      dp.slots = slots_max;
      dp.adtype = p.et;
      dp.bdtype = p.st;
      done = launch_dual(p.et, rs, p.st, ds, st, rgu, sd, dp);
      if (!done) {
        if (!launch_ffn(p.et, true, rgu, slots_max, st)) return MOE_ERR_SHAPE;
        if (!launch_ffn(p.st, false, sd, 1, st)) return MOE_ERR_SHAPE;
        done = true;
      }
    }
    if (!done && !launch_ffn(p.et, true, rgu, slots_max, st)) return MOE_ERR_SHAPE;
  }

  // ---- stage 3: routed down + combine
  mark(ev, kStPhase3, st);
  {
    FfnArgs rd = routed_args(p, b, false, wt, x, pairs);
    rd.coherent_out = 1;  // the last workgroup of each row tile reads them
    FfnShape ds;
    ffn_shape(p.dt, p.F, &ds);
    CombineArgs c{b.o, shared ? b.s : nullptr, b.w, y, p.M, p.H, p.k, b.ctr};
    if (pairs && launch_down_tok(p.dt, ds, st, rd, c)) {
      // one workgroup per (token, row tile), combined in LDS
    } else if (!launch_down_combine(p.dt, ds, st, rd, c, slots_max)) {
      rd.coherent_out = 0;
      if (!launch_ffn(p.dt, false, rd, slots_max, st)) return MOE_ERR_SHAPE;
      const int64_t n4 = (int64_t)p.M * (p.H / 4);
      hipLaunchKernelGGL(k_combine, dim3((unsigned)((n4 + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                         st, b.o, shared ? b.s : nullptr, b.w, y, p.M, p.H, p.k);
    }
  }
  mark(ev, kNumStages, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// ---- Allocation-free entry point.  Its workspace is this file-scope device
// array: every GPU the library runs on holds one copy until the process
// ends, and every call on that GPU shares it.  Host code must not pass the
// array's name to a kernel (that is a host-side stand-in): the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and is used everywhere the host needs the array.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_MAX_WORKSPACE];

// Fill kernel for the scratch hand-off areas (no memset node, so that a
// caller may capture the first call in a graph).
static __global__ __launch_bounds__(kBlock) void k_zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * kBlock + threadIdx.x; i < n; i += gridDim.x * kBlock) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
// Hand-off areas at the start of any workspace: counters and the routing
// keys of the largest layer.
constexpr int kHandoffBytesMax = kCounterBytes + kMaxExperts * kFusedMaxTokens * 4;

// Device address of `scratch` on the current device: looked up on the first
// call on each device, when its hand-off areas are also cleared on `st`.
int scratch_address(hipStream_t st, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_LAUNCH;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_zero_words, dim3(kHandoffBytesMax / 4 / kBlock), dim3(kBlock), 0, st,
                       (uint32_t*)p, kHandoffBytesMax / 4);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_version(void) { return kVersion; }

const char* moe_strerror(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer or negative size";
    case MOE_ERR_SHAPE: return "unsupported shape";
    case MOE_ERR_DTYPE: return "unsupported tensor type";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

int32_t moe_tensor_bytes(int32_t dtype, int64_t rows, int64_t cols, int64_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  if (rows < 0 || cols < 0) return MOE_ERR_SHAPE;
  switch (dtype) {
    case MOE_F32: *bytes = 4 * rows * cols; return MOE_OK;
    case MOE_Q8_0:
      if (cols % 32) return MOE_ERR_SHAPE;
      *bytes = (int64_t)align256((size_t)(2 * rows * (cols / 32))) + rows * cols;
      return MOE_OK;
    case MOE_Q4_K:
      if (cols % 256) return MOE_ERR_SHAPE;
      *bytes = 144 * rows * (cols / 256);
      return MOE_OK;
    case MOE_Q2_K: {
      if (cols % 256) return MOE_ERR_SHAPE;
      const int64_t n = rows * (cols / 256);
      const int64_t s = (int64_t)align256((size_t)(4 * n));
      *bytes = (int64_t)align256((size_t)(s + 16 * n)) + 64 * n;
      return MOE_OK;
    }
    case MOE_Q3_K: {
      if (cols % 256) return MOE_ERR_SHAPE;
      const int64_t n = rows * (cols / 256);
      const int64_t s = (int64_t)align256((size_t)(2 * n));
      const int64_t l = (int64_t)align256((size_t)(s + 16 * n));
      *bytes = (int64_t)align256((size_t)(l + 64 * n)) + 32 * n;
      return MOE_OK;
    }
    case MOE_Q6_K: {
      if (cols % 256) return MOE_ERR_SHAPE;
      const int64_t n = rows * (cols / 256);
      const int64_t s = (int64_t)align256((size_t)(2 * n));
      const int64_t l = (int64_t)align256((size_t)(s + 16 * n));
      *bytes = (int64_t)align256((size_t)(l + 128 * n)) + 64 * n;
      return MOE_OK;
    }
    default: return MOE_ERR_DTYPE;
  }
}

int32_t moe_workspace_bytes(const moe_layer_desc* desc, int32_t max_tokens, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  Plan p;
  const int rc = make_plan(desc, max_tokens, &p);
  if (rc != MOE_OK) return rc;
  *bytes = p.total;
  return MOE_OK;
}

int32_t moe_stage_count(const moe_layer_desc* desc, int32_t n_tokens) {
  Plan p;
  const int rc = make_plan(desc, n_tokens, &p);
  if (rc != MOE_OK) return -rc;
  return gemm_path(p) ? kGemmStages : kNumStages;
}

const char* moe_stage_name(const moe_layer_desc* desc, int32_t n_tokens, int32_t i) {
  const int n = moe_stage_count(desc, n_tokens);
  if (n <= 0 || i < 0 || i >= n) return nullptr;
  Plan p;
  make_plan(desc, n_tokens, &p);
  return gemm_path(p) ? kGemmStageNames[i] : kStageNames[i];
}

int32_t moe_route(const moe_layer_desc* desc, const float* router, const float* x,
                  int32_t n_tokens, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                  int32_t* expert_offsets, int32_t* token_slots, int32_t* active_experts,
                  int32_t* n_active, void* workspace, size_t workspace_bytes, void* hip_stream) {
  Plan p;
  const int rc = make_plan(desc, n_tokens, &p);
  if (rc != MOE_OK) return rc;
  if (n_tokens == 0) return MOE_OK;
  if (!router || !x || !topk_ids || !topk_w || !workspace) return MOE_ERR_NULL;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256) || !aligned(x, 16) || !aligned(router, 16)) return MOE_ERR_ARG;
  hipStream_t st = (hipStream_t)hip_stream;
  Buffers b = carve(p, workspace, topk_ids, topk_w);
  const BucketOut bo{expert_counts, expert_offsets, token_slots, active_experts, n_active};
  (void)hipGetLastError();
  enqueue_route_plain(p, router, x, b, bo, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int32_t moe_layer_forward(const moe_layer_desc* desc, const moe_layer_weights* weights,
                          const float* x, int32_t n_tokens, float* y, int32_t* topk_ids,
                          float* topk_w, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
  return forward_impl(desc, weights, x, n_tokens, y, topk_ids, topk_w, workspace, workspace_bytes,
                      hip_stream, nullptr, 0);
}

int32_t moe_layer_forward_noalloc(const moe_layer_desc* desc, const moe_layer_weights* weights,
                                  const float* x, int32_t n_tokens, float* y, int32_t* topk_ids,
                                  float* topk_w, void* hip_stream) {
  if (!desc || !weights) return MOE_ERR_NULL;
  Plan p;
  const int rc = make_plan(desc, n_tokens, &p);
  if (rc != MOE_OK) return rc;
  if (p.total > (size_t)MOE_NOALLOC_MAX_WORKSPACE) return MOE_ERR_WORKSPACE;
  if (n_tokens == 0) return MOE_OK;
  void* ws = nullptr;
  const int rs = scratch_address((hipStream_t)hip_stream, &ws);
  if (rs != MOE_OK) return rs;
  return forward_impl(desc, weights, x, n_tokens, y, topk_ids, topk_w, ws,
                      (size_t)MOE_NOALLOC_MAX_WORKSPACE, hip_stream, nullptr, 0);
}

int32_t moe_layer_forward_timed(const moe_layer_desc* desc, const moe_layer_weights* weights,
                                const float* x, int32_t n_tokens, float* y, int32_t* topk_ids,
                                float* topk_w, void* workspace, size_t workspace_bytes,
                                void* hip_stream, void* const* events, int32_t n_events) {
  if (!events) return MOE_ERR_NULL;
  return forward_impl(desc, weights, x, n_tokens, y, topk_ids, topk_w, workspace, workspace_bytes,
                      hip_stream, events, n_events);
}

int32_t moe_dequant_rows(int32_t dtype, const void* tensor, int64_t rows, int32_t cols,
                         int64_t row_start, int64_t row_count, float* out, void* hip_stream) {
  if (!routed_type(dtype)) return MOE_ERR_DTYPE;
  if (rows < 0 || cols <= 0 || row_start < 0 || row_count < 0) return MOE_ERR_SHAPE;
  if (cols % blk_of(dtype)) return MOE_ERR_SHAPE;
  if (row_start + row_count > rows) return MOE_ERR_SHAPE;
  if (row_count == 0) return MOE_OK;
  if (!tensor || !out) return MOE_ERR_NULL;
  const int64_t total = row_count * (int64_t)cols;
  int64_t blocks = (total + kBlock - 1) / kBlock;
  if (blocks > 65535) blocks = 65535;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)blocks), dim3(kBlock), 0, (hipStream_t)hip_stream,
                     dtype, (const uint8_t*)tensor, rows, cols, row_start, row_count, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"
