// C-ABI entry points of the routed-MoE verify layer (declared in
// include/moe_layer.h): argument validation, workspace layout, kernel
// selection and the launch sequence on the caller's HIP stream.
#include <hip/hip_runtime.h>

#include <cstring>

#include "common.h"
#include "ffn.h"
#include "misc.h"
#include "route.h"

using namespace svr;

namespace {

constexpr int kVersion = 100;  // 0.1.0

enum Stage {
  kStRouter = 0,
  kStTopk,
  kStBucket,
  kStSharedGateUp,
  kStRoutedGateUp,
  kStSharedDown,
  kStRoutedDown,
  kStCombine,
  kNumStages
};
const char* const kStageNames[kNumStages] = {"router_logits", "topk",        "bucket",
                                             "shared_gateup", "routed_gateup", "shared_down",
                                             "routed_down",   "combine"};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int wpc_of(int dtype) { return dtype == MOE_Q8_0 ? 16 : 32; }
int blk_of(int dtype) { return dtype == MOE_Q8_0 ? 32 : 256; }
bool quant_type(int dtype) { return dtype == MOE_Q8_0 || dtype == MOE_Q4_K; }

// Lanes per row and 16-byte chunks per lane for a row of K columns.
struct FfnShape {
  int lpr, cpl;
};
bool ffn_shape(int dtype, int K, FfnShape* s) {
  if (K <= 0 || K % blk_of(dtype)) return false;
  const int chunks = K / wpc_of(dtype);
  for (int lpr = 64; lpr >= 1; lpr >>= 1) {
    if (chunks % lpr == 0 && chunks / lpr <= kMaxChunksPerLane) {
      s->lpr = lpr;
      s->cpl = chunks / lpr;
      return true;
    }
  }
  return false;
}

// Tokens per pass: as many as keep the per-lane activation slice within 64
// floats (at a verify batch an expert serves about one token, so VGPRs go
// to loads in flight rather than to idle token slots).
constexpr int tp_for(int fmt, int cpl) {
  return (cpl * (fmt == kQ8_0 ? 16 : 32) <= 16) ? 4 : (cpl * (fmt == kQ8_0 ? 16 : 32) <= 32) ? 2 : 1;
}

struct Plan {
  int H, E, k, F, Fs, et, st, M;
  size_t logits, ids, w, counts, offsets, slots, active, nactive, h, hs, o, s, total;
};

int check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->ffn <= 0 || d->shared_ffn < 0)
    return MOE_ERR_SHAPE;
  if (!quant_type(d->expert_type)) return MOE_ERR_DTYPE;
  if (d->shared_ffn > 0 && !quant_type(d->shared_type)) return MOE_ERR_DTYPE;
  if (d->n_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (d->top_k > d->n_experts || d->top_k > kMaxTopK) return MOE_ERR_SHAPE;
  FfnShape s;
  if (!ffn_shape(d->expert_type, d->hidden, &s) || !ffn_shape(d->expert_type, d->ffn, &s))
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
  p->st = d->shared_type;
  p->M = M;
  const size_t Mz = (size_t)M, P = Mz * p->k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  p->logits = take(Mz * p->E * 4);
  p->ids = take(P * 4);
  p->w = take(P * 4);
  p->counts = take((size_t)p->E * 4);
  p->offsets = take((size_t)(p->E + 1) * 4);
  p->slots = take(P * 4);
  p->active = take((size_t)p->E * 4);
  p->nactive = take(4);
  p->h = take(P * p->F * 4);
  p->hs = take(Mz * p->Fs * 4);
  p->o = take(P * p->H * 4);
  p->s = take(Mz * p->H * 4);
  p->total = off;
  return MOE_OK;
}

template <int FMT, int CPL, bool GU>
void launch_ffn_t(dim3 grid, hipStream_t st, const FfnArgs& a) {
  hipLaunchKernelGGL((k_ffn<FMT, CPL, tp_for(FMT, CPL), GU>), grid, dim3(kBlock), 0, st, a);
}

template <int FMT, bool GU>
bool launch_ffn_c(int cpl, dim3 grid, hipStream_t st, const FfnArgs& a) {
  switch (cpl) {
    case 1: launch_ffn_t<FMT, 1, GU>(grid, st, a); return true;
    case 2: launch_ffn_t<FMT, 2, GU>(grid, st, a); return true;
    case 3: launch_ffn_t<FMT, 3, GU>(grid, st, a); return true;
    case 4: launch_ffn_t<FMT, 4, GU>(grid, st, a); return true;
    case 5: launch_ffn_t<FMT, 5, GU>(grid, st, a); return true;
    case 6: launch_ffn_t<FMT, 6, GU>(grid, st, a); return true;
    case 7: launch_ffn_t<FMT, 7, GU>(grid, st, a); return true;
    case 8: launch_ffn_t<FMT, 8, GU>(grid, st, a); return true;
    default: return false;
  }
}

// Launches one FFN role over `slots_max` expert slots.
bool launch_ffn(int dtype, bool gateup, FfnArgs a, int slots_max, hipStream_t st) {
  FfnShape s;
  if (!ffn_shape(dtype, a.K, &s)) return false;
  a.lpr = s.lpr;
  const int G = kWave / s.lpr;
  const int unit_step = 4 * G;  // rows a workgroup covers per step
  const int64_t total_units = (int64_t)a.rows_per_expert * slots_max;
  const int64_t target_blocks = 1024;
  int64_t steps = (total_units + unit_step * target_blocks - 1) / (unit_step * target_blocks);
  steps = steps < 4 ? 4 : (steps > 16 ? 16 : steps);
  a.units_per_block = (int)(unit_step * steps);
  dim3 grid((a.rows_per_expert + a.units_per_block - 1) / a.units_per_block, slots_max);
  if (dtype == MOE_Q8_0)
    return gateup ? launch_ffn_c<kQ8_0, true>(s.cpl, grid, st, a)
                  : launch_ffn_c<kQ8_0, false>(s.cpl, grid, st, a);
  return gateup ? launch_ffn_c<kQ4_K, true>(s.cpl, grid, st, a)
                : launch_ffn_c<kQ4_K, false>(s.cpl, grid, st, a);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Records stage event i if the caller asked for events; a failure shows up
// in the final hipGetLastError check.
inline void mark(hipEvent_t* ev, int i, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev[i], st);
}

struct Routing {
  int32_t *ids, *counts, *offsets, *slots, *active, *nactive;
  float *w, *logits;
};

void enqueue_route(const Plan& p, const float* router, const float* x, const Routing& r,
                   hipStream_t st, hipEvent_t* ev) {
  const int wpb = kBlock / kWave;
  mark(ev, kStRouter, st);
  hipLaunchKernelGGL(k_router_logits, dim3((p.E + wpb - 1) / wpb), dim3(kBlock), 0, st, router, x,
                     r.logits, p.H, p.E, p.M);
  mark(ev, kStTopk, st);
  hipLaunchKernelGGL(k_topk, dim3((p.M + wpb - 1) / wpb), dim3(kBlock), 0, st, r.logits, r.ids,
                     r.w, p.E, p.k, p.M);
  mark(ev, kStBucket, st);
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(kBlock), 0, st, r.ids, p.M * p.k, p.E, r.counts,
                     r.offsets, r.slots, r.active, r.nactive);
}

int forward_impl(const moe_layer_desc* desc, const moe_layer_weights* wt, const float* x,
                 int32_t n_tokens, float* y, int32_t* topk_ids, float* topk_w, void* workspace,
                 size_t workspace_bytes, void* hip_stream, void* const* events, int32_t n_events) {
  if (!desc || !wt) return MOE_ERR_NULL;
  Plan p;
  int rc = make_plan(desc, n_tokens, &p);
  if (rc != MOE_OK) return rc;
  if (events && n_events != kNumStages + 1) return MOE_ERR_ARG;
  hipStream_t st = (hipStream_t)hip_stream;
  hipEvent_t* ev = events ? (hipEvent_t*)events : nullptr;
  if (n_tokens == 0) {
    if (ev)
      for (int i = 0; i <= kNumStages; ++i) mark(ev, i, st);
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

  uint8_t* ws = (uint8_t*)workspace;
  Routing r;
  r.logits = (float*)(ws + p.logits);
  r.ids = topk_ids ? topk_ids : (int32_t*)(ws + p.ids);
  r.w = topk_w ? topk_w : (float*)(ws + p.w);
  r.counts = (int32_t*)(ws + p.counts);
  r.offsets = (int32_t*)(ws + p.offsets);
  r.slots = (int32_t*)(ws + p.slots);
  r.active = (int32_t*)(ws + p.active);
  r.nactive = (int32_t*)(ws + p.nactive);
  float* h = (float*)(ws + p.h);
  float* hs = (float*)(ws + p.hs);
  float* o = (float*)(ws + p.o);
  float* s = (float*)(ws + p.s);

  (void)hipGetLastError();  // clear a stale error from earlier, unrelated calls
  enqueue_route(p, wt->router, x, r, st, ev);

  const int slots_max = (p.M * p.k < p.E) ? p.M * p.k : p.E;

  // Shared expert gate/up + SwiGLU (identity token list).
  mark(ev, kStSharedGateUp, st);
  if (p.Fs > 0) {
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
    a.out = hs;
    if (!launch_ffn(p.st, true, a, 1, st)) return MOE_ERR_SHAPE;
  }
  // Routed gate/up + SwiGLU: h[pair][F].
  mark(ev, kStRoutedGateUp, st);
  {
    FfnArgs a{};
    a.w0 = (const uint8_t*)wt->gate;
    a.w1 = (const uint8_t*)wt->up;
    a.total_rows = (int64_t)p.E * p.F;
    a.rows_per_expert = p.F;
    a.K = p.H;
    a.active = r.active;
    a.n_active = r.nactive;
    a.offsets = r.offsets;
    a.slots = r.slots;
    a.top_k = p.k;
    a.act = x;
    a.act_by_pair = 0;
    a.out = h;
    if (!launch_ffn(p.et, true, a, slots_max, st)) return MOE_ERR_SHAPE;
  }
  // Shared down: s[t][H].
  mark(ev, kStSharedDown, st);
  if (p.Fs > 0) {
    FfnArgs a{};
    a.w0 = (const uint8_t*)wt->shared_down;
    a.total_rows = p.H;
    a.rows_per_expert = p.H;
    a.K = p.Fs;
    a.n_tokens = p.M;
    a.top_k = 1;
    a.act = hs;
    a.act_by_pair = 1;
    a.out = s;
    if (!launch_ffn(p.st, false, a, 1, st)) return MOE_ERR_SHAPE;
  }
  // Routed down: o[pair][H].
  mark(ev, kStRoutedDown, st);
  {
    FfnArgs a{};
    a.w0 = (const uint8_t*)wt->down;
    a.total_rows = (int64_t)p.E * p.H;
    a.rows_per_expert = p.H;
    a.K = p.F;
    a.active = r.active;
    a.n_active = r.nactive;
    a.offsets = r.offsets;
    a.slots = r.slots;
    a.top_k = p.k;
    a.act = h;
    a.act_by_pair = 1;
    a.out = o;
    if (!launch_ffn(p.et, false, a, slots_max, st)) return MOE_ERR_SHAPE;
  }
  // Combine.
  mark(ev, kStCombine, st);
  {
    const int64_t n4 = (int64_t)p.M * (p.H / 4);
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((n4 + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                       o, p.Fs > 0 ? s : nullptr, r.w, y, p.M, p.H, p.k);
  }
  mark(ev, kNumStages, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
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

int32_t moe_stage_count(void) { return kNumStages; }

const char* moe_stage_name(int32_t i) {
  return (i >= 0 && i < kNumStages) ? kStageNames[i] : nullptr;
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
  uint8_t* ws = (uint8_t*)workspace;
  Routing r;
  r.logits = (float*)(ws + p.logits);
  r.ids = topk_ids;
  r.w = topk_w;
  r.counts = expert_counts;
  r.offsets = expert_offsets;
  r.slots = token_slots;
  r.active = active_experts;
  r.nactive = n_active;
  (void)hipGetLastError();
  enqueue_route(p, router, x, r, st, nullptr);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int32_t moe_layer_forward(const moe_layer_desc* desc, const moe_layer_weights* weights,
                          const float* x, int32_t n_tokens, float* y, int32_t* topk_ids,
                          float* topk_w, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
  return forward_impl(desc, weights, x, n_tokens, y, topk_ids, topk_w, workspace, workspace_bytes,
                      hip_stream, nullptr, 0);
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
  if (!quant_type(dtype)) return MOE_ERR_DTYPE;
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
