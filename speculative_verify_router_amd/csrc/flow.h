// The whole small-batch layer as one launch: a work queue of items in
// dependency order, with hand-off counters instead of kernel boundaries.
//
// Items, in queue order:
//   R   router row e (E items); the workgroup that finishes the last one
//       runs top-k for every token and publishes ids and weights
//   SG  shared gate/up + SwiGLU, one row tile each
//   G   routed gate/up + SwiGLU of (token, slot) pair p, one row tile each,
//       pair-major; waits for the routing
//   SD  shared down, one output row tile each; waits for every SG item
//   D   routed down of pair p, one output row tile each, pair-major; waits
//       for every G item of pair p.  The last of the SD and D items of an
//       output row tile combines that tile of y.
//
// Each workgroup takes one item from an atomic counter when it starts, so
// every item that has been handed out is held by a running workgroup, and
// an item waits only for items earlier in the queue.  So the earliest
// unfinished item never waits on anything unfinished, and the queue drains
// whatever the number of resident workgroups.  Every wait is also bounded: past the limit the workgroup
// flags an error in the counter page, skips the item's arithmetic but still
// signals its completion, so every workgroup exits.
//
// The last workgroup to exit returns the counters it does not clear itself
// to zero; each combine counter is cleared by the workgroup that combines.
#pragma once

#include "ffn.h"
#include "phases.h"
#include "route.h"

namespace svr {

constexpr int kFlowMaxPairs = 256;  // M * k pairs (M <= 4, k <= 64)
constexpr int kFlowMaxTiles = 1024;  // output row tiles
constexpr int kFlowLdsOut = 2048;    // floats of item output staged in LDS
constexpr unsigned kSpinLimit = 1u << 21;  // polls of at least 0.3 us each

// Counters that many workgroups poll or bump each sit on their own
// 256-byte line, so that polls of one do not queue behind atomics on
// another; the per-pair gate/up counters sit 32 bytes apart.
struct alignas(256) FlowLine {
  unsigned v;
  unsigned pad[63];
};
struct FlowCounters {
  FlowLine queue;        // next item
  FlowLine exits;        // workgroups done
  FlowLine router_done;  // router rows finished
  FlowLine ready;        // 1 once ids and weights are published
  FlowLine sg_done;      // shared gate/up tiles finished
  FlowLine err;          // nonzero once a wait gave up (stays set)
  struct {
    unsigned v;
    unsigned pad[7];
  } gu_done[kFlowMaxPairs];             // routed gate/up tiles finished, per pair
  unsigned tile_done[kFlowMaxTiles];  // down items finished, per output row tile
};
static_assert(sizeof(FlowCounters) <= kCounterBytes, "counter area");

struct FlowArgs {
  RouteArgs r;
  FfnArgs sg, g, sd, d;
  CombineArgs c;
  FlowCounters* ctr;
  int n_r, n_sg, n_g, n_sd, n_d;  // items per kind
  int g_tiles, d_tiles;           // row tiles per pair
  int n_pairs;
  int sd_per_tile;                // shared down items per output row tile
};

// Values every wave of the workgroup holds alike (read from LDS after a
// barrier) are moved to a scalar register, so branches on them are uniform.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Polls (one thread) until *p >= target, about every 0.3 us; gives up,
// raising the error flag, once the flag is up (checked every 32 polls) or
// after kSpinLimit polls.
__device__ __forceinline__ int flow_poll(const unsigned* p, unsigned target, unsigned* err) {
  for (unsigned n = 0; n < kSpinLimit; ++n) {
    if (load_shared(p) >= target) return 1;
    if ((n & 31) == 31 && load_shared(err)) return 0;
    __builtin_amdgcn_s_sleep(12);
  }
  store_shared(err, 1u);
  return 0;
}

// Instantiated k_flow variants: (router NC, shared format, shared gate/up
// and down shape codes, routed format, routed gate/up and down shape
// codes).  H = 4096 with F = Fs = 1280 or 1536, Q4_K or Q8_0 routed,
// Q8_0 shared; and H <= 1024 with small Q8_0 experts and no shared expert.
#define SVR_FLOW_VARIANTS(X)                                                               \
  X(4, kQ8_0, shape_code(4, 64), shape_code(5, 16), kQ4_K, shape_code(2, 64), shape_code(3, 16)) \
  X(4, kQ8_0, shape_code(4, 64), shape_code(3, 32), kQ4_K, shape_code(2, 64), shape_code(3, 16)) \
  X(4, kQ8_0, shape_code(4, 64), shape_code(5, 16), kQ8_0, shape_code(4, 64), shape_code(5, 16)) \
  X(1, 0, shape_code(1, 0), shape_code(1, 0), kQ8_0, shape_code(1, 16), shape_code(1, 8))

enum FlowKind { kItemRouter = 0, kItemSharedGateUp, kItemGateUp, kItemSharedDown, kItemDown };

// Shared expert, rows of item `tile` for every token, outputs to LDS
// (token t in slot t).  The waves are split into M token groups of
// 4 / M waves (M <= 4) that divide the rows among them; with M = 3 one wave
// idles.  No wave-dependent loop: each wave runs at most one pass.
template <int FMT, int S, bool GATEUP>
__device__ __forceinline__ void flow_shared_tile(const FfnArgs& a, int tile, float* lds) {
  constexpr int CPL = shape_cpl(S), LPR = shape_lpr(S);
  const int ub = tile * a.units_per_block;
  const int ue = min(ub + a.units_per_block, a.rows_per_expert);
  const int G = kWave / (LPR ? LPR : a.lpr);
  const int wv = threadIdx.x >> 6;
  const int rg = kWavesPerBlock / a.n_tokens;  // waves per token
  const int t = wv / rg, q = wv - t * rg;
  const int ids1[1] = {t};
  if (t < a.n_tokens && ub + q * G < ue)
    ffn_pass<FMT, CPL, 1, GATEUP, 0, true, LPR>(a, 0, ids1, ub + q * G, rg * G, ue,
                                           LdsOut{lds, ub, a.units_per_block}, ids1);
}

// Item outputs staged in LDS -> rows [ub, ue) of `ntok` output rows of
// width `width` starting at `out` (written through for other workgroups).
__device__ __forceinline__ void flow_copy_out(const float* lds, int ld, float* out, int width,
                                              int ntok, int ub, int ue) {
  const int cnt = ue - ub;
  for (int i = threadIdx.x; i < ntok * cnt; i += kBlock) {
    const int t = i / cnt, rr = i - t * cnt;
    store_shared(out + (int64_t)t * width + ub + rr, lds[t * ld + rr]);
  }
}

// NC: router float4 chunks per lane; SF: shared format (0: no shared
// expert) with gate/up and down shape codes SGC, SDC; RF: routed format
// with gate/up and down shape codes GC, DC.
//
// One workgroup per item.  It takes its item from the queue counter when it
// starts, so items are handed out in queue order to workgroups that are
// running; a workgroup waits only for items earlier in the queue.  All six
// barriers sit at the top level of the kernel and every wave passes each of
// them once: item-specific code lies between them, contains no barrier, and
// every loop in it that precedes a barrier runs the same number of times in
// every wave.
template <int NC, int SF, int SGC, int SDC, int RF, int GC, int DC>
__global__ __launch_bounds__(kBlock) void k_flow(FlowArgs f) {
  __shared__ unsigned s_item, s_ok, s_prev;
  __shared__ RouterPart s_part;
  __shared__ float s_out[kFlowLdsOut];
  FlowCounters* ctr = f.ctr;
  const unsigned need_tile = (unsigned)(f.n_pairs + (f.n_sd ? f.sd_per_tile : 0));

  // B1: the item.
  if (threadIdx.x == 0) s_item = arrive(&ctr->queue.v);
  __syncthreads();
  const int it = uniform((int)s_item);
  int kind = kItemDown, idx = it - (f.n_r + f.n_sg + f.n_g + f.n_sd);
  if (it < f.n_r) {
    kind = kItemRouter, idx = it;
  } else if (it < f.n_r + f.n_sg) {
    kind = kItemSharedGateUp, idx = it - f.n_r;
  } else if (it < f.n_r + f.n_sg + f.n_g) {
    kind = kItemGateUp, idx = it - f.n_r - f.n_sg;
  } else if (it < f.n_r + f.n_sg + f.n_g + f.n_sd) {
    kind = kItemSharedDown, idx = it - f.n_r - f.n_sg - f.n_g;
  }
  const int pair = kind == kItemGateUp ? idx / f.g_tiles : kind == kItemDown ? idx / f.d_tiles : 0;
  const int tile = kind == kItemGateUp ? idx - pair * f.g_tiles
                   : kind == kItemDown ? idx - pair * f.d_tiles
                                       : idx;
  // Output row tile (combine counter) of a shared or routed down item.
  const int otile = kind == kItemSharedDown ? idx / f.sd_per_tile : tile;

  // B2: the item's inputs are ready (one thread polls).
  if (threadIdx.x == 0) {
    int ok = 1;
    if (kind == kItemGateUp)
      ok = flow_poll(&ctr->ready.v, 1u, &ctr->err.v);
    else if (kind == kItemSharedDown)
      ok = flow_poll(&ctr->sg_done.v, (unsigned)f.n_sg, &ctr->err.v);
    else if (kind == kItemDown)
      ok = flow_poll(&ctr->gu_done[pair].v, (unsigned)f.g_tiles, &ctr->err.v);
    s_ok = ok;
  }
  __syncthreads();
  const bool ok = uniform((int)s_ok) != 0;

  // The item's streaming work.
  if (kind == kItemRouter) {
    router_row_partials<NC>(f.r.router, f.r.x, f.r.H, f.r.M, idx, s_part);
  } else if (ok) {
    if constexpr (SF != 0) {
      if (kind == kItemSharedGateUp) flow_shared_tile<SF, SGC, true>(f.sg, tile, s_out);
      if (kind == kItemSharedDown) flow_shared_tile<SF, SDC, false>(f.sd, tile, s_out);
    }
    if (kind == kItemGateUp)
      ffn_tile_pair<RF, shape_cpl(GC), true, 0, true, shape_lpr(GC)>(f.g, pair, tile, s_out);
    if (kind == kItemDown)
      ffn_tile_pair<RF, shape_cpl(DC), false, kDownNst, true, shape_lpr(DC)>(f.d, pair, tile,
                                                                             s_out);
  }
  // B3: the router's partial sums and the item's LDS outputs are complete.
  __syncthreads();
  if (kind == kItemRouter) {
    router_row_finish(f.r.logits, f.r.E, f.r.M, idx, s_part);
  } else if (ok) {
    const FfnArgs& a = kind == kItemSharedGateUp ? f.sg
                       : kind == kItemGateUp     ? f.g
                       : kind == kItemSharedDown ? f.sd
                                                 : f.d;
    const int ub = tile * a.units_per_block;
    const int ue = min(ub + a.units_per_block, a.rows_per_expert);
    const bool shared = kind == kItemSharedGateUp || kind == kItemSharedDown;
    if (ub < ue)
      flow_copy_out(s_out, a.units_per_block, a.out + (shared ? 0 : (int64_t)pair * a.rows_per_expert),
                    a.rows_per_expert, shared ? a.n_tokens : 1, ub, ue);
  }

  // B4: every wave's hand-off stores are complete; count the item.
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* c = kind == kItemRouter          ? &ctr->router_done.v
                  : kind == kItemSharedGateUp ? &ctr->sg_done.v
                  : kind == kItemGateUp       ? &ctr->gu_done[pair].v
                                              : &ctr->tile_done[otile];
    s_prev = arrive(c);
  }
  // B5: the count is known to every wave.
  __syncthreads();
  const unsigned prev = (unsigned)uniform((int)s_prev);

  // The last router row runs the top-k (tokens in rounds of four, wave w
  // taking token round + w); the last down item of an output row tile
  // combines it.
  const bool last_router = kind == kItemRouter && prev == (unsigned)(f.r.E - 1);
  const bool last_tile =
      (kind == kItemSharedDown || kind == kItemDown) && prev == need_tile - 1;
  if (last_router) {
    const int wv = threadIdx.x >> 6;
    for (int t0 = 0; t0 < f.r.M; t0 += kWavesPerBlock) {
      const int t = t0 + wv;
      if (t < f.r.M)
        topk_token<true>(f.r.logits + (int64_t)t * f.r.E, f.r.ids + (int64_t)t * f.r.k,
                         f.r.w + (int64_t)t * f.r.k, f.r.E, f.r.k);
    }
  }
  if (last_tile) {
    const int r0 = otile * f.d.units_per_block;
    const int r1 = min(r0 + f.d.units_per_block, f.c.H);
    combine_rows(f.c.o, f.c.s, f.c.w, f.c.y, f.c.M, f.c.H, f.c.k, r0, r1);
  }
  // B6: every wave's top-k stores are complete before the routing is
  // published.
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (last_router) store_shared(&ctr->ready.v, 1u);
    if (last_tile) store_shared(&ctr->tile_done[otile], 0u);
  }

  // The last workgroup to finish resets the shared counters.
  if (threadIdx.x == 0 && arrive(&ctr->exits.v) == gridDim.x - 1) {
    store_shared(&ctr->router_done.v, 0u);
    store_shared(&ctr->ready.v, 0u);
    store_shared(&ctr->sg_done.v, 0u);
    for (int p = 0; p < f.n_pairs; ++p) store_shared(&ctr->gu_done[p].v, 0u);
    store_shared(&ctr->exits.v, 0u);
    store_shared(&ctr->queue.v, 0u);
  }
}

}  // namespace svr
