// Fused launches of the small-batch (decode / verify) path.
//
//   phase 1: router rows + shared-expert gate/up tiles; the last workgroup
//            of the grid waits for the router rows' keys, runs top-k for
//            every token and the bucketing, so routing costs no launch of
//            its own.
//   phase 2: routed gate/up tiles + shared-expert down tiles (up to four
//            tokens: per-pair tiles, the pairs of an expert that several
//            tokens select sharing its rows).
//   phase 3: routed down + combine: up to four tokens, one workgroup per
//            (token, row tile) that adds its slots in LDS (k_down_tok);
//            above, the last workgroup to finish a row tile (over all
//            active experts) combines that tile of the output
//            (k_down_combine).
//
// The routing keys and the hand-off counters live at the start of the
// workspace.  Each is returned to zero by the workgroup that consumes it,
// so a workspace that starts zero-filled stays valid from call to call.
#pragma once

#include "ffn.h"
#include "route.h"

namespace svr {

constexpr int kMaxTiles = 1008;  // combine counters available in the workspace

struct alignas(256) CounterLine {
  unsigned v;
  unsigned pad[63];
};

struct Counters {
  // Nonzero once the routing's wait for the router keys has given up;
  // written, never read, by the kernels: a diagnostic word for the caller.
  unsigned route_wait_err;
  unsigned pad[63];
  unsigned tile_done[kMaxTiles];
};
static_assert(sizeof(Counters) <= kCounterBytes, "counter page");

struct RouteArgs {
  const float* router;
  const float* x;
  uint32_t* keys;  // [M][E] routing keys, zero between calls
  uint2* pair_info;  // non-NULL (pair slots): each pair's {expert, token word}
  int32_t* ids;
  float* w;
  BucketOut b;
  int H, E, k, M;
  int n_router_blocks;
  Counters* ctr;
  int bucket;  // 1: also build the per-expert lists (not needed with pair slots)
};

// Router workgroups: one expert row each, its M logits published as keys.
template <int NC>
__device__ __forceinline__ void router_part(const RouteArgs& r, int blk) {
  router_row_keys<NC>(r.router, r.x, r.keys, r.H, r.E, r.M, blk);
}

// The routing workgroup (dispatched after every router workgroup it waits
// for): wave w takes tokens w, w + 4, ..., polls each token's keys,
// selects its experts and clears the keys; then, if asked, each pair's
// expert and token word (pair slots) or the per-expert lists.
__device__ __forceinline__ void route_part(const RouteArgs& r) {
  __shared__ int32_t s_ids[kPairTokens * kMaxTopK];
  __shared__ uint32_t s_table[kMaxExperts];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  for (int t = wv; t < r.M; t += kWavesPerBlock) {
    const TopkLane tl =
        topk_keys_poll(r.keys + (int64_t)t * r.E, r.ids + (int64_t)t * r.k,
                       r.w + (int64_t)t * r.k, r.E, r.k, &r.ctr->route_wait_err);
    if (r.pair_info && lane < r.k) s_ids[t * r.k + lane] = tl.e;
  }
  if (r.pair_info) {  // M <= kPairTokens
    __syncthreads();
    if (wv == 0) pair_infos_wave(s_ids, r.M, r.k, s_table, r.pair_info);
  }
  if (r.bucket) {
    __syncthreads();
    bucket_block(r.ids, r.M * r.k, r.E, r.b);
  }
}

// Phase 1.  SFMT == 0: no shared expert; SS: shared gate/up shape code.
// Grid: router workgroups, shared gate/up tiles, then the routing workgroup.
template <int NC, int SFMT, int SS>
__global__ __launch_bounds__(kBlock) void k_phase1(RouteArgs r, FfnArgs s) {
  if (blockIdx.x == gridDim.x - 1) {
    route_part(r);
  } else if ((int)blockIdx.x < r.n_router_blocks) {
    router_part<NC>(r, blockIdx.x);
  } else if constexpr (SFMT != 0) {
    ffn_tile<SFMT, shape_cpl(SS), true, shape_lpr(SS)>(s, 0, blockIdx.x - r.n_router_blocks);
  }
}

// Two FFN roles in one grid: blocks [0, na) take tiles of role A (grid of
// a_tiles x slots, tile fastest), the rest tiles of role B (one slot).
// SA, SB: shape codes.  A gate/up role A with pair slots serves each
// expert's tokens in one pass (token words).
template <int FA, int SA, bool GA, int FB, int SB, bool GB>
__global__ __launch_bounds__(kBlock) void k_dual(FfnArgs a, int a_tiles, int na, FfnArgs b) {
  const int blk = blockIdx.x;
  if (blk < na) {
    ffn_tile<FA, shape_cpl(SA), GA, shape_lpr(SA), GA>(a, blk / a_tiles, blk % a_tiles);
  } else {
    ffn_tile<FB, shape_cpl(SB), GB, shape_lpr(SB)>(b, 0, blk - na);
  }
}

// Combine of rows [r0, r1) of y: y[t][r] = s[t][r] + sum_j w[t][j] o[t*k+j][r],
// with s, w and the expert outputs o written by other workgroups of the
// same launch (all read past the per-XCD L2).  Each thread takes four
// consecutive rows of one token and requests the k slots' float4s eight at
// a time before adding them in slot order.
__device__ __forceinline__ void combine_rows(const float* __restrict__ o,
                                             const float* __restrict__ s,
                                             const float* __restrict__ w, float* __restrict__ y,
                                             int M, int H, int k, int r0, int r1) {
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(o, (uint32_t)((int64_t)M * k * H * 4));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, s ? (uint32_t)((int64_t)M * H * 4) : 0u);
  const int n4 = (r1 - r0) >> 2;
  for (int i = threadIdx.x; i < M * n4; i += kBlock) {
    const int t = i / n4;
    const int r = r0 + 4 * (i - t * n4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (s) acc = bload16_shared(rs, (uint32_t)(((int64_t)t * H + r) * 4));
    for (int j0 = 0; j0 < k; j0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        v[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j0 + jj < k)
          v[jj] = bload16_shared(ro, (uint32_t)((((int64_t)t * k + j0 + jj) * H + r) * 4));
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj < k) {
          const float wj = load_shared(w + t * k + j0 + jj);
          acc.x = fmaf(wj, v[jj].x, acc.x);
          acc.y = fmaf(wj, v[jj].y, acc.y);
          acc.z = fmaf(wj, v[jj].z, acc.z);
          acc.w = fmaf(wj, v[jj].w, acc.w);
        }
      }
    }
    *reinterpret_cast<float4*>(y + (int64_t)t * H + r) = make_float4(acc.x, acc.y, acc.z, acc.w);
  }
}

struct CombineArgs {
  const float* o;
  const float* s;
  const float* w;
  float* y;
  int M, H, k;
  Counters* ctr;
};

// Phase 3: routed down tiles, then the combine of each finished row tile.
// Ring depth of the routed down rows: a one-matrix row of a few hundred
// bytes per lane group needs several steps in flight to cover the latency.
#ifndef SVR_DOWN_NST
#define SVR_DOWN_NST 4
#endif
constexpr int kDownNst = SVR_DOWN_NST;

// Phase 3 for pair slots (up to four tokens): one workgroup of eight waves
// per (token, row tile).  In each pass of eight slots, wave w streams the
// tile's rows of the expert of pair (t, j0 + w) against that pair's h and
// leaves them in LDS; after a barrier each thread owns one row and adds
// the pass's slots in order onto y[t][r] = s[t][r] + sum_j w[t][j] o_j[r].
// The combine needs no counters and no reads past L2: routing, h and s all
// come from earlier launches.
constexpr int kDownTokWaves = 8;
constexpr int kDownTokThreads = kDownTokWaves * kWave;
constexpr int kDownTokRows = kDownTokThreads;  // rows of a tile, one per thread

template <int FMT, int S>
__global__ __launch_bounds__(kDownTokThreads) void k_down_tok(FfnArgs a, CombineArgs c,
                                                              int tiles) {
  constexpr int CPL = shape_cpl(S), LPR = shape_lpr(S);
  __shared__ float s_o[kDownTokWaves * kDownTokRows];
  const int t = blockIdx.x / tiles, tile = blockIdx.x - t * tiles;
  // The wave index, and with it the pair and its expert, is uniform over
  // the wave; saying so keeps the expert's buffer resources in scalar
  // registers (a per-lane resource turns every load into a readfirstlane
  // loop).
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ub = tile * a.units_per_block;
  const int ue = min(ub + a.units_per_block, a.rows_per_expert);
  const int r = ub + (int)threadIdx.x;  // the row this thread combines
  const bool own = r < ue;
  float acc = 0.f;
  if (own && c.s) acc = c.s[(int64_t)t * c.H + r];
  const int G = kWave / (LPR ? LPR : a.lpr);
  for (int j0 = 0; j0 < c.k; j0 += kDownTokWaves) {
    const int j = j0 + wv;
    if (j < c.k) {  // wave-uniform
      const int p = t * c.k + j;
      const int ids1[1] = {p}, slot1[1] = {wv};
      const int e = __builtin_amdgcn_readfirstlane(a.pair_expert[p]);
      ffn_pass<FMT, CPL, 1, false, kDownNst, true, LPR>(
          a, e, ids1, ub, G, ue, LdsOut{s_o, ub, kDownTokRows}, slot1);
    }
    __syncthreads();
    if (own) {
      const int nj = min(kDownTokWaves, c.k - j0);
      for (int w = 0; w < nj; ++w)
        acc = fmaf(c.w[(int64_t)t * c.k + j0 + w], s_o[w * kDownTokRows + (r - ub)], acc);
    }
    __syncthreads();  // s_o is refilled by the next pass
  }
  if (own) c.y[(int64_t)t * c.H + r] = acc;
}

template <int FMT, int S>
__global__ __launch_bounds__(kBlock) void k_down_combine(FfnArgs a, CombineArgs c) {
  constexpr int CPL = shape_cpl(S), LPR = shape_lpr(S);
  __shared__ int s_last;
  const int tile = blockIdx.x, slot = blockIdx.y;
  const int n_act = a.pair_expert ? a.n_pairs : *a.n_active;
  if (slot >= n_act) return;  // block-uniform; these blocks never count
  ffn_tile<FMT, CPL, false, LPR>(a, slot, tile);  // o rows stored with store_shared
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive(&c.ctr->tile_done[tile]) == (unsigned)(n_act - 1);
  __syncthreads();
  if (!s_last) return;
  const int r0 = tile * a.units_per_block;
  const int r1 = min(r0 + a.units_per_block, c.H);
  combine_rows(c.o, c.s, c.w, c.y, c.M, c.H, c.k, r0, r1);
  if (threadIdx.x == 0)
    __hip_atomic_store(&c.ctr->tile_done[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace svr
