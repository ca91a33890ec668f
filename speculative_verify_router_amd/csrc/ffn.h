// Fused dequantise-and-multiply skinny GEMM for the expert FFNs.
//
// Routed gate/up/down are Q4_K, Q2_K, Q3_K, Q6_K or Q8_0 and the shared expert Q8_0
// ("Step 3.7 Flash Mixed-Quant GGUF", Tensor recipe; "Step-5 Preview GGUF",
// Precision distribution table and Tensor-type table).  At a verify batch of four tokens with 8
// of 288-352 experts each, an expert serves about one token, so this is an
// HBM-bound matrix-vector product: each selected expert's quant blocks are
// streamed once for all of that expert's tokens.
//
// Mapping.  A 16-byte chunk of the quant plane is the unit of loading:
// 16 weights for Q8_0, one 32-weight sub-block for Q4_K, four 16-weight
// sub-blocks for Q2_K and Q3_K, two for Q6_K (low bits; Q3_K's and Q6_K's
// high bits come from a plane of their own).  A row of K
// columns has K / kWpc chunks, covered by a group of `lpr` consecutive
// lanes (lpr | 64), lane j of the group taking chunks j, j+lpr, ...,
// j+(CPL-1)*lpr.  A wave works on 64/lpr rows at once and every wave load
// instruction reads whole 128-byte lines.  Each lane keeps its K-slice of
// the activations in VGPRs for the whole pass, so activations are read once
// per wave, not once per row.  Row loads go through a ring of NST register
// stages: while one step's chunks are multiplied, the next NST-1 steps'
// chunks are in flight.  Loads use per-expert buffer resources, so rows
// past the expert's end read as zero and need no clamping.
//
// Work split.  Routed experts: the four waves of a workgroup take
// different rows (tokens in passes of TP).  The shared expert serves every
// token, so there the waves take different tokens over the same rows and
// the rows are fetched from HBM once.
#pragma once

#include "quant.h"

namespace svr {

struct FfnArgs {
  const uint8_t* w0;        // gate (gate/up role) or down: planar tensor base
  const uint8_t* w1;        // up (gate/up role only)
  int64_t total_rows;       // rows of the stacked tensor
  int rows_per_expert;      // output rows per expert
  int K;                    // columns (input width)
  const int32_t* active;    // slot -> expert id; NULL: one expert, id 0
  const int32_t* n_active;  // number of valid slots; NULL: 1
  const int32_t* offsets;   // [E+1] list offsets; NULL: identity list of n_tokens
  const int32_t* slots;     // pair indices grouped by expert
  int n_tokens;             // identity-list length
  int top_k;                // pair p belongs to token p / top_k (1 for identity lists)
  const float* act;         // activation rows of width K
  int act_by_pair;          // activation row = pair (1) or token (0)
  float* out;               // output rows of width rows_per_expert
  int lpr;                  // lanes per row (power of two dividing 64)
  int units_per_block;      // output rows per workgroup
  int split_tokens;         // 1: waves take tokens, 0: waves take rows
  int coherent_out;         // 1: outputs are read by other workgroups of this launch
  const int32_t* pair_expert;  // pair slots: slot p is pair p, expert pair_expert[p]
  int n_pairs;                 // number of pair slots (pair_expert != NULL)
  // Pair slots, gate/up: NULL, or each pair's {expert, token word}
  // (pair_infos_wave): the pairs of an expert share its rows and each
  // serves all of the expert's tokens.
  const uint2* pair_info;
  int max_rows;     // host side: cap on units_per_block (0: none)
};

// A role's lane shape as one template argument: chunks per lane | lanes
// per row << 8 (lanes per row 0: read from FfnArgs::lpr at run time).
constexpr int shape_code(int cpl, int lpr) { return cpl | (lpr << 8); }
constexpr int shape_cpl(int code) { return code & 255; }
constexpr int shape_lpr(int code) { return code >> 8; }

// Tokens per pass: keep the per-lane activation slice within 64 floats.
constexpr int wpc_for(int fmt) {
  return fmt == kQ8_0 ? 16 : (fmt == kQ4_K || fmt == kQ6_K) ? 32 : 64;
}
constexpr int tp_for(int fmt, int cpl) {
  return (cpl * wpc_for(fmt) <= 16) ? 4 : (cpl * wpc_for(fmt) <= 32) ? 2 : 1;
}

// Ring depth: as many stages (2 to 5) as fit in about kRingVgprs VGPRs of
// in-flight chunks.
#ifndef SVR_RING_VGPRS
#define SVR_RING_VGPRS 100
#endif
constexpr int kRingVgprs = SVR_RING_VGPRS;
constexpr int chunk_vgprs(int fmt) {
  return fmt == kQ8_0 ? 5 : fmt == kQ4_K ? 8 : fmt == kQ2_K ? 6 : 8;  // Q3_K, Q6_K: 8
}
constexpr int nst_for(int fmt, int cpl, bool gateup) {
  return (cpl * (gateup ? 2 : 1) * chunk_vgprs(fmt) * 5 <= kRingVgprs)   ? 5
         : (cpl * (gateup ? 2 : 1) * chunk_vgprs(fmt) * 4 <= kRingVgprs) ? 4
         : (cpl * (gateup ? 2 : 1) * chunk_vgprs(fmt) * 3 <= kRingVgprs) ? 3
                                                                          : 2;
}

template <int FMT, int CPL, bool GATEUP>
struct Stage {
  Chunk<FMT> c0[CPL];
  Chunk<FMT> c1[GATEUP ? CPL : 1];
};

// cc[ci]: the chunk lane loads for its ci-th position.  Where the lane
// groups cover more positions than the row has chunks, the spare positions
// load the row's last chunk (a line the group reads anyway) against a zero
// activation slice, so they add nothing.
template <int FMT, int CPL, bool GATEUP>
__device__ __forceinline__ void load_stage(Stage<FMT, CPL, GATEUP>& s, const QPlanes& p0,
                                           const QPlanes& p1, uint32_t qo, uint32_t so,
                                           const int (&cc)[CPL]) {
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) {
    load_chunk(s.c0[ci], p0, qo, so, cc[ci]);
    if (GATEUP) load_chunk(s.c1[ci], p1, qo, so, cc[ci]);
  }
}

// Outputs kept in LDS instead of being stored row by row: row u of token
// slot t goes to p[t * ld + u - row0].  Stores inside the row loop would
// count against the same wait counter as the ring's loads.
struct LdsOut {
  float* p;
  int row0, ld;
};

template <int FMT, int CPL, int NT, bool GATEUP, bool LDSOUT, int LPR>
__device__ __forceinline__ void compute_stage(const Stage<FMT, CPL, GATEUP>& s,
                                              const XSlice<FMT> (&xs)[NT][CPL], const FfnArgs& a,
                                              int j, int lpr_rt, int u, bool ok,
                                              const int (&out_row)[NT], const int (&cc)[CPL],
                                              const LdsOut& lo, const int (&slot)[NT]) {
  const int lpr = LPR ? LPR : lpr_rt;
  float acc0[NT], acc1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc0[t] = acc1[t] = 0.f;
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) {
    const int sub = cc[ci] & 7;  // Q4_K sub-block of this chunk (unused otherwise)
    const ChunkScale k0 = decode_scale(s.c0[ci], sub);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc0[t] = chunk_fma(s.c0[ci], k0, xs[t][ci], acc0[t]);
    if (GATEUP) {
      const ChunkScale k1 = decode_scale(s.c1[ci], sub);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc1[t] = chunk_fma(s.c1[ci], k1, xs[t][ci], acc1[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float v0 = group_sum_last(acc0[t], lpr);
    float v = v0;
    if (GATEUP) v = silu(v0) * group_sum_last(acc1[t], lpr);
    if (ok && j == lpr - 1) {
      if (LDSOUT) {
        lo.p[slot[t] * lo.ld + (u - lo.row0)] = v;
      } else {
        float* dst = a.out + (int64_t)out_row[t] * a.rows_per_expert + u;
        if (a.coherent_out)
          store_shared(dst, v);
        else
          *dst = v;
      }
    }
  }
}

// One pass of a wave over rows first, first+step, ... < ue of `expert`, for
// the NT tokens whose pair ids are given (LDSOUT: outputs to lo, token t of
// the pass in slot lds_slot[t]).
// NSTD: ring depth (0: nst_for); LPR: lanes per row when known at compile
// time (0: a.lpr); XCOH: the activations were written earlier in this
// launch (read past L2).
template <int FMT, int CPL, int NT, bool GATEUP, int NSTD = 0, bool LDSOUT = false, int LPR = 0,
          bool XCOH = false>
__device__ __forceinline__ void ffn_pass(const FfnArgs& a, int expert, const int* pair_ids,
                                         int first, int step, int ue, LdsOut lo = LdsOut{},
                                         const int* lds_slot = nullptr) {
  constexpr int NST = NSTD ? NSTD : nst_for(FMT, CPL, GATEUP);
  const int lane = threadIdx.x & (kWave - 1);
  const int lpr = LPR ? LPR : a.lpr;
  const int g = lane / lpr;
  const int j = lane - g * lpr;
  if (first >= ue) return;  // wave-uniform

  const int64_t row0 = (int64_t)expert * a.rows_per_expert;
  const QPlanes p0 = expert_planes<FMT>(a.w0, a.total_rows, a.K, row0, a.rows_per_expert);
  const QPlanes p1 =
      expert_planes<FMT>(GATEUP ? a.w1 : a.w0, a.total_rows, a.K, row0, a.rows_per_expert);

  const int nchunks = a.K / QTraits<FMT>::kWpc;
  int cc[CPL];
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) cc[ci] = min(j + lpr * ci, nchunks - 1);

  int out_row[NT], slot[NT], xrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int p = pair_ids[t];
    out_row[t] = p;
    slot[t] = LDSOUT ? lds_slot[t] : 0;
    xrow[t] = a.act_by_pair ? p : p / a.top_k;
  }

  // Row of lane group g at step base: base + g.  The loop is branch-free
  // over whole groups of NST steps: every prefetch is issued, its row
  // clamped to the tile's last row (a line already fetched), so the wait
  // before each step counts a fixed number of loads issued after it.  Rows
  // at or past `ue` are computed but not written.
  // Plane offsets advance by a fixed amount per step; clamping an offset
  // to the last row's is clamping the row (both are increasing in it).
  const uint32_t q_last = (uint32_t)(ue - 1) * p0.qrow, s_last = (uint32_t)(ue - 1) * p0.srow;
  const uint32_t q_step = (uint32_t)step * p0.qrow, s_step = (uint32_t)step * p0.srow;
  uint32_t q_pre = (uint32_t)(first + g) * p0.qrow, s_pre = (uint32_t)(first + g) * p0.srow;
  Stage<FMT, CPL, GATEUP> S[NST];
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    load_stage(S[s], p0, p1, min(q_pre, q_last), min(s_pre, s_last), cc);
    q_pre += q_step;
    s_pre += s_step;
  }
  // The activations after the weights' first stages: both round trips
  // overlap, and the slices are quantised while the weights are in flight
  // (the scheduling barrier keeps the compiler from sinking the weight
  // loads below the quantisation).  With several lane groups per wave (all
  // needing the same slices) each slice is quantised once per wave.
  __builtin_amdgcn_sched_barrier(0);
  XSlice<FMT> xs[NT][CPL];
  if constexpr (LPR > 0 && LPR < kWave)
    load_slices_once<FMT, NT, CPL, LPR, XCOH>(xs, a.act, xrow, a.K, j, nchunks);
  else
    load_slices<FMT, NT, CPL, XCOH>(xs, a.act, xrow, a.K, j, lpr, nchunks);
  for (int base = first; base < ue; base += NST * step) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int cur = base + s * step;
      load_stage(S[(s + NST - 1) % NST], p0, p1, min(q_pre, q_last), min(s_pre, s_last), cc);
      q_pre += q_step;
      s_pre += s_step;
      compute_stage<FMT, CPL, NT, GATEUP, LDSOUT, LPR>(S[s], xs, a, j, lpr, cur + g, cur + g < ue,
                                                       out_row, cc, lo, slot);
    }
  }
}

template <int FMT, int CPL, int TP, bool GATEUP, int LPR>
__device__ __forceinline__ void ffn_pass_nt(const FfnArgs& a, int expert, const int* ids, int nt,
                                            int first, int step, int ue) {
  if (nt >= TP) {
    ffn_pass<FMT, CPL, TP, GATEUP, 0, false, LPR>(a, expert, ids, first, step, ue);
  } else if (TP > 1 && nt == 1) {
    ffn_pass<FMT, CPL, 1, GATEUP, 0, false, LPR>(a, expert, ids, first, step, ue);
  } else if (TP > 2 && nt == 2) {
    ffn_pass<FMT, CPL, (TP > 2 ? 2 : 1), GATEUP, 0, false, LPR>(a, expert, ids, first, step, ue);
  } else if (TP > 3 && nt == 3) {
    ffn_pass<FMT, CPL, (TP > 3 ? 3 : 1), GATEUP, 0, false, LPR>(a, expert, ids, first, step, ue);
  }
}

// Pair slots: rows [tile * units_per_block, ...) of the expert of (token,
// slot) pair `slot`, the four waves taking different rows.  With token
// words (gate/up), the n pairs of an expert selected by n tokens split the
// tile's row steps n ways (the pair of the expert's r-th token takes steps
// r, r + n, ...) and each runs one pass for all n tokens: the expert's rows
// are streamed once, and every workgroup has the arithmetic of a one-token
// tile.  Each output is computed as in a pass of its own token.
// SHARE: read the pairs' {expert, word} (else every pair runs its own
// pass, which gives the same outputs).
template <int FMT, int CPL, bool GATEUP, int NSTD = 0, bool LDSOUT = false, int LPR = 0,
          bool SHARE = false>
__device__ __forceinline__ void ffn_tile_pair(const FfnArgs& a, int slot, int tile,
                                              float* lds = nullptr) {
  if (slot >= a.n_pairs) return;
  const int ub = tile * a.units_per_block;
  const int ue = min(ub + a.units_per_block, a.rows_per_expert);
  if (ub >= ue) return;
  const int G = kWave / (LPR ? LPR : a.lpr);
  const int first = ub + (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * G;
  const int step = kWavesPerBlock * G;
  int e;
  if constexpr (GATEUP && !LDSOUT && SHARE) {
    if (a.pair_info) {
      const uint2 info = a.pair_info[slot];  // one load: expert and word
      e = __builtin_amdgcn_readfirstlane((int)info.x);
      const uint32_t word = __builtin_amdgcn_readfirstlane(info.y);
      const int t = slot / a.top_k;
      int ids[kPairTokens];
      int n = 0, r = 0;
#pragma unroll
      for (int u = 0; u < kPairTokens; ++u) {
        const int b = (int)((word >> (8 * u)) & 255u);
        if (b) {
          if (u < t) ++r;
          ids[n++] = u * a.top_k + b - 1;
        }
      }
      if (n > 1) {
        const int f = ub + (r * kWavesPerBlock + (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * G;
        const int s = n * step;
        // Passes of at most two tokens: a three- or four-token pass needs
        // more registers than the one-token pass (spilling into AGPRs and
        // halving the whole grid's occupancy); a second pass finds the
        // rows in L2.
        ffn_pass<FMT, CPL, 2, true, NSTD, false, LPR>(a, e, ids, f, s, ue);
        if (n == 3) {
          ffn_pass<FMT, CPL, 1, true, NSTD, false, LPR>(a, e, ids + 2, f, s, ue);
        } else if (n == 4) {
          ffn_pass<FMT, CPL, 2, true, NSTD, false, LPR>(a, e, ids + 2, f, s, ue);
        }
        return;
      }
      // n == 1: this pair's own token, the pass below
    } else {
      e = __builtin_amdgcn_readfirstlane(a.pair_expert[slot]);
    }
  } else {
    e = __builtin_amdgcn_readfirstlane(a.pair_expert[slot]);
  }
  const int ids1[1] = {slot}, slot0[1] = {0};
  ffn_pass<FMT, CPL, 1, GATEUP, NSTD, LDSOUT, LPR>(a, e, ids1, first, step, ue,
                                                   LdsOut{lds, ub, a.units_per_block}, slot0);
}

// One expert for the identity token list (the shared expert): rows
// [tile * units_per_block, ...) for every token.  With up to four tokens
// the waves form one group of 4 / M waves per token that share its rows
// (M = 3: one wave idles); with more, wave w takes tokens w, w + 4, ...
// over all rows.  So the rows are fetched from HBM once per workgroup and
// idle waves of a small batch still stream.
template <int FMT, int CPL, bool GATEUP, int NSTD = 0, int LPR = 0, bool XCOH = false>
__device__ __forceinline__ void ffn_tile_tokens(const FfnArgs& a, int tile) {
  const int ub = tile * a.units_per_block;
  const int ue = min(ub + a.units_per_block, a.rows_per_expert);
  if (ub >= ue) return;
  const int G = kWave / (LPR ? LPR : a.lpr);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (a.n_tokens <= kWavesPerBlock) {
    const int rg = kWavesPerBlock / a.n_tokens;
    const int t = wv / rg, q = wv - t * rg;
    const int ids1[1] = {t};
    if (t < a.n_tokens)
      ffn_pass<FMT, CPL, 1, GATEUP, NSTD, false, LPR, XCOH>(a, 0, ids1, ub + q * G, rg * G, ue);
    return;
  }
  for (int t = wv; t < a.n_tokens; t += kWavesPerBlock) {
    const int ids1[1] = {t};
    ffn_pass<FMT, CPL, 1, GATEUP, NSTD, false, LPR, XCOH>(a, 0, ids1, ub, G, ue);
  }
}

// Work of workgroup (tile, slot): rows [tile * units_per_block, ...) of the
// expert in `slot`, for every token routed to it.  SHARE: pair slots follow
// the token words (ffn_tile_pair).
template <int FMT, int CPL, bool GATEUP, int LPR = 0, bool SHARE = false>
__device__ __forceinline__ void ffn_tile(const FfnArgs& a, int slot, int tile) {
  constexpr int TP = tp_for(FMT, CPL);
  const int ub = tile * a.units_per_block;
  if (a.pair_expert) {
    // One (token, slot) pair per slot: every workgroup does the same work.
    ffn_tile_pair<FMT, CPL, GATEUP, 0, false, LPR, SHARE>(a, slot, tile);
    return;
  }
  if (a.n_active && slot >= *a.n_active) return;
  const int expert = a.active ? a.active[slot] : 0;
  const int begin = a.offsets ? a.offsets[expert] : 0;
  const int count = a.offsets ? a.offsets[expert + 1] - begin : a.n_tokens;
  const int ue = min(ub + a.units_per_block, a.rows_per_expert);
  if (ub >= ue || count <= 0) return;
  const int wv = threadIdx.x >> 6;
  const int G = kWave / (LPR ? LPR : a.lpr);
  int ids[TP];
  if (a.split_tokens) {
    ffn_tile_tokens<FMT, CPL, GATEUP, 0, LPR>(a, tile);
  } else {
    for (int p0 = 0; p0 < count; p0 += TP) {
#pragma unroll
      for (int t = 0; t < TP; ++t) {
        const int q = min(p0 + t, count - 1);
        ids[t] = a.slots ? a.slots[begin + q] : q;
      }
      ffn_pass_nt<FMT, CPL, TP, GATEUP, LPR>(a, expert, ids, min(TP, count - p0), ub + wv * G,
                                        kWavesPerBlock * G, ue);
    }
  }
}

// Grid: (row tiles, expert slots).
template <int FMT, int CPL, bool GATEUP>
__global__ __launch_bounds__(kBlock) void k_ffn(FfnArgs a) {
  ffn_tile<FMT, CPL, GATEUP>(a, blockIdx.y, blockIdx.x);
}

}  // namespace svr
