// Routing: router GEMV, wave-level top-k with renormalised softmax weights,
// and per-expert bucketing of (token, slot) pairs.
//
// The router is an F32 matrix ("Step-5 Preview GGUF", Precision
// distribution table, routers row); 8 of 352 experts are selected per token
// ("Step-5 Preview GGUF", Model background, configuration table).  The score
// function is not on the pages; the softmax top-k with renormalisation used
// here is the layer's contract (include/moe_layer.h).
#pragma once

#include "common.h"

namespace svr {

// ---------------------------------------------------------------------------
// Router GEMV for a small batch: one workgroup per router row, wave w taking
// quarter w of the row.  Each lane requests its float4 chunks of the row and
// of up to four tokens at once (NC per lane), so a row costs about one
// memory round trip; the four quarter sums are added in a fixed order.
// ---------------------------------------------------------------------------
// s_part[wave][row of 16 lanes][token]: partial sums, added in a fixed order.
typedef float RouterPart[kWavesPerBlock][4][16];

// Part 1: each wave's partial sums of row e for up to 16 tokens into s_part.
template <int NC>
__device__ __forceinline__ void router_row_partials(const float* __restrict__ router,
                                                    const float* __restrict__ x, int H, int M,
                                                    int e, RouterPart& s_part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int Q = H >> 4;  // float4 chunks per quarter
  const int c0 = wv * Q;
  const float* wrow = router + (int64_t)e * H;
  float4 w[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    w[i] = (c < Q) ? ldf4(wrow + 4 * (c0 + c)) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int t0 = 0; t0 < M; t0 += 4) {
    float4 v[4][NC];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + kWave * i;
        v[t][i] = (t0 + t < M && c < Q) ? ldf4(x + (int64_t)(t0 + t) * H + 4 * (c0 + c))
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        a0 = fmaf(w[i].x, v[t][i].x, a0);
        a1 = fmaf(w[i].y, v[t][i].y, a1);
        a0 = fmaf(w[i].z, v[t][i].z, a0);
        a1 = fmaf(w[i].w, v[t][i].w, a1);
      }
      const float rs = group_sum_last(a0 + a1, 16);  // row sums in lanes 15, 31, 47, 63
      if ((lane & 15) == 15 && t0 + t < M) s_part[wv][lane >> 4][t0 + t] = rs;
    }
  }
}

// Part 2 for the fused small-batch path: token threadIdx.x < M publishes
// its logit as an order-preserving key (never 0) with a write-through store;
// the routing workgroup of the same launch polls for it (topk_keys_poll).
__device__ __forceinline__ void router_row_publish(uint32_t* __restrict__ keys, int E, int M,
                                                   int e, const RouterPart& s_part) {
  if (threadIdx.x < M) {
    float acc = 0.f;
#pragma unroll
    for (int w4 = 0; w4 < kWavesPerBlock; ++w4)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc += s_part[w4][r][threadIdx.x];
    store_shared(keys + (int64_t)threadIdx.x * E + e, order_key(acc));
  }
}

template <int NC>
__device__ __forceinline__ void router_row_keys(const float* __restrict__ router,
                                                const float* __restrict__ x,
                                                uint32_t* __restrict__ keys, int H, int E, int M,
                                                int e) {
  __shared__ RouterPart s_part;
  router_row_partials<NC>(router, x, H, M, e, s_part);
  __syncthreads();
  router_row_publish(keys, E, M, e, s_part);
}

// Router GEMV for any batch size (prefill): one wave per router row, tokens
// four at a time, the row re-read from L2 per group.
static __global__ __launch_bounds__(kBlock) void k_router_logits(const float* __restrict__ router,
                                                          const float* __restrict__ x,
                                                          float* __restrict__ logits, int H,
                                                          int E, int M) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (e >= E) return;  // wave-uniform: no block-level barrier below
  const int H4 = H >> 2;
  const float* wrow = router + (int64_t)e * H;
  for (int t0 = 0; t0 < M; t0 += 4) {
    const int nt = min(4, M - t0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < H4; c += kWave) {
      const float4 w = ldf4(wrow + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nt) {
          const float4 v = ldf4(x + (int64_t)(t0 + i) * H + 4 * c);
          acc[i] = fmaf(w.x, v.x, acc[i]);
          acc[i] = fmaf(w.y, v.y, acc[i]);
          acc[i] = fmaf(w.z, v.z, acc[i]);
          acc[i] = fmaf(w.w, v.w, acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = wave_sum(acc[i]);
      if (i < nt && lane == 0) logits[(int64_t)(t0 + i) * E + e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k of one token by one wave.  Lane l holds logits e = l + 64*i as
// order-preserving 32-bit keys (larger logit, larger key; -0 taken as +0,
// NaN as -inf), and keeps as its candidate the best of its untaken ones
// (largest key, then lowest index).  Each of the k rounds takes the wave
// maximum of the candidate keys with DPP row scans and row broadcasts; the
// lane holding it (the lowest expert index if keys tie exactly) owns the
// winner, marks it taken and refreshes its candidate.  Then
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
// ---------------------------------------------------------------------------

// Selection of one token from its keys in registers: key[i] is the key of
// expert lane + 64 i (0, below every real key, for lanes past E).  With
// `poison` the weights are written as NaN (a routing wait gave up), so the
// layer's outputs show it.
struct TopkLane {
  int e;    // lane j < k: the j-th selected expert
  float w;  // its renormalised weight
};

template <int NV>
__device__ __forceinline__ TopkLane topk_select(const uint32_t (&key)[NV], int E,
                                                int32_t* __restrict__ ids,
                                                float* __restrict__ wts, int k, bool coherent,
                                                bool poison) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nv = (E + kWave - 1) / kWave;
  // Candidate: best untaken local key (bit i of `taken` marks key[i] taken).
  uint32_t taken = 0u;
  uint32_t ck = 0u;
  int ci = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (i < nv && key[i] > ck) {
      ck = key[i];
      ci = i;
    }
  uint32_t my_key = 0u;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    const uint32_t best = wave_max_u32(ck);
    const uint64_t hold = __ballot(ck == best);
    int wl;
    if (__popcll(hold) == 1) {
      wl = __ffsll((unsigned long long)hold) - 1;
    } else {  // exact tie between lanes: the lowest expert index wins
      const uint32_t e_me = (ck == best) ? (uint32_t)(lane + kWave * ci) : 0xFFFFFFFFu;
      wl = (int)(wave_min_u32(e_me) & (kWave - 1));
    }
    const int we = __builtin_amdgcn_readlane(lane + kWave * ci, wl);
    if (lane == j) {
      my_key = best;
      my_e = we;
    }
    if (lane == wl) {
      taken |= 1u << ci;
      ck = 0u;
      ci = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i < nv && !((taken >> i) & 1u) && key[i] > ck) {
          ck = key[i];
          ci = i;
        }
    }
  }
  const float my_v = key_value(my_key);
  const float vmax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
  const float ex = (lane < k) ? __expf(my_v - vmax) : 0.f;
  const float tot = wave_sum(ex);
  const float wj = poison ? __builtin_nanf("") : ex / tot;
  if (lane < k && ids) {
    if (coherent) {  // read by other workgroups of the same launch
      store_shared(ids + lane, (int32_t)my_e);
      store_shared(wts + lane, wj);
    } else {
      ids[lane] = my_e;
      wts[lane] = wj;
    }
  }
  return TopkLane{my_e, wj};
}

template <bool COHERENT, int NV>
__device__ __forceinline__ void topk_token_nv(const float* __restrict__ row,
                                              int32_t* __restrict__ ids, float* __restrict__ wts,
                                              int E, int k) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nv = (E + kWave - 1) / kWave;
  uint32_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    key[i] = 0u;  // below every real key: never selected while k <= E
    if (i < nv && e < E) key[i] = order_key(COHERENT ? load_shared(row + e) : row[e]);
  }
  (void)topk_select<NV>(key, E, ids, wts, k, COHERENT, false);
}

// Polls allowed for one token's keys (each a round trip past L2 and a short
// sleep): far beyond any launch, only a bound so that no wave can wait
// forever.
constexpr int kKeyPollLimit = 1 << 20;

// A wave reads one token's keys, published by other workgroups of this
// launch with write-through stores, past L2 until none is 0 (a bounded
// number of polls).  Returns false, and sets *err, if it gave up.
template <int NV>
__device__ __forceinline__ bool poll_keys(const uint32_t* __restrict__ row, int E,
                                          uint32_t (&key)[NV], unsigned* err) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nv = (E + kWave - 1) / kWave;
  bool missing = true;
  for (int n = 0; n < kKeyPollLimit; ++n) {
    missing = false;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + kWave * i;
      key[i] = 0u;
      if (i < nv && e < E) {
        key[i] = load_shared(row + e);
        missing |= key[i] == 0u;
      }
    }
    if (__ballot(missing) == 0) break;
    __builtin_amdgcn_s_sleep(1);
  }
  const bool gave_up = __ballot(missing) != 0;
  if (gave_up && lane == 0) store_shared(err, 1u);
  return !gave_up;
}

// Top-k of one token whose keys other workgroups of this launch publish
// with write-through stores (router_row_publish): poll, select, and clear
// the row for the next call.  If the poll gave up the token's weights are
// poisoned (NaN).
template <int NV>
__device__ __forceinline__ TopkLane topk_keys_poll_nv(uint32_t* __restrict__ row,
                                                      int32_t* __restrict__ ids,
                                                      float* __restrict__ wts, int E, int k,
                                                      unsigned* err) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nv = (E + kWave - 1) / kWave;
  uint32_t key[NV];
  const bool ok = poll_keys<NV>(row, E, key, err);
  const TopkLane res = topk_select<NV>(key, E, ids, wts, k, true, !ok);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    if (i < nv && e < E) store_shared(row + e, 0u);
  }
  return res;
}

// Lane j < k of the result holds the token's j-th expert and weight.
__device__ __forceinline__ TopkLane topk_keys_poll(uint32_t* __restrict__ row,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ wts, int E, int k,
                                                   unsigned* err) {
  if (E <= 5 * kWave) return topk_keys_poll_nv<5>(row, ids, wts, E, k, err);
  if (E <= 6 * kWave) return topk_keys_poll_nv<6>(row, ids, wts, E, k, err);
  if (E <= 8 * kWave) return topk_keys_poll_nv<8>(row, ids, wts, E, k, err);
  return topk_keys_poll_nv<kMaxExperts / kWave>(row, ids, wts, E, k, err);
}

// NV keys per lane, the fewest that hold E: 5 for up to 320 experts (the
// Step-3.5-Flash shape, 288), 6 for up to 384 (Step-5, 352), then 8 and 16.
template <bool COHERENT>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int32_t* __restrict__ ids,
                                           float* __restrict__ wts, int E, int k) {
  if (E <= 5 * kWave)
    topk_token_nv<COHERENT, 5>(row, ids, wts, E, k);
  else if (E <= 6 * kWave)
    topk_token_nv<COHERENT, 6>(row, ids, wts, E, k);
  else if (E <= 8 * kWave)
    topk_token_nv<COHERENT, 8>(row, ids, wts, E, k);
  else
    topk_token_nv<COHERENT, kMaxExperts / kWave>(row, ids, wts, E, k);
}

static __global__ __launch_bounds__(kBlock) void k_topk(const float* __restrict__ logits,
                                                 int32_t* __restrict__ ids,
                                                 float* __restrict__ wts, int E, int k, int M) {
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= M) return;
  topk_token<false>(logits + (int64_t)t * E, ids + (int64_t)t * k, wts + (int64_t)t * k, E, k);
}

// ---------------------------------------------------------------------------
// Shared experts of a verify batch (up to kPairTokens tokens, pair slots).
// Pair p = t*k + j gets {expert, word}, where byte u of the word is 1 + the
// slot of token u's pair on the same expert (0: token u does not select
// it): every pair of an expert gets the same word, and the expert's gate/up
// pass serves all of its tokens at once, its rows split between those
// pairs' workgroups.  One wave (every lane calls it) builds
// the words in an LDS table of one word per expert (`table`, E words): each
// pair clears its expert's word, ORs in its own byte (a token selects an
// expert at most once, so no bytes collide), and reads the word back.  The
// LDS operations of one wave complete in order, so no barrier is needed
// between the steps.  ids: the M*k selected experts (global or LDS).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pair_infos_wave(const int32_t* ids, int M, int k,
                                                uint32_t* table, uint2* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int P = M * k;
  // (an expert id outside [0, kMaxExperts) would only come from a routing
  // that gave up; it still indexes inside the table)
  auto slot_of = [&](int p) { return (uint32_t)ids[p] & (uint32_t)(kMaxExperts - 1); };
  for (int p = lane; p < P; p += kWave) table[slot_of(p)] = 0u;
  for (int p = lane; p < P; p += kWave) {
    const int t = p / k;
    atomicOr(&table[slot_of(p)], (uint32_t)(p - t * k + 1) << (8 * t));
  }
  for (int p = lane; p < P; p += kWave) out[p] = make_uint2((uint32_t)ids[p], table[slot_of(p)]);
}

static __global__ __launch_bounds__(kWave) void k_pair_infos(const int32_t* __restrict__ ids,
                                                             uint2* __restrict__ out, int M,
                                                             int k) {
  __shared__ uint32_t table[kMaxExperts];
  pair_infos_wave(ids, M, k, table, out);
}

// ---------------------------------------------------------------------------
// Bucketing by one workgroup: counts[E], offsets[E+1] (exclusive scan),
// active[] (experts with pairs, ascending, then -1), n_active, and slots[]:
// the pair indices p = t*k + j of each expert in ascending p (so ascending
// t).  Pairs are ranked in order by wave 0, 64 at a time: lanes holding the
// same expert are matched with ballots over the id bits, and the rank of a
// pair among equal ids of its chunk is a popcount.
// ---------------------------------------------------------------------------
struct BucketOut {
  int32_t *counts, *offsets, *slots, *active, *n_active;
};

__device__ void bucket_block(const int32_t* __restrict__ ids, int n_pairs, int E,
                             const BucketOut& o) {
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_cur[kMaxExperts];
  __shared__ int32_t s_wave_c[kWavesPerBlock], s_wave_a[kWavesPerBlock];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kBlock) s_cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < n_pairs; p += kBlock) atomicAdd(&s_cnt[ids[p]], 1);
  __syncthreads();
  // Exclusive scans of the counts and of the active flags over E <= 1024
  // experts: each thread owns 4 consecutive experts.
  int c4[4], a4[4];
  int csum = 0, asum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    c4[i] = (e < E) ? s_cnt[e] : 0;
    a4[i] = c4[i] > 0;
    csum += c4[i];
    asum += a4[i];
  }
  int cinc = csum, ainc = asum;
  const int lane = tid & (kWave - 1), wv = tid >> 6;
  for (int off = 1; off < kWave; off <<= 1) {
    const int oc = __shfl_up(cinc, off, kWave);
    const int oa = __shfl_up(ainc, off, kWave);
    if (lane >= off) {
      cinc += oc;
      ainc += oa;
    }
  }
  if (lane == kWave - 1) {
    s_wave_c[wv] = cinc;
    s_wave_a[wv] = ainc;
  }
  __syncthreads();
  int cbase = 0, abase = 0;
  for (int w = 0; w < wv; ++w) {
    cbase += s_wave_c[w];
    abase += s_wave_a[w];
  }
  int cex = cbase + cinc - csum, aex = abase + ainc - asum;
  if (tid == kBlock - 1 && o.n_active) *o.n_active = aex + asum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < E) {
      if (o.counts) o.counts[e] = c4[i];
      if (o.offsets) o.offsets[e] = cex;
      s_cur[e] = cex;
      if (o.active) o.active[e] = -1;
    }
    cex += c4[i];
  }
  if (tid == kBlock - 1 && o.offsets) o.offsets[E] = cex;
  __syncthreads();
  if (o.active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E && a4[i]) o.active[aex] = e;
      aex += a4[i];
    }
  }
  if (o.slots && wv == 0) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int p0 = 0; p0 < n_pairs; p0 += kWave) {
      const int p = p0 + lane;
      const bool valid = p < n_pairs;
      const int e = valid ? ids[p] : -1;
      uint64_t same = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
      }
      if (valid) o.slots[s_cur[e] + __popcll(same & below)] = p;
      __builtin_amdgcn_wave_barrier();
      if (valid && (same & below) == 0) s_cur[e] += __popcll(same);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

static __global__ __launch_bounds__(kBlock) void k_bucket(const int32_t* __restrict__ ids, int n_pairs,
                                                   int E, BucketOut o) {
  bucket_block(ids, n_pairs, E, o);
}

// The same outputs for large batches, by one workgroup of 16 waves: wave w
// ranks its own contiguous chunk of pairs, starting each expert's cursor at
// the expert's offset plus the pairs of that expert in earlier chunks.
constexpr int kWideWaves = 16;
constexpr int kWideBlock = kWideWaves * kWave;

static __global__ __launch_bounds__(kWideBlock) void k_bucket_wide(const int32_t* __restrict__ ids,
                                                            int n_pairs, int E, BucketOut o) {
  __shared__ int32_t s_hist[kWideWaves][kMaxExperts];  // per-chunk counts, then cursors
  __shared__ int32_t s_wc[kWideWaves], s_wa[kWideWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  for (int i = tid; i < kWideWaves * kMaxExperts; i += kWideBlock) s_hist[i / kMaxExperts][i % kMaxExperts] = 0;
  const int chunk = (n_pairs + kWideWaves * kWave - 1) / (kWideWaves * kWave) * kWave;
  const int c0 = min(wv * chunk, n_pairs), c1 = min(c0 + chunk, n_pairs);
  __syncthreads();
  for (int p = c0 + lane; p < c1; p += kWave) atomicAdd(&s_hist[wv][ids[p]], 1);
  __syncthreads();
  // Thread e: expert e's count, and its per-chunk counts turned into
  // exclusive prefixes over the chunks.
  int cnt = 0;
  if (tid < E) {
    for (int w = 0; w < kWideWaves; ++w) {
      const int h = s_hist[w][tid];
      s_hist[w][tid] = cnt;
      cnt += h;
    }
  }
  const int act = cnt > 0;
  int cinc = cnt, ainc = act;
  for (int off = 1; off < kWave; off <<= 1) {
    const int oc = __shfl_up(cinc, off, kWave);
    const int oa = __shfl_up(ainc, off, kWave);
    if (lane >= off) {
      cinc += oc;
      ainc += oa;
    }
  }
  if (lane == kWave - 1) {
    s_wc[wv] = cinc;
    s_wa[wv] = ainc;
  }
  if (tid < E && o.active) o.active[tid] = -1;
  __syncthreads();
  int cbase = 0, abase = 0;
  for (int w = 0; w < wv; ++w) {
    cbase += s_wc[w];
    abase += s_wa[w];
  }
  const int off = cbase + cinc - cnt, aex = abase + ainc - act;
  if (tid < E) {
    if (o.counts) o.counts[tid] = cnt;
    if (o.offsets) o.offsets[tid] = off;
    if (o.active && act) o.active[aex] = tid;
    for (int w = 0; w < kWideWaves; ++w) s_hist[w][tid] += off;
  }
  if (tid == E - 1) {
    if (o.offsets) o.offsets[E] = off + cnt;
    if (o.n_active) *o.n_active = aex + act;
  }
  __syncthreads();
  if (!o.slots) return;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int p0 = c0; p0 < c1; p0 += kWave) {
    const int p = p0 + lane;
    const bool valid = p < c1;
    const int e = valid ? ids[p] : -1;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    if (valid) o.slots[s_hist[wv][e] + __popcll(same & below)] = p;
    __builtin_amdgcn_wave_barrier();
    if (valid && (same & below) == 0) s_hist[wv][e] += __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace svr
