// Routing kernels: router GEMV, wave-level top-k with renormalised softmax
// weights, and per-expert bucketing of (token, slot) pairs.
//
// The router is an F32 matrix ("Step-5 Preview GGUF", Precision
// distribution table, routers row); 8 of 352 experts are selected per token
// ("Step-5 Preview GGUF", Model background, configuration table).  The score
// function is not on the pages; the softmax top-k with renormalisation used
// here is the layer's stated contract (include/moe_layer.h).
#pragma once

#include "common.h"

namespace svr {

// ---------------------------------------------------------------------------
// Router GEMV: logits[t][e] = sum_h router[e][h] * x[t][h].
// One wave per router row; lane l reads float4 chunks l, l+64, ... of the
// row (1 KiB per wave instruction, fully coalesced) and the same chunks of
// up to 4 tokens at a time, then a butterfly sum per token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_router_logits(const float* __restrict__ router,
                                                          const float* __restrict__ x,
                                                          float* __restrict__ logits, int H,
                                                          int E, int M) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
  if (e >= E) return;  // wave-uniform: no block-level barrier below
  const int H4 = H >> 2;
  const float* wrow = router + (size_t)e * H;
  for (int t0 = 0; t0 < M; t0 += 4) {
    const int nt = min(4, M - t0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < H4; c += kWave) {
      const float4 w = ldf4(wrow + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nt) {
          const float4 v = ldf4(x + (size_t)(t0 + i) * H + 4 * c);
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
      if (i < nt && lane == 0) logits[(size_t)(t0 + i) * E + e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token.  Lane l holds logits e = l + 64*i.  k rounds of
// a wave arg-max on the key (value descending, index ascending); the winner
// is marked taken.  Then w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
// NaN logits are treated as -inf.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

__global__ __launch_bounds__(kBlock) void k_topk(const float* __restrict__ logits,
                                                 int32_t* __restrict__ ids,
                                                 float* __restrict__ wts, int E, int k, int M) {
  constexpr int NV = kMaxExperts / kWave;  // 16 values per lane at most
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
  if (t >= M) return;
  const float* row = logits + (size_t)t * E;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    float a = (e < E) ? row[e] : -INFINITY;
    v[i] = (a != a) ? -INFINITY : a;
  }
  uint32_t taken = 0;
  for (int i = 0; i < NV; ++i)
    if (lane + kWave * i >= E) taken |= 1u << i;
  float my_v = -INFINITY;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + kWave * i;
      if (!((taken >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oe = __shfl_xor(be, off, kWave);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float vmax = __shfl(my_v, 0, kWave);
  const float ex = (lane < k) ? __expf(my_v - vmax) : 0.f;
  const float tot = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    wts[(size_t)t * k + lane] = ex / tot;
  }
}

// ---------------------------------------------------------------------------
// Bucketing: one workgroup.  counts[E], offsets[E+1] (exclusive scan),
// active[] (experts with pairs, ascending, then -1), n_active, and
// slots[]: the pair indices p = t*k + j of each expert in ascending p (and
// so ascending t).  Pairs are ranked in order by wave 0, 64 at a time: lanes
// holding the same expert are matched with ballots over the id bits, so the
// rank of a pair among equal ids of its chunk is a popcount.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_bucket(const int32_t* __restrict__ ids, int n_pairs,
                                                   int E, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ slots,
                                                   int32_t* __restrict__ active,
                                                   int32_t* __restrict__ n_active) {
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_cur[kMaxExperts];
  __shared__ int32_t s_wave_tot[kBlock / kWave];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kBlock) s_cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < n_pairs; p += kBlock) atomicAdd(&s_cnt[ids[p]], 1);
  __syncthreads();
  // Exclusive scan of counts and of the "active" flags over E <= 1024
  // entries: each thread owns 4 consecutive experts.
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
  // Block scan of (csum, asum) packed: counts < 2^16 per expert is not
  // guaranteed, so scan the two sums separately.
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
  __shared__ int32_t s_wave_a[kBlock / kWave];
  if (lane == kWave - 1) {
    s_wave_tot[wv] = cinc;
    s_wave_a[wv] = ainc;
  }
  __syncthreads();
  int cbase = 0, abase = 0;
  for (int w = 0; w < wv; ++w) {
    cbase += s_wave_tot[w];
    abase += s_wave_a[w];
  }
  int cex = cbase + cinc - csum, aex = abase + ainc - asum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < E) {
      if (counts) counts[e] = c4[i];
      if (offsets) offsets[e] = cex;
      s_cur[e] = cex;
      if (active) active[e] = -1;
    }
    cex += c4[i];
  }
  if (tid == kBlock - 1 && offsets) offsets[E] = cex;
  if (tid == kBlock - 1 && n_active) *n_active = aex + asum;
  __syncthreads();
  if (active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E && a4[i]) active[aex] = e;
      aex += a4[i];
    }
  }
  if (slots && wv == 0) {
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
      if (valid) {
        const int rank = __popcll(same & below);
        slots[s_cur[e] + rank] = p;
      }
      __builtin_amdgcn_wave_barrier();
      if (valid && (same & below) == 0) s_cur[e] += __popcll(same);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace svr
