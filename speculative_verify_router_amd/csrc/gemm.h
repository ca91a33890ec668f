// Batched (prefill) path: the expert FFNs as grouped GEMMs on the bf16
// matrix cores, and the router as an fp32 MFMA GEMM.
//
// Precision scheme.  Quant values are integers and go into the MFMA
// exactly; scales stay fp32 and are applied once per 32-column sub-block;
// activations go in as two bf16 terms, hi = x truncated to bf16 and
// lo = bf16(x - hi), so that hi + lo carries 16 significant bits of x
// ("Step-5 Preview GGUF": prefill micro-batches of 512 tokens; the tensor
// types are the Q4_K / Q8_0 of its precision table).
//
// Operands of v_mfma_f32_16x16x32_bf16 (D[16][16] += A[16][32] B[32][16]):
// lane l = 16 g + n holds A row n, columns 8g..8g+7, B columns n, rows
// 8g..8g+7, and D rows 4g..4g+3 of column n.  A = 16 activation rows
// (tokens), B = 16 weight rows, so each lane's outputs belong to ONE weight
// row and four tokens, and a per-row scale is one scalar per lane.
//
// Within a group of 8 columns the operands are taken in the order
// 0,4,1,5,2,6,3,7 (the order in which shifts and masks pull the nibbles of
// a Q4_K dword apart); activations are stored in that order.
//
// Q4_K weights enter as the bf16 value 1 + q/16 (exponent of 1, q in the
// top four mantissa bits: one shift and one AND-OR per pair), so with
// P = sum (1 + q/16) x over a sub-block and X = sum x,
//   sum w x = 16 d sc (P - X) - dmin m X = a P - c X,
//   a = 16 d sc,  c = a + dmin m.
// X comes from the same MFMA with an all-ones B operand, in the D layout.
// Q8_0 weights are the int8 values converted to bf16 (exact), sum w x = d P.
#pragma once

#include "common.h"
#include "quant.h"

namespace svr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Split activations.  Row layout: for each group of 8 columns, 16 bytes of
// hi terms then 16 bytes of lo terms, both in the order 0,4,1,5,2,6,3,7:
// 4 bytes per element, K * 4 bytes per row.

__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// hi / lo bf16 terms of v (finite): hi = truncation, lo = RNE(v - hi).
__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  hi = u >> 16;
  lo = bf16_rne_bits(v - __builtin_bit_cast(float, u & 0xFFFF0000u));
}

// Eight consecutive columns v[0..7] -> (hi dwords, lo dwords) in operand order.
__device__ __forceinline__ void split8(const float (&v)[8], uint4& hi, uint4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_bf16(v[i], h[i], l[i]);
  hi = make_uint4(h[0] | h[4] << 16, h[1] | h[5] << 16, h[2] | h[6] << 16, h[3] | h[7] << 16);
  lo = make_uint4(l[0] | l[4] << 16, l[1] | l[5] << 16, l[2] | l[6] << 16, l[3] | l[7] << 16);
}

// x[rows][K] fp32 -> xs[rows][K] split.  One thread per 8 columns.
__global__ __launch_bounds__(kBlock) void k_split_act(const float* __restrict__ x, int64_t n8,
                                                      uint4* __restrict__ xs) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n8) return;
  const float4 a = ldf4(x + 8 * i), b = ldf4(x + 8 * i + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint4 hi, lo;
  split8(v, hi, lo);
  xs[2 * i] = hi;
  xs[2 * i + 1] = lo;
}

// ---------------------------------------------------------------------------
// Token tiles: up to 16 consecutive positions of one expert's bucket.
// Routed: built from the bucket offsets (experts in index order); dense (the
// shared expert): positions are tokens, tile i = tokens 16i.. .

struct TileList {
  int32_t* tiles;    // [cap][3]: expert, first position, count
  int32_t* n_tiles;  // [1]
};

// One workgroup; E <= kMaxExperts.  Exclusive scan of ceil(count / 16)
// over the experts, then each expert writes its tiles.
__global__ __launch_bounds__(kBlock) void k_tiles(const int32_t* __restrict__ offsets, int E,
                                                  TileList tl) {
  __shared__ int s_wave[kWavesPerBlock];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  int n4[4], c4[4], o4[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    o4[i] = (e < E) ? offsets[e] : 0;
    c4[i] = (e < E) ? offsets[e + 1] - o4[i] : 0;
    n4[i] = (c4[i] + 15) >> 4;
    sum += n4[i];
  }
  int inc = sum;
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == kWave - 1) s_wave[wv] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wv; ++w) base += s_wave[w];
  int t = base + inc - sum;
  if (tid == kBlock - 1) *tl.n_tiles = t + sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < n4[i]; ++j, ++t) {
      tl.tiles[3 * t] = tid * 4 + i;
      tl.tiles[3 * t + 1] = o4[i] + 16 * j;
      tl.tiles[3 * t + 2] = min(16, c4[i] - 16 * j);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM over token tiles.

struct GemmArgs {
  const uint8_t* w0;  // planar tensor: gate or down
  const uint8_t* w1;  // up (gate/up pass), else unused
  int64_t total_rows;  // rows of the stacked tensor
  int rows;            // output rows per expert (R)
  int K;               // columns
  const uint4* act;    // split activations, rows of K * 4 bytes
  int64_t act_rows;    // rows in act (bounds of its buffer resource)
  void* out;           // gate/up: split h rows of R * 4 bytes; down: fp32 rows of R
  const int32_t* tiles;    // routed tile list, or nullptr (dense)
  const int32_t* n_tiles;  // routed tile count
  int dense_tokens;        // dense: number of tokens
  const int32_t* slots;    // routed: position -> pair id (token * top_k + slot)
  int top_k;
  int act_gather;    // activation row = slots[pos] / top_k (else pos)
  int out_scatter;   // output row = slots[pos] (else pos)
  int row_blocks;    // workgroups per token tile
};

// Q4_K sub-block i (0..7; a constant once unrolled) of a super-block
// header h: a = 16 d sc, c = a + dmin m (d16 = 16 d).
__device__ __forceinline__ void q4k_scale(const uint4& h, int i, float d16, float dmin, float& a,
                                          float& c) {
  const uint64_t lo = (uint64_t)h.y | ((uint64_t)h.z << 32);
  const uint64_t hi = (uint64_t)h.z | ((uint64_t)h.w << 32);
  const uint32_t sc = (uint32_t)(lo >> (6 * i)) & 63u;
  const uint32_t m = (uint32_t)(hi >> (16 + 6 * i)) & 63u;
  a = d16 * (float)sc;
  c = fmaf(dmin, (float)m, a);
}

// One Q4_K dword (8 nibbles, weights 8g..8g+7 of a sub-block) -> B operand
// elements 1 + q/16 in the order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u32x4 q4k_operand(uint32_t w) {
  constexpr uint32_t kMask = 0x00780078u, kOne = 0x3F803F80u;
  u32x4 b;
  b.x = ((w << 3) & kMask) | kOne;
  b.y = ((w >> 1) & kMask) | kOne;
  b.z = ((w >> 5) & kMask) | kOne;
  b.w = ((w >> 9) & kMask) | kOne;
  return b;
}

// Two Q8_0 dwords (int8 weights 8g..8g+7) -> bf16 B operand elements.
__device__ __forceinline__ u32x4 q8_operand(uint32_t w0, uint32_t w1) {
  u32x4 b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float f0 = (float)(int)(int8_t)(w0 >> (8 * j));
    const float f1 = (float)(int)(int8_t)(w1 >> (8 * j));
    // Small integers: the bf16 truncation is exact.
    b[j] = (__builtin_bit_cast(uint32_t, f0) >> 16) | (__builtin_bit_cast(uint32_t, f1) & 0xFFFF0000u);
  }
  return b;
}

// Per step (one 32-column sub-block) the operands a wave loads.
template <int FMT, int NM, int RTR>
struct GStep {
  uint4 ahi, alo;                                   // activations (A operand)
  uint32_t w[NM][RTR][FMT == kQ8_0 ? 2 : 1];  // weight dwords (B operand)
  uint32_t d[NM][RTR];                         // Q8_0 fp16 scale bits
};

// Steps of the software pipeline kept in flight.
constexpr int kGemmRing = 4;

// A wave's work: token tile (first position pos0, cnt tokens) x RTR row
// tiles of 16 rows from r0, of NM matrices (2: gate and up).  Outputs:
// gate/up -> h = silu(gate) * up, split; down -> fp32.
template <int FMT, bool GATEUP, int RTR>
__device__ __forceinline__ void gemm_wave(const GemmArgs& a, int e, int pos0, int cnt, int r0) {
  constexpr int NM = GATEUP ? 2 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, g = lane >> 4;
  const int S = a.K >> 5;  // sub-blocks

  // Activation row of this lane's A operand (row n of the tile).  Rows
  // past the tile repeat its first row: they only feed output rows that are
  // not stored.
  const int pos = pos0 + (n < cnt ? n : 0);
  const int arow = a.act_gather ? a.slots[pos] / a.top_k : pos;
  const uint32_t aoff = (uint32_t)arow * (uint32_t)a.K * 4u + 32u * (uint32_t)g;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.act, (uint32_t)(a.act_rows * a.K * 4));

  QPlanes P[NM];
  P[0] = expert_planes<FMT>(a.w0, a.total_rows, a.K, (int64_t)e * a.rows, a.rows);
  if (GATEUP) P[NM - 1] = expert_planes<FMT>(a.w1, a.total_rows, a.K, (int64_t)e * a.rows, a.rows);
  // Byte offsets of this lane's weight row (row r0 + 16 rt + n) in each plane.
  uint32_t qo[RTR], so[RTR];
#pragma unroll
  for (int rt = 0; rt < RTR; ++rt) {
    const uint32_t r = (uint32_t)(r0 + 16 * rt + n);
    qo[rt] = r * P[0].qrow + (FMT == kQ8_0 ? 8u : 4u) * (uint32_t)g;
    so[rt] = r * P[0].srow;
  }

  auto load_step = [&](GStep<FMT, NM, RTR>& st, int s) {
    const uint32_t ao = aoff + 128u * (uint32_t)s;
    st.ahi = bload16(ar, ao);
    st.alo = bload16(ar, ao + 16u);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RTR; ++rt) {
        if constexpr (FMT == kQ4_K) {
          st.w[m][rt][0] = __builtin_amdgcn_raw_buffer_load_b32(P[m].q, qo[rt] + 16u * s, 0, 0);
        } else {
          const uint32_t o = qo[rt] + 32u * s;
          st.w[m][rt][0] = __builtin_amdgcn_raw_buffer_load_b32(P[m].q, o, 0, 0);
          st.w[m][rt][1] = __builtin_amdgcn_raw_buffer_load_b32(P[m].q, o + 4u, 0, 0);
          st.d[m][rt] = bload2(P[m].s, so[rt] + 2u * s);
        }
      }
  };

  f32x4 acc[NM][RTR];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < RTR; ++rt) acc[m][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  GStep<FMT, NM, RTR> ring[kGemmRing];
#pragma unroll
  for (int i = 0; i < kGemmRing - 1; ++i) load_step(ring[i], min(i, S - 1));

  // Q4_K super-block headers (16 bytes per 8 sub-blocks) of the lane's
  // rows: the current one, and the next one loaded a super-block ahead so
  // that waiting for it never drains the ring.
  uint4 hd[NM][RTR], hn[NM][RTR];
  float d16[NM][RTR], dmn[NM][RTR];
  if constexpr (FMT == kQ4_K) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RTR; ++rt) hn[m][rt] = bload16(P[m].s, so[rt]);
  }

  // Steps come in groups of 8 (one Q4_K super-block; Q8_0 pads the last
  // group with zero-scale steps).  Ring slot of step s is s % kGemmRing.
  for (int s0 = 0; s0 < S; s0 += 8) {
    if constexpr (FMT == kQ4_K) {
      const uint32_t next = 2u * (uint32_t)min(s0 + 8, S - 8);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt) {
          hd[m][rt] = hn[m][rt];
          hn[m][rt] = bload16(P[m].s, so[rt] + next);
          d16[m][rt] = 16.0f * f16_lo(hd[m][rt].x);
          dmn[m][rt] = f16_hi(hd[m][rt].x);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s0 + i;
      load_step(ring[(i + kGemmRing - 1) % kGemmRing], min(s + kGemmRing - 1, S - 1));
      const GStep<FMT, NM, RTR>& st = ring[i % kGemmRing];
      const u32x4 ahi = {st.ahi.x, st.ahi.y, st.ahi.z, st.ahi.w};
      const u32x4 alo = {st.alo.x, st.alo.y, st.alo.z, st.alo.w};
      f32x4 X = zero;
      if constexpr (FMT == kQ4_K) X = mfma_bf16(alo, ones, mfma_bf16(ahi, ones, zero));
      const bool live = s < S;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt) {
          u32x4 b;
          float sa, sc = 0.f;
          if constexpr (FMT == kQ4_K) {
            b = q4k_operand(st.w[m][rt][0]);
            q4k_scale(hd[m][rt], i, d16[m][rt], dmn[m][rt], sa, sc);
          } else {
            b = q8_operand(st.w[m][rt][0], st.w[m][rt][1]);
            sa = live ? f16_to_f32(st.d[m][rt]) : 0.f;
          }
          const f32x4 p = mfma_bf16(alo, b, mfma_bf16(ahi, b, zero));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v = fmaf(sa, p[j], acc[m][rt][j]);
            if constexpr (FMT == kQ4_K) v = fmaf(-sc, X[j], v);
            acc[m][rt][j] = v;
          }
        }
    }
  }

  // Epilogue: lane holds rows r0 + 16 rt + n for tokens 4g + j.
#pragma unroll
  for (int rt = 0; rt < RTR; ++rt) {
    const int r = r0 + 16 * rt + n;
    if (r >= a.rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * g + j;
      if (t >= cnt) continue;
      const int pos = pos0 + t;
      const int orow = a.out_scatter ? a.slots[pos] : pos;
      if (GATEUP) {
        const float h = silu(acc[0][rt][j]) * acc[NM - 1][rt][j];
        uint32_t hi, lo;
        split_bf16(h, hi, lo);
        // Element r of the row: group r / 8, operand position of r % 8.
        const int q = r & 7;
        const int p = (q < 4) ? 2 * q : 2 * (q - 4) + 1;
        uint16_t* row = reinterpret_cast<uint16_t*>(a.out) + (int64_t)orow * a.rows * 2;
        row[(r >> 3) * 16 + p] = (uint16_t)hi;
        row[(r >> 3) * 16 + 8 + p] = (uint16_t)lo;
      } else {
        reinterpret_cast<float*>(a.out)[(int64_t)orow * a.rows + r] = acc[0][rt][j];
      }
    }
  }
}

// Grid: row_blocks x (token-tile capacity rounded up to 8).  Blocks go to
// the eight XCDs round-robin; block b takes token tile 8 (b / 8 / row_blocks)
// + b % 8 and row block (b / 8) % row_blocks, so the row blocks of one token
// tile share an XCD (and its L2 copy of the tile's activations) and the
// tiles spread over all XCDs.
template <int FMT, bool GATEUP, int RTR>
__global__ __launch_bounds__(kBlock) void k_gemm(GemmArgs a) {
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int tile = (j / a.row_blocks) * 8 + xcd, rb = j % a.row_blocks;
  int e, pos0, cnt;
  if (a.tiles) {
    if (tile >= *a.n_tiles) return;
    e = a.tiles[3 * tile];
    pos0 = a.tiles[3 * tile + 1];
    cnt = a.tiles[3 * tile + 2];
  } else {
    e = 0;
    pos0 = 16 * tile;
    cnt = min(16, a.dense_tokens - pos0);
    if (cnt <= 0) return;
  }
  const int r0 = (rb * kWavesPerBlock + (threadIdx.x >> 6)) * 16 * RTR;
  if (r0 >= a.rows) return;
  gemm_wave<FMT, GATEUP, RTR>(a, e, pos0, cnt, r0);
}

// ---------------------------------------------------------------------------
// Router logits for a batch: l[t][e] = sum_h Wr[e][h] x[t][h] on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32, lane 16 g + n: A row n column g, B
// column n row g, D rows 4g..4g+3 of column n).  A workgroup computes one
// 16-token x 16-expert tile; its four waves take quarters of H and their
// partial tiles are added in LDS in a fixed order.

__global__ __launch_bounds__(kBlock) void k_router_mfma(const float* __restrict__ wr,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ logits, int H, int E,
                                                        int M) {
  __shared__ f32x4 s_part[kWavesPerBlock - 1][kWave];
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int t0 = 16 * blockIdx.x, e0 = 16 * blockIdx.y;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * (uint32_t)H * 4u);
  const __amdgpu_buffer_rsrc_t wrr = make_rsrc(wr, (uint32_t)E * (uint32_t)H * 4u);
  // Rows past M or E read as zero (offsets past the resources).
  const uint32_t xo = (t0 + n < M) ? (uint32_t)(t0 + n) * H * 4u : 0xFFFFFFF0u;
  const uint32_t wo = (e0 + n < E) ? (uint32_t)(e0 + n) * H * 4u : 0xFFFFFFF0u;
  const int kq = H / kWavesPerBlock;  // H % 64 == 0
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = wv * kq; k < (wv + 1) * kq; k += 16) {
    const uint32_t ko = 4u * (uint32_t)(k + 4 * g);
    const f32x4 av = __builtin_amdgcn_raw_buffer_load_b128(xr, xo == 0xFFFFFFF0u ? xo : xo + ko, 0, 0);
    const f32x4 bv = __builtin_amdgcn_raw_buffer_load_b128(wrr, wo == 0xFFFFFFF0u ? wo : wo + ko, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
  }
  if (wv > 0) s_part[wv - 1][lane] = acc;
  __syncthreads();
  if (wv > 0) return;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock - 1; ++w) acc += s_part[w][lane];
  const int e = e0 + n;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 4 * g + j;
    if (t < M && e < E) logits[(int64_t)t * E + e] = acc[j];
  }
}

}  // namespace svr
