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
// Q4_K weights enter as the bf16 value 1 + q/128 (the exponent of 1 with q
// in the low four mantissa bits: one shift and one bit-field insert per
// pair), so with P = sum (1 + q/128) x over a sub-block and X = sum x,
//   sum w x = 128 d sc (P - X) - dmin m X = a P - c X,
//   a = 128 d sc,  c = a + dmin m.
// X comes from the same MFMA with an all-ones B operand, in the D layout.
// Q8_0 weights are the int8 values converted to bf16 (exact), sum w x = d P.
// Q2_K weights enter as 1 + sc q/128 (sc q <= 45, so the product fits the
// seven mantissa bits): a 32-column step holds two 16-weight sub-blocks
// (operand lanes g < 2 and g >= 2), and with X0 / X1 the activation sums of
// the two halves (all-ones B operands masked to those lanes)
//   sum w x = 128 d (P - X0 - X1) - dmin (m0 X0 + m1 X1) = a P - c0 X0 - c1 X1,
//   a = 128 d,  c0 = a + dmin m0,  c1 = a + dmin m1.
// Q3_K weights enter as 1 + Q/128 (Q the unsigned 3-bit quant) against
// activations masked to one half of the step at a time (P0, X0 over
// columns 0..15, P1, X1 over 16..31), and with D_h = d (S_h - 32)
//   sum w x = sum_h D_h (128 P_h - 132 X_h)   (Q - 4 = 128 (1 + Q/128) - 132).
// Q6_K the same way with its 6-bit Q (<= 63), D_h = d sc_h and
//   sum w x = sum_h D_h (128 P_h - 160 X_h)   (Q - 32 = 128 (1 + Q/128) - 160).
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
static __global__ __launch_bounds__(kBlock) void k_split_act(const float* __restrict__ x, int64_t n8,
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
static __global__ __launch_bounds__(kBlock) void k_tiles(const int32_t* __restrict__ offsets, int E,
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

// Q4_K sub-block i (0..7) of a super-block header h: a = 128 d sc,
// c = a + dmin m.  The six-bit fields are cut from the 96-bit stream
// (h.y, h.z, h.w) with 32-bit funnel shifts: 64-bit shifts would need the
// loaded words in aligned register pairs, and the copies into them would
// wait for the load.
__device__ __forceinline__ float2 q4k_scale(const uint4& h, int i) {
  const float d128 = 128.0f * f16_lo(h.x), dmin = f16_hi(h.x);
  const int bs = 6 * i, bm = 16 + 6 * i;  // sc at stream bit bs, m at 32 + bm
  const uint32_t sc =
      __builtin_amdgcn_alignbit(bs < 32 ? h.z : h.w, bs < 32 ? h.y : h.z, bs & 31) & 63u;
  const uint32_t m =
      __builtin_amdgcn_alignbit(h.w, bm < 32 ? h.z : h.w, bm & 31) & 63u;
  const float a = d128 * (float)sc;
  return make_float2(a, fmaf(dmin, (float)m, a));
}

// One Q4_K dword (8 nibbles, weights 8g..8g+7 of a sub-block) -> B operand
// elements 1 + q/128 in the order 0,4,1,5,2,6,3,7.  `one` = 0x3F803F80
// held in a VGPR the compiler cannot see through (opaque_vgpr), so that
// each pair is one v_bfi_b32 rather than an AND and an OR with literals.
__device__ __forceinline__ u32x4 q4k_operand(uint32_t w, uint32_t one) {
  constexpr uint32_t kMask = 0x000F000Fu;
  u32x4 b;
  b.x = (w & kMask) | (one & ~kMask);
  b.y = ((w >> 4) & kMask) | (one & ~kMask);
  b.z = ((w >> 8) & kMask) | (one & ~kMask);
  b.w = ((w >> 12) & kMask) | (one & ~kMask);
  return b;
}

// One Q2_K sub-block dword, shifted so that the lane's eight weights are the
// 2-bit fields at bits 8t and 8t + 2 of byte t (t = 0..3) -> B operand
// elements 1 + sc q/128 in the order 0,4,1,5,2,6,3,7.  The pair (q_t,
// q_t+4) is packed into the two halves first and multiplied by sc once
// (sc q <= 45: no carry between the halves).
__device__ __forceinline__ u32x4 q2k_operand(uint32_t u, uint32_t sc) {
  u32x4 b;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t pr = __builtin_amdgcn_ubfe(u, 8 * t, 2) | (__builtin_amdgcn_ubfe(u, 8 * t + 2, 2) << 16);
    b[t] = (pr * sc) | 0x3F803F80u;
  }
  return b;
}

// Q3_K: low bits as in q2k_operand (u), high bits of the lane's weights at
// bits 8t and 8t + 1 of hv -> B operand elements 1 + Q/128, Q = low | high << 2.
__device__ __forceinline__ u32x4 q3k_operand(uint32_t u, uint32_t hv) {
  u32x4 b;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t q0 = __builtin_amdgcn_ubfe(u, 8 * t, 2) | (__builtin_amdgcn_ubfe(hv, 8 * t, 1) << 2);
    const uint32_t q1 = __builtin_amdgcn_ubfe(u, 8 * t + 2, 2) | (__builtin_amdgcn_ubfe(hv, 8 * t + 1, 1) << 2);
    b[t] = (q0 | (q1 << 16)) | 0x3F803F80u;
  }
  return b;
}

// Q6_K: low-nibble dword w of the lane's eight weights (Q4_K order) and
// their high bit pairs in hv (weight t and t + 4 at bits 8 (t / 2) + 2 (t % 2)
// and 16 more) -> B operand elements 1 + Q/128, Q = low | high << 4.
__device__ __forceinline__ u32x4 q6k_operand(uint32_t w, uint32_t hv) {
  u32x4 b;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t lo = (w >> (4 * t)) & 0x000F000Fu;
    const uint32_t hi = (hv >> (8 * (t >> 1) + 2 * (t & 1))) & 0x00030003u;
    b[t] = lo | (hi << 4) | 0x3F803F80u;
  }
  return b;
}

// v, in a VGPR, as a value unknown to the optimiser (emits no instruction).
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
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

// K is processed in slabs of 8 sub-blocks (256 columns: one Q4_K
// super-block).  Per slab a workgroup stages in LDS
//  * the token tile's activations, once for its four waves, as
//    [step 8][hi, lo][group 4][row 16] x 16 bytes (16 KB), double-buffered;
//  * each wave's weight rows, loaded as whole 128-byte lines (lane 16 g + n
//    reads 16 bytes of row n) and read back per step in operand order, as
//    [matrix][row tile][load j][lane 64] x 16 bytes.
// Scale data (a Q4_K header, or eight Q8_0 fp16 scales: 16 bytes per row
// and slab) is fetched for eight slabs at a time, one whole 128-byte line
// per row, lane 16 g + n holding slabs 2g and 2g + 1 of row n; at each slab
// the lanes of a row take that slab's 16 bytes from the lane holding them.
// (Fetched slab by slab, the lines would leave L2 before their next 16
// bytes are needed and be read from memory eight times.)  The global loads
// of slab k+1 are issued right after slab k is written to LDS, so waits
// happen only at slab boundaries.
constexpr int kSlab = 8;
constexpr int kActSlabBytes = kSlab * 2 * 4 * 16 * 16;

// 16-byte weight loads per lane, row tile and slab (128 / 256 bytes per row).
template <int FMT>
constexpr int slab_loads() {
  return FMT == kQ4_K || FMT == kQ3_K ? 2 : FMT == kQ2_K ? 1 : FMT == kQ6_K ? 3 : 4;
}
// Formats whose 16-weight sub-block scales split each 32-column step in two
// (products against activations masked to each half).
template <int FMT>
constexpr bool split_steps() { return FMT == kQ3_K || FMT == kQ6_K; }

template <int FMT, int NM, int RTR, int TT = 1>
struct Slab {
  uint4 act[TT][4];                         // this thread's part of each tile's activation slab
  uint4 q[NM][RTR][slab_loads<FMT>()];      // weight lines
};

// Lane `src`'s value v, for every lane (ds_bpermute, four dwords).
__device__ __forceinline__ uint4 lane_fetch(int src, const uint4& v) {
  const int a = src * 4;
  return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.x),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.y),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.z),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.w));
}

template <int FMT, bool GATEUP, int RTR>
struct GemmLds {
  static constexpr int NM = GATEUP ? 2 : 1;
  static constexpr int kWaveBytes = NM * RTR * slab_loads<FMT>() * 1024;
  uint4 act[2][kActSlabBytes / 16];
  uint4 w[kWavesPerBlock][kWaveBytes / 16];
  // Per wave: (a, c) of [matrix][row tile][step pair 4][row 16][step % 2].
  float2 sc[kWavesPerBlock][NM * RTR * kSlab * 16];
};

// A workgroup's work: token tile (positions pos0.., cnt of them) x four
// waves of RTR row tiles of 16 rows (wave w: rows r0 + 16 RTR w ..), of NM
// matrices (2: gate and up).  Outputs: gate/up -> h = silu(gate) * up,
// split; down -> fp32.
//
// TT = 2 (Q8_0 only): two token tiles (pos0/cnt and pos1/cnt1; cnt1 may be
// 0) share every weight operand, each tile's products going to its own
// accumulators.  The two tiles' activation slabs take the two LDS
// activation buffers, single-buffered: a barrier before each slab's stores
// keeps them from overwriting what slower waves still read.
template <int FMT, bool GATEUP, int RTR, int TT = 1>
__device__ __forceinline__ void gemm_block(const GemmArgs& a, int e, int pos0, int cnt, int rb0,
                                           GemmLds<FMT, GATEUP, RTR>& L, int pos1 = 0,
                                           int cnt1 = 0) {
  static_assert(TT == 1 || (TT == 2 && FMT == kQ8_0), "two token tiles: Q8_0 only");
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int NQ = slab_loads<FMT>();
  // quant bytes per row and slab
  constexpr uint32_t kSlabRowBytes =
      (FMT == kQ4_K || FMT == kQ6_K) ? 128u : (FMT == kQ2_K || FMT == kQ3_K) ? 64u : 256u;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int S = a.K >> 5;  // sub-blocks
  const int NS = (S + kSlab - 1) / kSlab;
  const int r0 = rb0 + 16 * RTR * wv;

  // Activations: thread T stages LDS entries T + 256 j (j < 4), i.e. row
  // n = T % 16 of (step, hi/lo, group) u = T / 16 + 16 j, so that the 64
  // lanes of a wave write 1 KB of consecutive LDS.  Its source is unit
  // 8 step + 2 group + hi/lo of row n's 1 KB slab chunk.
  const int an = tid & 15, au = tid >> 4;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.act, (uint32_t)(a.act_rows * a.K * 4));
  uint32_t aoff[TT][4];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    // rows past a tile repeat its first row (a missing second tile: the first's)
    const int tp = (t == 1 && cnt1 > 0) ? pos1 : pos0, tc = (t == 1 && cnt1 > 0) ? cnt1 : cnt;
    const int apos = tp + (an < tc ? an : 0);
    const int arow = a.act_gather ? a.slots[apos] / a.top_k : apos;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = au + 16 * j;  // (step u / 8, hi/lo (u / 4) % 2, group u % 4)
      aoff[t][j] = (uint32_t)arow * (uint32_t)a.K * 4u +
                   16u * (uint32_t)(8 * (u >> 3) + 2 * (u & 3) + ((u >> 2) & 1));
    }
  }

  QPlanes P[NM];
  P[0] = expert_planes<FMT>(a.w0, a.total_rows, a.K, (int64_t)e * a.rows, a.rows);
  if (GATEUP) P[NM - 1] = expert_planes<FMT>(a.w1, a.total_rows, a.K, (int64_t)e * a.rows, a.rows);
  uint32_t qo[RTR], so[RTR], ho[RTR];
#pragma unroll
  for (int rt = 0; rt < RTR; ++rt) {
    const uint32_t r = (uint32_t)(r0 + 16 * rt + n);
    qo[rt] = r * P[0].qrow + 16u * (uint32_t)g;
    so[rt] = r * P[0].srow;
    // Q3_K high bits: K / 8 bytes per row (2 x the scale plane), 32 per
    // slab, lanes g and g + 2 load the same 16 bytes; Q6_K: K / 4 bytes per
    // row, 64 per slab, lane g loads bytes 16 g.
    ho[rt] = FMT == kQ6_K ? 4u * so[rt] + 16u * (uint32_t)g : 2u * so[rt] + 16u * (uint32_t)(g & 1);
  }

  const bool q8_aligned = (a.K & 255) == 0;
  // Scale data of slabs 8q + 2g (hg0) and 8q + 2g + 1 (hg1) of row n (two
  // arrays, not one: a select between them must not become an indexed
  // load from scratch memory).
  uint4 hg0[NM][RTR], hg1[NM][RTR];
  uint32_t dg0[NM][RTR], dg1[NM][RTR];  // Q2_K: d | dmin << 16 of the same slabs
  auto load_group = [&](int q) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t o = so[rt] + 16u * (uint32_t)min(8 * q + 2 * g + t, NS - 1);
          // 16-byte aligned for Q4_K and for Q8_0 rows with K % 256 == 0;
          // other Q8_0 rows (K / 16 bytes of scales) take their eight fp16
          // scales one by one.
          uint4 v;
          if (FMT != kQ8_0 || q8_aligned) {
            v = bload16(P[m].s, o);
          } else {
            uint32_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = bload2(P[m].s, o + 2u * i);
            v = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16,
                           h[6] | h[7] << 16);
          }
          if (t == 0) hg0[m][rt] = v;
          else hg1[m][rt] = v;
          if constexpr (FMT == kQ2_K || FMT == kQ3_K || FMT == kQ6_K) {
            // d-plane offset of a row = its scale-plane offset / 4 (Q2_K:
            // d | dmin) or / 8 (Q3_K, Q6_K: d)
            const uint32_t dv = FMT == kQ2_K ? bload4(P[m].d, o >> 2) : bload2(P[m].d, o >> 3);
            if (t == 0) dg0[m][rt] = dv;
            else dg1[m][rt] = dv;
          }
        }
  };
  auto load_slab = [&](Slab<FMT, NM, RTR, TT>& sl, int k) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) sl.act[t][j] = bload16(ar, aoff[t][j] + 1024u * (uint32_t)k);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RTR; ++rt) {
        if constexpr (FMT == kQ3_K) {
          sl.q[m][rt][0] = bload16(P[m].q, qo[rt] + kSlabRowBytes * (uint32_t)k);
          sl.q[m][rt][1] = bload16(P[m].h, ho[rt] + 32u * (uint32_t)k);
        } else if constexpr (FMT == kQ6_K) {
          sl.q[m][rt][0] = bload16(P[m].q, qo[rt] + kSlabRowBytes * (uint32_t)k);
          sl.q[m][rt][1] = bload16(P[m].q, qo[rt] + kSlabRowBytes * (uint32_t)k + 64u);
          sl.q[m][rt][2] = bload16(P[m].h, ho[rt] + 64u * (uint32_t)k);
        } else {
#pragma unroll
          for (int j = 0; j < NQ; ++j)
            sl.q[m][rt][j] = bload16(P[m].q, qo[rt] + kSlabRowBytes * (uint32_t)k + 64u * j);
        }
      }
  };

  f32x4 acc[NM][RTR], acc1[NM][RTR];  // acc1: the second token tile (TT = 2)
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < RTR; ++rt) acc[m][rt] = acc1[m][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t one = opaque_vgpr(0x3F803F80u);
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  // Q2_K: all-ones B operands over the first / second 16 columns of a step
  // (operand lanes g < 2 hold columns 0..15).
  const uint32_t one0 = g < 2 ? 0x3F803F80u : 0u, one1 = g < 2 ? 0u : 0x3F803F80u;
  const u32x4 ones0 = {one0, one0, one0, one0}, ones1 = {one1, one1, one1, one1};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  uint4* const wl = L.w[wv];
  float2* const scl = L.sc[wv];
  // Q2_K: the current slab's 16 scale/min bytes and a = 128 d of each row
  // (every lane of row n holds row n's).
  uint4 hks[NM][RTR];
  float aq[NM][RTR];

  // Slab k: stage it in LDS, issue the loads of slab k + 1 into the
  // registers it leaves free, compute its eight steps.
  auto consume = [&](Slab<FMT, NM, RTR, TT>& sl, int k) {
    uint4* const al = L.act[TT == 1 ? (k & 1) : 0];
    if constexpr (TT == 2) {
      if (k > 0) __syncthreads();  // every wave is done with the previous slab
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) L.act[t][tid + 256 * j] = sl.act[t][j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) al[tid + 256 * j] = sl.act[0][j];
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
        for (int j = 0; j < NQ; ++j) wl[((m * RTR + rt) * NQ + j) * 64 + lane] = sl.q[m][rt][j];
    // Scales of the slab: the four lanes of a row decode two steps each
    // (lane 16 g + n: steps 2g, 2g + 1 of row n, one 16-byte store).
    const int hsrc = 16 * ((k & 7) >> 1) + n;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RTR; ++rt) {
        const bool odd = k & 1;
        const uint4 hv = make_uint4(odd ? hg1[m][rt].x : hg0[m][rt].x, odd ? hg1[m][rt].y : hg0[m][rt].y,
                                    odd ? hg1[m][rt].z : hg0[m][rt].z, odd ? hg1[m][rt].w : hg0[m][rt].w);
        const uint4 hk = lane_fetch(hsrc, hv);
        float2 ac2[2];
        if constexpr (FMT == kQ2_K) {
          const uint32_t dk =
              (uint32_t)__builtin_amdgcn_ds_bpermute(4 * hsrc, (int)(odd ? dg1[m][rt] : dg0[m][rt]));
          const float a128 = 128.0f * f16_lo(dk), dmin = f16_hi(dk);
          hks[m][rt] = hk;
          aq[m][rt] = a128;
          // steps 2g, 2g + 1: sub-blocks 4g .. 4g + 3, mins in the high nibbles
          const uint32_t mw = g == 0 ? hk.x : g == 1 ? hk.y : g == 2 ? hk.z : hk.w;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float m0 = (float)__builtin_amdgcn_ubfe(mw, 16 * t + 4, 4);
            const float m1 = (float)__builtin_amdgcn_ubfe(mw, 16 * t + 12, 4);
            ac2[t] = make_float2(fmaf(dmin, m0, a128), fmaf(dmin, m1, a128));
          }
        }
        if constexpr (FMT == kQ3_K) {
          // steps 2g, 2g + 1: sub-blocks 4g .. 4g + 3; D_h = d (S_h - 32)
          const uint32_t dk =
              (uint32_t)__builtin_amdgcn_ds_bpermute(4 * hsrc, (int)(odd ? dg1[m][rt] : dg0[m][rt]));
          const float d = f16_lo(dk);
          const uint32_t sw = (g == 0 ? hk.x : g == 1 ? hk.y : g == 2 ? hk.z : hk.w) ^ 0x20202020u;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            // held in ints: converted as signed values
            const int s0 = __builtin_amdgcn_sbfe((int)sw, 16 * t, 6);
            const int s1 = __builtin_amdgcn_sbfe((int)sw, 16 * t + 8, 6);
            ac2[t] = make_float2(d * (float)s0, d * (float)s1);
          }
        }
        if constexpr (FMT == kQ6_K) {
          // steps 2g, 2g + 1: sub-blocks 4g .. 4g + 3; D_h = d sc_h (int8)
          const uint32_t dk =
              (uint32_t)__builtin_amdgcn_ds_bpermute(4 * hsrc, (int)(odd ? dg1[m][rt] : dg0[m][rt]));
          const float d = f16_lo(dk);
          const uint32_t sw = g == 0 ? hk.x : g == 1 ? hk.y : g == 2 ? hk.z : hk.w;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int s0 = __builtin_amdgcn_sbfe((int)sw, 16 * t, 8);
            const int s1 = __builtin_amdgcn_sbfe((int)sw, 16 * t + 8, 8);
            ac2[t] = make_float2(d * (float)s0, d * (float)s1);
          }
        }
#pragma unroll
        for (int t = 0; t < 2 && FMT != kQ2_K && !split_steps<FMT>(); ++t) {
          const int i = 2 * g + t;
          float2 ac;
          if constexpr (FMT == kQ4_K) {
            ac = q4k_scale(hk, i);
          } else {
            const uint4 h = hk;
            const uint64_t lo = (uint64_t)h.x | ((uint64_t)h.y << 32);
            const uint64_t hi = (uint64_t)h.z | ((uint64_t)h.w << 32);
            const uint32_t dw = (uint32_t)((g < 2 ? lo : hi) >> (32 * (g & 1)));  // halves 2g, 2g+1
            const bool live = kSlab * k + i < S;
            ac = make_float2(live ? f16_to_f32(t ? dw >> 16 : dw) : 0.f, 0.f);
          }
          ac2[t] = ac;
        }
        reinterpret_cast<float4*>(scl)[((m * RTR + rt) * 4 + g) * 16 + n] =
            make_float4(ac2[0].x, ac2[0].y, ac2[1].x, ac2[1].y);
      }
    __syncthreads();
    if (k + 1 < NS) {
      if ((k & 7) == 7) load_group((k + 1) >> 3);
      load_slab(sl, k + 1);
    }

    const uint32_t* wl32 = reinterpret_cast<const uint32_t*>(wl);
    // acc += a P - c X for one step's products (row scale pair ac = (a, c));
    // Q2_K: acc += a P - c0 X0 - c1 X1 with ac = (c0, c1) and a per slab.
    f32x4 pp[NM][RTR], pp1[NM][RTR], Xp, Xp1;
    float2 acp[NM][RTR];
    auto apply = [&](const f32x4 (&pv)[NM][RTR], const f32x4 (&pv1)[NM][RTR], const f32x4& Xv,
                     const f32x4& Xv1, const float2 (&acv)[NM][RTR]) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v;
            if constexpr (split_steps<FMT>()) {
              constexpr float kX = FMT == kQ3_K ? -132.0f : -160.0f;
              v = fmaf(acv[m][rt].x, fmaf(128.0f, pv[m][rt][j], kX * Xv[j]), acc[m][rt][j]);
              v = fmaf(acv[m][rt].y, fmaf(128.0f, pv1[m][rt][j], kX * Xv1[j]), v);
            } else if constexpr (FMT == kQ2_K) {
              v = fmaf(aq[m][rt], pv[m][rt][j], acc[m][rt][j]);
              v = fmaf(-acv[m][rt].x, Xv[j], v);
              v = fmaf(-acv[m][rt].y, Xv1[j], v);
            } else {
              v = fmaf(acv[m][rt].x, pv[m][rt][j], acc[m][rt][j]);
              if constexpr (FMT == kQ4_K) v = fmaf(-acv[m][rt].y, Xv[j], v);
            }
            acc[m][rt][j] = v;
          }
    };
    if constexpr (TT == 2) {
      // Q8_0, two token tiles: acc += d P per step, the scale FMAs one step
      // behind the products.
      f32x4 q[TT][NM][RTR], qp[TT][NM][RTR];
      auto apply2 = [&](const f32x4 (&pv)[TT][NM][RTR], const float2 (&acv)[NM][RTR]) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              acc[m][rt][j] = fmaf(acv[m][rt].x, pv[0][m][rt][j], acc[m][rt][j]);
              acc1[m][rt][j] = fmaf(acv[m][rt].x, pv[1][m][rt][j], acc1[m][rt][j]);
            }
      };
#pragma unroll
      for (int i = 0; i < kSlab; ++i) {
        u32x4 ahi[TT], alo[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const uint4 h4 = L.act[t][((i * 2 + 0) * 4 + g) * 16 + n];
          const uint4 l4 = L.act[t][((i * 2 + 1) * 4 + g) * 16 + n];
          ahi[t] = u32x4{h4.x, h4.y, h4.z, h4.w};
          alo[t] = u32x4{l4.x, l4.y, l4.z, l4.w};
        }
        u32x4 b[NM][RTR];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RTR; ++rt) {
            const int base = (m * RTR + rt) * NQ;
            const int u = 2 * i + (g >> 1);
            const uint2 w = reinterpret_cast<const uint2*>(wl)[((base + (i >> 1)) * 64 + (u & 3) * 16 + n) * 2 + (g & 1)];
            b[m][rt] = q8_operand(w.x, w.y);
          }
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt) q[t][m][rt] = mfma_bf16(ahi[t], b[m][rt], zero);
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt) q[t][m][rt] = mfma_bf16(alo[t], b[m][rt], q[t][m][rt]);
        if (i > 0) apply2(qp, acp);
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt) qp[t][m][rt] = q[t][m][rt];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RTR; ++rt)
            acp[m][rt] = scl[(((m * RTR + rt) * 4 + (i >> 1)) * 16 + n) * 2 + (i & 1)];
      }
      apply2(qp, acp);
      return;
    }
#pragma unroll
    for (int i = 0; i < kSlab; ++i) {
      const uint4 h4 = al[((i * 2 + 0) * 4 + g) * 16 + n];
      const uint4 l4 = al[((i * 2 + 1) * 4 + g) * 16 + n];
      const u32x4 ahi = {h4.x, h4.y, h4.z, h4.w};
      const u32x4 alo = {l4.x, l4.y, l4.z, l4.w};
      u32x4 b[NM][RTR];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt) {
          const int base = (m * RTR + rt) * NQ;
          if constexpr (FMT == kQ4_K) {
            b[m][rt] = q4k_operand(wl32[((base + (i >> 2)) * 64 + (i & 3) * 16 + n) * 4 + g], one);
          } else if constexpr (FMT == kQ2_K) {
            // Sub-block s = 2i + g/2 of the slab: its quant dword (bytes 4s of
            // the row's 64, held by loading lane s/4 of the row) and scale.
            const int s2 = 2 * i + (g >> 1);
            const uint32_t qd = wl32[(base * 64 + (s2 >> 2) * 16 + n) * 4 + (s2 & 3)];
            const uint32_t sw = (i >> 1) == 0 ? hks[m][rt].x : (i >> 1) == 1 ? hks[m][rt].y
                              : (i >> 1) == 2 ? hks[m][rt].z : hks[m][rt].w;
            b[m][rt] = q2k_operand(qd >> (4 * (g & 1)), __builtin_amdgcn_ubfe(sw, 8 * (s2 & 3), 4));
          } else if constexpr (FMT == kQ3_K) {
            // Low bits of sub-block s = 2i + g/2 (load 0, as Q2_K); high bits
            // of the sub-block pair i (bytes 4i of the row's 32: load 1, lane
            // i/4 of the row), sub-block s in nibble s % 2.
            const int s2 = 2 * i + (g >> 1);
            const uint32_t qd = wl32[(base * 64 + (s2 >> 2) * 16 + n) * 4 + (s2 & 3)];
            const uint32_t hw = wl32[((base + 1) * 64 + (i >> 2) * 16 + n) * 4 + (i & 3)];
            b[m][rt] = q3k_operand(qd >> (4 * (g & 1)), hw >> (4 * (g >> 1) + 2 * (g & 1)));
          } else if constexpr (FMT == kQ6_K) {
            // Low nibbles of group i as in Q4_K (loads 0, 1); its 8 high
            // bytes at 8 i of the row's 64 (load 2, lane i / 2), the lane's
            // columns in high dword g / 2 of the group, pair g % 2.
            const uint32_t lw = wl32[((base + (i >> 2)) * 64 + (i & 3) * 16 + n) * 4 + g];
            const uint32_t hw = wl32[((base + 2) * 64 + (i >> 1) * 16 + n) * 4 + 2 * (i & 1) + (g >> 1)];
            b[m][rt] = q6k_operand(lw, hw >> (4 * (g & 1)));
          } else {
            const int u = 2 * i + (g >> 1);
            const uint2 w = reinterpret_cast<const uint2*>(wl)[((base + (i >> 1)) * 64 + (u & 3) * 16 + n) * 2 + (g & 1)];
            b[m][rt] = q8_operand(w.x, w.y);
          }
        }
      // hi terms for every row tile first, then lo terms, so that no MFMA
      // waits on the one just issued.
      f32x4 p[NM][RTR], p1[NM][RTR], X = zero, X1 = zero;
      if constexpr (split_steps<FMT>()) {
        // the two 16-column halves of the step, each against its own
        // activations (the other half's lanes zeroed)
        const u32x4 ahi0 = g < 2 ? ahi : u32x4{0u, 0u, 0u, 0u}, ahi1 = g < 2 ? u32x4{0u, 0u, 0u, 0u} : ahi;
        const u32x4 alo0 = g < 2 ? alo : u32x4{0u, 0u, 0u, 0u}, alo1 = g < 2 ? u32x4{0u, 0u, 0u, 0u} : alo;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RTR; ++rt) {
            p[m][rt] = mfma_bf16(ahi0, b[m][rt], zero);
            p1[m][rt] = mfma_bf16(ahi1, b[m][rt], zero);
          }
        X = mfma_bf16(ahi0, ones, zero);
        X1 = mfma_bf16(ahi1, ones, zero);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RTR; ++rt) {
            p[m][rt] = mfma_bf16(alo0, b[m][rt], p[m][rt]);
            p1[m][rt] = mfma_bf16(alo1, b[m][rt], p1[m][rt]);
          }
        X = mfma_bf16(alo0, ones, X);
        X1 = mfma_bf16(alo1, ones, X1);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTR && !split_steps<FMT>(); ++rt) p[m][rt] = mfma_bf16(ahi, b[m][rt], zero);
      if constexpr (FMT == kQ4_K) X = mfma_bf16(ahi, ones, zero);
      if constexpr (FMT == kQ2_K) {
        X = mfma_bf16(ahi, ones0, zero);
        X1 = mfma_bf16(ahi, ones1, zero);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTR && !split_steps<FMT>(); ++rt) p[m][rt] = mfma_bf16(alo, b[m][rt], p[m][rt]);
      if constexpr (FMT == kQ4_K) X = mfma_bf16(alo, ones, X);
      if constexpr (FMT == kQ2_K) {
        X = mfma_bf16(alo, ones0, X);
        X1 = mfma_bf16(alo, ones1, X1);
      }
      // Scale the previous step's products while this step's MFMAs run.
      if (i > 0) apply(pp, pp1, Xp, Xp1, acp);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt) {
          pp[m][rt] = p[m][rt];
          pp1[m][rt] = p1[m][rt];
          acp[m][rt] = scl[(((m * RTR + rt) * 4 + (i >> 1)) * 16 + n) * 2 + (i & 1)];
        }
      Xp = X;
      Xp1 = X1;
    }
    apply(pp, pp1, Xp, Xp1, acp);
  };
  Slab<FMT, NM, RTR, TT> sl;
  load_group(0);
  load_slab(sl, 0);
  for (int k = 0; k < NS; ++k) consume(sl, k);

  // Epilogue: lane holds rows r0 + 16 rt + n for tokens 4g + j.
  auto store_tile = [&](const f32x4 (&av)[NM][RTR], int tpos0, int tcnt) {
#pragma unroll
    for (int rt = 0; rt < RTR; ++rt) {
      const int r = r0 + 16 * rt + n;
      if (r >= a.rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * g + j;
        if (t >= tcnt) continue;
        const int pos = tpos0 + t;
        const int orow = a.out_scatter ? a.slots[pos] : pos;
        if (GATEUP) {
          const float h = silu(av[0][rt][j]) * av[NM - 1][rt][j];
          uint32_t hi, lo;
          split_bf16(h, hi, lo);
          // Element r of the row: group r / 8, operand position of r % 8.
          const int q = r & 7;
          const int p = (q < 4) ? 2 * q : 2 * (q - 4) + 1;
          uint16_t* row = reinterpret_cast<uint16_t*>(a.out) + (int64_t)orow * a.rows * 2;
          row[(r >> 3) * 16 + p] = (uint16_t)hi;
          row[(r >> 3) * 16 + 8 + p] = (uint16_t)lo;
        } else {
          reinterpret_cast<float*>(a.out)[(int64_t)orow * a.rows + r] = av[0][rt][j];
        }
      }
    }
  };
  store_tile(acc, pos0, cnt);
  if (TT == 2 && cnt1 > 0) store_tile(acc1, pos1, cnt1);
}

// Grid: row_blocks x (capacity of work units rounded up to 8); a unit is
// one token tile, or TT consecutive tiles of the dense list.  Blocks go to
// the eight XCDs round-robin; XCD x takes the x-th eighth of the live unit
// list, in order: block b takes its ((b / 8) / row_blocks)-th unit and row
// block (b / 8) % row_blocks.  So the row blocks of one token tile share an
// XCD (and its L2 copy of the tile's activations), and the tiles of an
// expert with more than 16 tokens run back to back on one XCD and find its
// weight rows in that L2.  Every wave of a workgroup passes the same
// slab barriers; waves whose rows lie past the expert compute zeros.
// TT = 2 (dense Q8_0, the shared expert): each workgroup takes two token
// tiles, so every weight operand it builds serves 32 tokens.
template <int FMT, bool GATEUP, int RTR, int TT = 1>
__global__ __launch_bounds__(kBlock) void k_gemm(GemmArgs a) {
  __shared__ GemmLds<FMT, GATEUP, RTR> lds;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int n_tiles = a.tiles ? *a.n_tiles : (a.dense_tokens + 15) / 16;
  const int n_units = (n_tiles + TT - 1) / TT;
  const int per_xcd = (n_units + 7) / 8;
  const int slot = j / a.row_blocks, rb = j % a.row_blocks;
  const int unit = xcd * per_xcd + slot;
  if (slot >= per_xcd || unit >= n_units) return;
  const int tile = TT * unit;
  int e, pos0, cnt;
  if (a.tiles) {
    e = a.tiles[3 * tile];
    pos0 = a.tiles[3 * tile + 1];
    cnt = a.tiles[3 * tile + 2];
  } else {
    e = 0;
    pos0 = 16 * tile;
    cnt = min(16, a.dense_tokens - pos0);
    if (cnt <= 0) return;
  }
  if constexpr (TT == 2) {
    // the dense list only (the host launches TT = 2 for no other)
    const int pos1 = pos0 + 16, cnt1 = max(0, min(16, a.dense_tokens - pos1));
    gemm_block<FMT, GATEUP, RTR, 2>(a, e, pos0, cnt, rb * kWavesPerBlock * 16 * RTR, lds, pos1,
                                    cnt1);
  } else {
    gemm_block<FMT, GATEUP, RTR>(a, e, pos0, cnt, rb * kWavesPerBlock * 16 * RTR, lds);
  }
}

// ---------------------------------------------------------------------------
// Router logits for a batch: l[t][e] = sum_h Wr[e][h] x[t][h] on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32, lane 16 g + n: A row n column g, B
// column n row g, D rows 4g..4g+3 of column n).  A workgroup computes a
// 32-token x 32-expert tile as four 16 x 16 sub-tiles; its four waves take
// quarters of H, each wave all four sub-tiles, so that every operand load
// feeds two MFMAs (loads of 16 rows x 64 bytes are what bounds this kernel:
// the address path, not the matrix cores).  The waves' partial tiles are
// added in LDS in a fixed order.  Each sub-tile sums exactly as a
// workgroup of its own would.
// NG: groups of 16 columns per wave when known at compile time (H / 64),
// else 0; a known count lets the whole ring be unrolled.
template <int NG>
__global__ __launch_bounds__(kBlock) void k_router_mfma(const float* __restrict__ wr,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ logits, int H, int E,
                                                        int M) {
  __shared__ f32x4 s_part[kWavesPerBlock - 1][2][2][kWave];
  // The wave index is uniform; saying so keeps the loop bounds scalar.
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int t0 = 32 * blockIdx.x, e0 = 32 * blockIdx.y;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * (uint32_t)H * 4u);
  const __amdgpu_buffer_rsrc_t wrr = make_rsrc(wr, (uint32_t)E * (uint32_t)H * 4u);
  // Rows past M or E read as zero (offsets past the resources).
  uint32_t xo[2], wo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    xo[h] = (t0 + 16 * h + n < M) ? (uint32_t)(t0 + 16 * h + n) * H * 4u : 0xFFFFFFF0u;
    wo[h] = (e0 + 16 * h + n < E) ? (uint32_t)(e0 + 16 * h + n) * H * 4u : 0xFFFFFFF0u;
  }
  const int kq = H / kWavesPerBlock;  // H % 64 == 0: whole groups of 16 columns
  const int kb = wv * kq, ng = NG ? NG : kq / 16;  // this wave's first column and groups
  // Loads run kRing groups of 16 columns ahead of the MFMAs.  The loop is
  // branch-free over whole rounds of kRing groups, so the wait before each
  // group counts a fixed number of later loads: groups past the wave's last
  // read offsets beyond the buffers, i.e. zeros, and add exactly nothing.
  constexpr int kRing = 4;
  constexpr uint32_t kOut = 0xFFFFFFF0u;
  auto load = [&](int gi, f32x4 (&av)[2], f32x4 (&bv)[2]) {
    const bool live = gi < ng;
    const uint32_t ko = 4u * (uint32_t)(kb + 16 * gi + 4 * g);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      av[h] = __builtin_amdgcn_raw_buffer_load_b128(xr, live && xo[h] != kOut ? xo[h] + ko : kOut, 0, 0);
      bv[h] = __builtin_amdgcn_raw_buffer_load_b128(wrr, live && wo[h] != kOut ? wo[h] + ko : kOut, 0, 0);
    }
  };
  // Slot u holds group u mod kRing; each step first refills the slot the
  // previous step used, then multiplies the slot loaded kRing - 1 steps ago.
  f32x4 av[kRing][2], bv[kRing][2];
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) load(u, av[u], bv[u]);
  f32x4 acc[2][2];  // [token half][expert half]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[i][h] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < ng; r += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      constexpr int kLead = kRing - 1;
      load(r + u + kLead, av[(u + kLead) % kRing], bv[(u + kLead) % kRing]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[i][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][i][j], bv[u][h][j], acc[i][h], 0, 0, 0);
      // Keep each step's loads ahead of its products: scheduled together,
      // the loads of a whole round sink to its end and every round waits
      // for all of them.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) s_part[wv - 1][i][h][lane] = acc[i][h];
  }
  __syncthreads();
  if (wv > 0) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 a = acc[i][h];
#pragma unroll
      for (int w = 0; w < kWavesPerBlock - 1; ++w) a += s_part[w][i][h][lane];
      const int e = e0 + 16 * h + n;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 16 * i + 4 * g + j;
        if (t < M && e < E) logits[(int64_t)t * E + e] = a[j];
      }
    }
}

}  // namespace svr
