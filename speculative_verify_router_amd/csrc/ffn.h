// Fused dequantise-and-multiply skinny GEMM for the expert FFNs.
//
// Routed gate/up/down are Q4_K or Q8_0 and the shared expert Q8_0 ("Step
// 3.7 Flash Mixed-Quant GGUF", Tensor recipe; "Step-5 Preview GGUF",
// Precision distribution table).  At a verify batch of four tokens with 8
// of 288-352 experts each, an expert serves about one token, so this is an
// HBM-bound matrix-vector product: each selected expert's quant blocks are
// streamed exactly once, for all of that expert's tokens together.
//
// Mapping.  A 16-byte chunk of the quant plane is the unit of loading:
// 16 weights for Q8_0, one 32-weight sub-block for Q4_K.  A row of K
// columns has C = K/16 (Q8_0) or K/32 (Q4_K) chunks, covered by a group of
// `lpr` consecutive lanes (lpr | 64), lane j of the group taking chunks
// j, j+lpr, ..., j+(CPL-1)*lpr.  A wave therefore works on 64/lpr rows at
// once and every wave load instruction reads whole 128-byte lines.  Each
// lane keeps its K-slice of the activations in VGPRs for the whole pass, so
// activations are read from L2 once per wave, not once per row.
//
// Arithmetic (fp32 FMA throughout, no packed-fp32 forms):
//  * Q8_0: bytes are flipped to q+128 with one XOR per dword so that
//    v_cvt_f32_ubyte converts them; sum((q+128) x) - 128 sum(x) = sum(q x).
//  * Q4_K: a dword of quants masked with 0x0F0F0F0F gives the even weights
//    and with 0xF0F0F0F0 gives 16x the odd weights; the odd activations are
//    stored pre-scaled by 1/16 (exact), so one accumulator serves both.
//    w = d*sc*q - dmin*m folds to d*sc*sum(q x) - dmin*m*sum(x) per
//    sub-block, with sum(x) precomputed per lane.
#pragma once

#include "common.h"

namespace svr {

enum QFmt { kQ8_0 = 1, kQ4_K = 2 };

template <int FMT>
struct QTraits;
template <>
struct QTraits<kQ8_0> {
  static constexpr int kWpc = 16;  // weights per 16-byte chunk
};
template <>
struct QTraits<kQ4_K> {
  static constexpr int kWpc = 32;
};

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
  int units_per_block;      // output rows per workgroup (multiple of 4*64/lpr)
};

// Per-lane view of one 16-byte chunk of a row: its quants and its scale data.
template <int FMT>
struct Chunk;
template <>
struct Chunk<kQ8_0> {
  uint4 q;
  uint32_t d;  // fp16 bits
};
template <>
struct Chunk<kQ4_K> {
  uint4 q;
  uint4 h;  // super-block header
};

template <int FMT>
__device__ __forceinline__ void load_chunk(Chunk<FMT>& ch, const uint8_t* base, int64_t total_rows,
                                           int K, int64_t row, int c);

template <>
__device__ __forceinline__ void load_chunk<kQ8_0>(Chunk<kQ8_0>& ch, const uint8_t* base,
                                                  int64_t total_rows, int K, int64_t row, int c) {
  const int64_t nb = K >> 5;
  const int64_t qoff = ((2 * total_rows * nb) + 255) & ~(int64_t)255;
  ch.q = ld16(base + qoff + row * K + 16 * c);
  ch.d = *reinterpret_cast<const uint16_t*>(base + 2 * (row * nb + (c >> 1)));
}

template <>
__device__ __forceinline__ void load_chunk<kQ4_K>(Chunk<kQ4_K>& ch, const uint8_t* base,
                                                  int64_t total_rows, int K, int64_t row, int c) {
  const int64_t ns = K >> 8;
  const int64_t hb = 16 * total_rows * ns;
  ch.q = ld16(base + hb + row * (K >> 1) + 16 * c);
  ch.h = ld16(base + 16 * (row * ns + (c >> 3)));
}

// Activation slice of one token for one chunk position.
template <int FMT>
struct XSlice {
  float v[QTraits<FMT>::kWpc];
  float sum;  // Q8_0: 128 * sum(x); Q4_K: sum(x)
};

template <int FMT>
__device__ __forceinline__ void load_x(XSlice<FMT>& xs, const float* row, int c) {
  constexpr int W = QTraits<FMT>::kWpc;
  const float* p = row + W * c;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < W / 4; ++i) {
    const float4 a = ldf4(p + 4 * i);
    s += (a.x + a.y) + (a.z + a.w);
    if (FMT == kQ4_K) {
      xs.v[4 * i + 0] = a.x;
      xs.v[4 * i + 1] = a.y * 0.0625f;
      xs.v[4 * i + 2] = a.z;
      xs.v[4 * i + 3] = a.w * 0.0625f;
    } else {
      xs.v[4 * i + 0] = a.x;
      xs.v[4 * i + 1] = a.y;
      xs.v[4 * i + 2] = a.z;
      xs.v[4 * i + 3] = a.w;
    }
  }
  xs.sum = (FMT == kQ8_0) ? 128.f * s : s;
}

template <int FMT>
__device__ __forceinline__ void zero_x(XSlice<FMT>& xs) {
#pragma unroll
  for (int i = 0; i < QTraits<FMT>::kWpc; ++i) xs.v[i] = 0.f;
  xs.sum = 0.f;
}

// Scale data of a chunk, decoded once and applied to every token.
struct ChunkScale {
  float a;  // multiplies sum(q x)
  float b;  // multiplies the precomputed activation sum (subtracted)
};

__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ8_0>& ch, int /*sub*/) {
  const float d = f16_to_f32(ch.d);
  return {d, d};
}

__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ4_K>& ch, int sub) {
  const float d = f16_to_f32(ch.h.x);
  const float dmin = f16_to_f32(ch.h.x >> 16);
  const uint64_t lo = (uint64_t)ch.h.y | ((uint64_t)ch.h.z << 32);  // stream bits 0..63
  const uint64_t hi = (uint64_t)ch.h.z | ((uint64_t)ch.h.w << 32);  // stream bits 32..95
  const uint32_t sc = (uint32_t)(lo >> (6 * sub)) & 63u;
  const uint32_t m = (uint32_t)(hi >> (16 + 6 * sub)) & 63u;
  return {d * (float)sc, dmin * (float)m};
}

// sum over the chunk of q'_i * x_i, with q' as described above.
__device__ __forceinline__ float chunk_dot(const Chunk<kQ8_0>& ch, const XSlice<kQ8_0>& xs) {
  const uint32_t w[4] = {ch.q.x ^ 0x80808080u, ch.q.y ^ 0x80808080u, ch.q.z ^ 0x80808080u,
                         ch.q.w ^ 0x80808080u};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s0 = fmaf(ubyte_f<0>(w[k]), xs.v[4 * k + 0], s0);
    s1 = fmaf(ubyte_f<1>(w[k]), xs.v[4 * k + 1], s1);
    s0 = fmaf(ubyte_f<2>(w[k]), xs.v[4 * k + 2], s0);
    s1 = fmaf(ubyte_f<3>(w[k]), xs.v[4 * k + 3], s1);
  }
  return s0 + s1;
}

__device__ __forceinline__ float chunk_dot(const Chunk<kQ4_K>& ch, const XSlice<kQ4_K>& xs) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = w[k] & 0x0F0F0F0Fu;
    const uint32_t hi = w[k] & 0xF0F0F0F0u;
    s0 = fmaf(ubyte_f<0>(lo), xs.v[8 * k + 0], s0);
    s1 = fmaf(ubyte_f<0>(hi), xs.v[8 * k + 1], s1);
    s0 = fmaf(ubyte_f<1>(lo), xs.v[8 * k + 2], s0);
    s1 = fmaf(ubyte_f<1>(hi), xs.v[8 * k + 3], s1);
    s0 = fmaf(ubyte_f<2>(lo), xs.v[8 * k + 4], s0);
    s1 = fmaf(ubyte_f<2>(hi), xs.v[8 * k + 5], s1);
    s0 = fmaf(ubyte_f<3>(lo), xs.v[8 * k + 6], s0);
    s1 = fmaf(ubyte_f<3>(hi), xs.v[8 * k + 7], s1);
  }
  return s0 + s1;
}

// One pass over the workgroup's rows for NT tokens (NT <= TP).
template <int FMT, int CPL, int NT, bool GATEUP>
__device__ __forceinline__ void ffn_pass(const FfnArgs& a, int expert, const int* pair_ids,
                                         int ub, int ue) {
  constexpr int UNR = (CPL <= 4) ? 2 : 1;  // rows in flight per wave step
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int lpr = a.lpr;
  const int G = kWave / lpr;
  const int g = lane / lpr;
  const int j = lane - g * lpr;

  // Activation slices of the NT tokens.
  XSlice<FMT> xs[NT][CPL];
  int out_row[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int p = pair_ids[t];
    const int arow = a.act_by_pair ? p : p / a.top_k;
    out_row[t] = p;
    const float* xr = a.act + (int64_t)arow * a.K;
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) load_x<FMT>(xs[t][ci], xr, j + lpr * ci);
  }

  const int64_t rbase = (int64_t)expert * a.rows_per_expert;
  const int stride = 4 * G;  // rows covered by the workgroup per step
  // The loop bound is wave-uniform (base), so every lane takes part in the
  // group reductions; lanes whose row lies past `ue` load a valid row and
  // skip the store.
  for (int base = ub + wv * G; base < ue; base += stride * UNR) {
    Chunk<FMT> c0[UNR][CPL];
    Chunk<FMT> c1[UNR][GATEUP ? CPL : 1];
    int urow[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int u = base + g + r * stride;
      urow[r] = u;
      const int ul = min(u, ue - 1);  // keep loads in bounds for idle lanes
      const int64_t row = rbase + ul;
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) {
        load_chunk<FMT>(c0[r][ci], a.w0, a.total_rows, a.K, row, j + lpr * ci);
        if (GATEUP) load_chunk<FMT>(c1[r][ci], a.w1, a.total_rows, a.K, row, j + lpr * ci);
      }
    }
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      float acc0[NT], acc1[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc0[t] = acc1[t] = 0.f;
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) {
        const int s = (j + lpr * ci) & 7;  // Q4_K sub-block of this chunk
        const ChunkScale k0 = decode_scale(c0[r][ci], s);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float dsum = chunk_dot(c0[r][ci], xs[t][ci]);
          acc0[t] = fmaf(k0.a, dsum, fmaf(-k0.b, xs[t][ci].sum, acc0[t]));
        }
        if (GATEUP) {
          const ChunkScale k1 = decode_scale(c1[r][ci], s);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float dsum = chunk_dot(c1[r][ci], xs[t][ci]);
            acc1[t] = fmaf(k1.a, dsum, fmaf(-k1.b, xs[t][ci].sum, acc1[t]));
          }
        }
      }
      const bool ok = urow[r] < ue;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float v0 = group_sum(acc0[t], lpr);
        if (GATEUP) {
          const float v1 = group_sum(acc1[t], lpr);
          if (ok && j == 0)
            a.out[(int64_t)out_row[t] * a.rows_per_expert + urow[r]] = silu(v0) * v1;
        } else {
          if (ok && j == 0) a.out[(int64_t)out_row[t] * a.rows_per_expert + urow[r]] = v0;
        }
      }
    }
  }
}

// Grid: (row tiles, expert slots).  A workgroup serves rows
// [blockIdx.x * units_per_block, ...) of the expert in slot blockIdx.y for
// every token routed to it, TP tokens per pass.
template <int FMT, int CPL, int TP, bool GATEUP>
__global__ __launch_bounds__(kBlock) void k_ffn(FfnArgs a) {
  const int slot = blockIdx.y;
  if (a.n_active && slot >= *a.n_active) return;
  const int expert = a.active ? a.active[slot] : 0;
  const int begin = a.offsets ? a.offsets[expert] : 0;
  const int count = a.offsets ? a.offsets[expert + 1] - begin : a.n_tokens;
  const int ub = blockIdx.x * a.units_per_block;
  const int ue = min(ub + a.units_per_block, a.rows_per_expert);
  if (ub >= ue) return;
  for (int p0 = 0; p0 < count; p0 += TP) {
    int ids[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const int q = min(p0 + t, count - 1);
      ids[t] = a.slots ? a.slots[begin + q] : q;
    }
    const int nt = min(TP, count - p0);
    if (nt >= TP) {
      ffn_pass<FMT, CPL, TP, GATEUP>(a, expert, ids, ub, ue);
    } else if (TP > 1 && nt == 1) {
      ffn_pass<FMT, CPL, 1, GATEUP>(a, expert, ids, ub, ue);
    } else if (TP > 2 && nt == 2) {
      ffn_pass<FMT, CPL, (TP > 2 ? 2 : 1), GATEUP>(a, expert, ids, ub, ue);
    } else if (TP > 3 && nt == 3) {
      ffn_pass<FMT, CPL, (TP > 3 ? 3 : 1), GATEUP>(a, expert, ids, ub, ue);
    }
  }
}

}  // namespace svr
