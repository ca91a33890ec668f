// Planar Q8_0 / Q4_K blocks: 16-byte chunk loads, scale decoding and the
// fused dequantise-and-dot of one chunk against fp32 activations.
//
// Formats (include/moe_layer.h): Q8_0 blocks of 32 int8 with an fp16 scale
// d, w = d*q; Q4_K super-blocks of 256 with fp16 d, dmin and per-32 6-bit
// sc, m, 4-bit q, w = d*sc*q - dmin*m ("Step-5 Preview GGUF" and "Step 3.7
// Flash Mixed-Quant GGUF" name these tensor types; their bit layouts are
// this library's).
//
// Dot product.  A quant nibble or biased byte placed in the low bits of an
// fp16 half is the subnormal q * 2^-24 exactly, so one AND turns two
// weights into two fp16 operands, and v_fma_mix_f32 multiplies each by an
// fp32 activation and accumulates in fp32.  The 2^24 goes into the scale.
//  * Q4_K dword (8 nibbles, weights 2b / 2b+1 in the low / high nibble of
//    byte b): mask 0x000F000F -> (w0, w4), 0x00F000F0 -> 16*(w1, w5), and
//    the same after >> 8 -> (w2, w6), 16*(w3, w7).  Odd activations are held
//    pre-scaled by 1/16 (exact).
//  * Q8_0 dword: XOR 0x80808080 biases int8 to q+128 in 0..255; mask
//    0x00FF00FF -> (b0, b2), after >> 8 -> (b1, b3).  sum((q+128) x) minus
//    128 sum(x) recovers sum(q x).
#pragma once

#include "common.h"

namespace svr {

enum QFmt { kQ8_0 = 1, kQ4_K = 2 };

template <int FMT>
struct QTraits;
template <>
struct QTraits<kQ8_0> {
  static constexpr int kWpc = 16;  // weights per 16-byte quant chunk
};
template <>
struct QTraits<kQ4_K> {
  static constexpr int kWpc = 32;
};

// The two planes of one expert's rows of a stacked planar tensor, as buffer
// resources (32-bit offsets; reads past the expert's rows return zero).
// Both formats carry K/16 bytes of scale data per row: Q8_0 K/32 fp16
// scales, Q4_K K/256 headers of 16 bytes.
struct QPlanes {
  __amdgpu_buffer_rsrc_t q, s;
  uint32_t qrow, srow;  // bytes per row in each plane
};

template <int FMT>
__device__ __forceinline__ QPlanes expert_planes(const uint8_t* base, int64_t total_rows, int K,
                                                 int64_t row0, int rows) {
  QPlanes p;
  p.srow = (uint32_t)(K >> 4);
  p.qrow = (FMT == kQ8_0) ? (uint32_t)K : (uint32_t)(K >> 1);
  const int64_t sbytes = total_rows * (int64_t)p.srow;
  const int64_t qstart = (FMT == kQ8_0) ? ((sbytes + 255) & ~(int64_t)255) : sbytes;
  p.s = make_rsrc(base + row0 * p.srow, (uint32_t)rows * p.srow);
  p.q = make_rsrc(base + qstart + row0 * p.qrow, (uint32_t)rows * p.qrow);
  return p;
}

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
  uint4 h;  // super-block header: d | dmin << 16, then the 96-bit sc/m stream
};

// Chunk c of a row whose plane offsets are qo = row * qrow and so = row * srow.
__device__ __forceinline__ void load_chunk(Chunk<kQ8_0>& ch, const QPlanes& p, uint32_t qo,
                                           uint32_t so, int c) {
  ch.q = bload16(p.q, qo + 16u * c);
  ch.d = bload2(p.s, so + 2u * (c >> 1));
}
__device__ __forceinline__ void load_chunk(Chunk<kQ4_K>& ch, const QPlanes& p, uint32_t qo,
                                           uint32_t so, int c) {
  ch.q = bload16(p.q, qo + 16u * c);
  ch.h = bload16(p.s, so + 16u * (c >> 3));
}

// Activations of one chunk position for one token.
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
    const float odd = (FMT == kQ4_K) ? 0.0625f : 1.0f;
    xs.v[4 * i + 0] = a.x;
    xs.v[4 * i + 1] = a.y * odd;
    xs.v[4 * i + 2] = a.z;
    xs.v[4 * i + 3] = a.w * odd;
  }
  xs.sum = (FMT == kQ8_0) ? 128.f * s : s;
}

// load_x for activations another workgroup of this launch wrote with
// store_shared: 16-byte loads past the per-XCD L2.  `base` is the start of
// the activation buffer, `row_off` the row's first element.
template <int FMT>
__device__ __forceinline__ void load_x_shared(XSlice<FMT>& xs, const float* base, int row_off,
                                              int c) {
  constexpr int W = QTraits<FMT>::kWpc;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, 0x7FFFFFF0u);
  const uint32_t off = 4u * (uint32_t)(row_off + W * c);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < W / 4; ++i) {
    const f32x4 a = bload16_shared(r, off + 16u * i);
    s += (a.x + a.y) + (a.z + a.w);
    const float odd = (FMT == kQ4_K) ? 0.0625f : 1.0f;
    xs.v[4 * i + 0] = a.x;
    xs.v[4 * i + 1] = a.y * odd;
    xs.v[4 * i + 2] = a.z;
    xs.v[4 * i + 3] = a.w * odd;
  }
  xs.sum = (FMT == kQ8_0) ? 128.f * s : s;
}

template <int FMT>
__device__ __forceinline__ void zero_x(XSlice<FMT>& xs) {
#pragma unroll
  for (int i = 0; i < QTraits<FMT>::kWpc; ++i) xs.v[i] = 0.f;
  xs.sum = 0.f;
}

// acc += a * dot - b * xs.sum for one chunk: the chunk's contribution.
struct ChunkScale {
  float a, b;
};

__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ8_0>& ch, int /*sub*/) {
  const float d = f16_to_f32(ch.d);
  return {d * 16777216.0f, d};
}

__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ4_K>& ch, int sub) {
  const float d = f16_lo(ch.h.x);
  const float dmin = f16_hi(ch.h.x);
  const uint64_t lo = (uint64_t)ch.h.y | ((uint64_t)ch.h.z << 32);  // stream bits 0..63
  const uint64_t hi = (uint64_t)ch.h.z | ((uint64_t)ch.h.w << 32);  // stream bits 32..95
  const uint32_t sc = (uint32_t)(lo >> (6 * sub)) & 63u;
  const uint32_t m = (uint32_t)(hi >> (16 + 6 * sub)) & 63u;
  return {d * 16777216.0f * (float)sc, dmin * (float)m};
}

// sum_i q'_i * 2^-24 * x_i over the chunk.
__device__ __forceinline__ float chunk_dot(const Chunk<kQ8_0>& ch, const XSlice<kQ8_0>& xs) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = w[k] ^ 0x80808080u;
    const uint32_t m0 = u & 0x00FF00FFu;
    const uint32_t m1 = (u >> 8) & 0x00FF00FFu;
    s0 = fmaf(f16_lo(m0), xs.v[4 * k + 0], s0);
    s1 = fmaf(f16_hi(m0), xs.v[4 * k + 2], s1);
    s0 = fmaf(f16_lo(m1), xs.v[4 * k + 1], s0);
    s1 = fmaf(f16_hi(m1), xs.v[4 * k + 3], s1);
  }
  return s0 + s1;
}

__device__ __forceinline__ float chunk_dot(const Chunk<kQ4_K>& ch, const XSlice<kQ4_K>& xs) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t m0 = w[k] & 0x000F000Fu;
    const uint32_t m1 = w[k] & 0x00F000F0u;
    const uint32_t sh = w[k] >> 8;
    const uint32_t m2 = sh & 0x000F000Fu;
    const uint32_t m3 = sh & 0x00F000F0u;
    s0 = fmaf(f16_lo(m0), xs.v[8 * k + 0], s0);
    s1 = fmaf(f16_hi(m0), xs.v[8 * k + 4], s1);
    s0 = fmaf(f16_lo(m1), xs.v[8 * k + 1], s0);
    s1 = fmaf(f16_hi(m1), xs.v[8 * k + 5], s1);
    s0 = fmaf(f16_lo(m2), xs.v[8 * k + 2], s0);
    s1 = fmaf(f16_hi(m2), xs.v[8 * k + 6], s1);
    s0 = fmaf(f16_lo(m3), xs.v[8 * k + 3], s0);
    s1 = fmaf(f16_hi(m3), xs.v[8 * k + 7], s1);
  }
  return s0 + s1;
}

}  // namespace svr
