// Planar Q8_0 / Q4_K / Q2_K / Q3_K / Q6_K blocks: 16-byte chunk loads, scale
// decoding and the fused dequantise-and-dot of one chunk against 16-bit
// activations.
//
// Formats (include/moe_layer.h): Q8_0 blocks of 32 int8 with an fp16 scale
// d, w = d*q; Q4_K super-blocks of 256 with fp16 d, dmin and per-32 6-bit
// sc, m, 4-bit q, w = d*sc*q - dmin*m; Q2_K super-blocks of 256 with fp16
// d, dmin and per-16 4-bit sc, m, 2-bit q, the same rule; Q3_K
// super-blocks of 256 with fp16 d and per-16 6-bit S, 3-bit Q,
// w = d*(S-32)*(Q-4); Q6_K super-blocks of 256 with fp16 d and per-16 int8
// sc, 6-bit Q, w = d*sc*(Q-32) ("Step-5 Preview GGUF" and "Step 3.7 Flash
// Mixed-Quant GGUF" name these tensor types; their bit layouts are this
// library's).
//
// Dot product.  The weights' integer quants go into v_dot4_i32_i8 as they
// are: a Q8_0 quant dword is four int8 weights; a Q4_K dword (8 nibbles,
// weights 2b / 2b+1 in the low / high nibble of byte b) gives the even
// weights with one AND and the odd ones with a shift and an AND; a Q2_K
// dword is one 16-weight sub-block whose four 2-bit planes (weights
// 4j..4j+3 in bits 2j of each byte) come out with a shift and an AND each,
// and Q3_K adds each plane's high bits with one more shift and an AND-OR;
// Q6_K's low nibbles come out as Q4_K's and take their two high bits the
// same way.
// The activations enter as 16-bit integers in two int8 limbs (XSlice below),
// so each chunk's dot product is exact in int32 and the block scales are
// applied once per chunk in fp32.
#pragma once

#include "common.h"

namespace svr {

enum QFmt { kQ8_0 = 1, kQ4_K = 2, kQ2_K = 3, kQ3_K = 4, kQ6_K = 5 };

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
template <>
struct QTraits<kQ2_K> {
  static constexpr int kWpc = 64;  // four 16-weight sub-blocks
};
template <>
struct QTraits<kQ3_K> {
  static constexpr int kWpc = 64;
};
template <>
struct QTraits<kQ6_K> {
  static constexpr int kWpc = 32;  // two 16-weight sub-blocks of low nibbles
};

// The planes of one expert's rows of a stacked planar tensor, as buffer
// resources (32-bit offsets; reads past the expert's rows return zero).
// Every format carries K/16 bytes of scale data per row in plane s: Q8_0
// K/32 fp16 scales, Q4_K K/256 headers of 16 bytes, Q2_K K/256 records of
// 16 scale bytes.  Q2_K keeps d and dmin in a third plane d of K/64 bytes
// per row, so a row's offset there is its plane-s offset / 4.  Q3_K keeps
// fp16 d in plane d (K/128 bytes per row: offset / 8), its low quant bits
// in plane q and its high bits in plane h (K/8 bytes per row: offset * 2).
// Q6_K: the same four planes with K/2 bytes of low nibbles per row in plane
// q and K/4 bytes of high bit pairs in plane h (offset * 4).
struct QPlanes {
  __amdgpu_buffer_rsrc_t q, s, d, h;
  uint32_t qrow, srow;  // bytes per row in planes q and s
};

__device__ __forceinline__ int64_t round256(int64_t v) { return (v + 255) & ~(int64_t)255; }

template <int FMT>
__device__ __forceinline__ QPlanes expert_planes(const uint8_t* base, int64_t total_rows, int K,
                                                 int64_t row0, int rows) {
  QPlanes p;
  p.srow = (uint32_t)(K >> 4);
  p.qrow = (FMT == kQ8_0)                    ? (uint32_t)K
           : (FMT == kQ4_K || FMT == kQ6_K) ? (uint32_t)(K >> 1)
                                            : (uint32_t)(K >> 2);
  const int64_t sbytes = total_rows * (int64_t)p.srow;
  if constexpr (FMT == kQ3_K || FMT == kQ6_K) {
    const uint32_t drow = (uint32_t)(K >> 7), hrow = (uint32_t)(FMT == kQ3_K ? K >> 3 : K >> 2);
    const int64_t sstart = round256(total_rows * (int64_t)drow);
    const int64_t qstart = round256(sstart + sbytes);
    const int64_t hstart = round256(qstart + total_rows * (int64_t)p.qrow);
    p.d = make_rsrc(base + row0 * drow, (uint32_t)rows * drow);
    p.s = make_rsrc(base + sstart + row0 * p.srow, (uint32_t)rows * p.srow);
    p.q = make_rsrc(base + qstart + row0 * p.qrow, (uint32_t)rows * p.qrow);
    p.h = make_rsrc(base + hstart + row0 * hrow, (uint32_t)rows * hrow);
  } else if constexpr (FMT == kQ2_K) {
    const uint32_t drow = (uint32_t)(K >> 6);
    const int64_t sstart = round256(total_rows * (int64_t)drow);
    const int64_t qstart = round256(sstart + sbytes);
    p.d = make_rsrc(base + row0 * drow, (uint32_t)rows * drow);
    p.s = make_rsrc(base + sstart + row0 * p.srow, (uint32_t)rows * p.srow);
    p.q = make_rsrc(base + qstart + row0 * p.qrow, (uint32_t)rows * p.qrow);
    p.h = p.s;
  } else {
    const int64_t qstart = (FMT == kQ8_0) ? round256(sbytes) : sbytes;
    p.s = make_rsrc(base + row0 * p.srow, (uint32_t)rows * p.srow);
    p.q = make_rsrc(base + qstart + row0 * p.qrow, (uint32_t)rows * p.qrow);
    p.d = p.h = p.s;
  }
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
template <>
struct Chunk<kQ2_K> {
  uint4 q;       // dword k: sub-block 4 (c % 4) + k of the super-block
  uint32_t sc;   // byte k: that sub-block's sc | m << 4
  uint32_t dd;   // d | dmin << 16
};
template <>
struct Chunk<kQ3_K> {
  uint4 q;       // low two bits; dword k: sub-block 4 (c % 4) + k
  uint2 hb;      // high bits; dword t: sub-blocks 2t (low nibbles), 2t + 1
  uint32_t sc;   // byte k: S of sub-block k
  uint32_t d;    // fp16 d (low half)
};
template <>
struct Chunk<kQ6_K> {
  uint4 q;       // low nibbles of the 32-weight group c (as a Q4_K chunk)
  uint2 hb;      // high bit pairs; dword t: group dwords 2t, 2t + 1
  uint32_t sc;   // bytes 0, 1: int8 scales of sub-blocks 2c, 2c + 1
  uint32_t d;    // fp16 d (low half)
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
__device__ __forceinline__ void load_chunk(Chunk<kQ2_K>& ch, const QPlanes& p, uint32_t qo,
                                           uint32_t so, int c) {
  ch.q = bload16(p.q, qo + 16u * c);
  ch.sc = bload4(p.s, so + 4u * c);
  ch.dd = bload4(p.d, (so >> 2) + 4u * (c >> 2));
}
__device__ __forceinline__ void load_chunk(Chunk<kQ3_K>& ch, const QPlanes& p, uint32_t qo,
                                           uint32_t so, int c) {
  ch.q = bload16(p.q, qo + 16u * c);
  ch.hb = bload8(p.h, 2u * so + 8u * c);
  ch.sc = bload4(p.s, so + 4u * c);
  ch.d = bload2(p.d, (so >> 3) + 2u * (c >> 2));
}
__device__ __forceinline__ void load_chunk(Chunk<kQ6_K>& ch, const QPlanes& p, uint32_t qo,
                                           uint32_t so, int c) {
  ch.q = bload16(p.q, qo + 16u * c);
  ch.hb = bload8(p.h, 4u * so + 8u * c);
  ch.sc = bload2(p.s, so + 2u * c);
  ch.d = bload2(p.d, (so >> 3) + 2u * (c >> 3));
}

// Activations of one chunk position for one token, as 16-bit integers.
//
// A lane quantises each of its chunk slices of activations when it loads
// them: q_i = rint(x_i / s) with s = max|x| / 32639 over the slice (64
// values for Q2_K, 32 for Q4_K, 16 for Q8_0), split q = 256 hi + lo with hi, lo in
// int8, and packed in the byte order of the chunk's quant dwords.  Then
// v_dot4_i32_i8 multiplies four weights by four limbs and accumulates
// exactly in int32, and sum_i w_i x_i = (dot_hi * 256 + dot_lo) * s * scale.
// The rounding to 16 bits relative to the slice maximum is the only
// approximation (relative error at most 2^-16 of the slice maximum per
// value).  The rounding uses the float trick: x / s + (1.5 * 2^23 + 128)
// rounds x / s to the nearest integer in the low mantissa bits, whose
// byte 1 is then hi and byte 0 xor 0x80 is lo.
template <int FMT>
struct XSlice;
template <>
struct XSlice<kQ4_K> {
  // h[2k] / l[2k]: limbs of weights 8k, 8k+2, 8k+4, 8k+6 (the low nibbles of
  // quant dword k); h[2k+1] / l[2k+1]: weights 8k+1, 8k+3, 8k+5, 8k+7.
  uint32_t h[8], l[8];
  float s;    // the slice's scale
  float sum;  // sum of the quantised activations, for the min term
};
template <>
struct XSlice<kQ8_0> {
  uint32_t h[4], l[4];  // dword k: limbs of weights 4k..4k+3 (byte order)
  float s;
  float sum;  // unused
};
template <>
struct XSlice<kQ2_K> {
  uint32_t h[16], l[16];  // dword 4k + j: limbs of weights 16k + 4j .. 16k + 4j + 3
  float s;
  float sum[4];  // s * (sum of the quantised activations) of sub-block k
};
template <>
struct XSlice<kQ3_K> {
  uint32_t h[16], l[16];  // as for Q2_K
  float s;
  int nsum4[4];  // -4 * (sum of the quantised activations) of sub-block k
};
template <>
struct XSlice<kQ6_K> {
  uint32_t h[8], l[8];  // as for Q4_K (even / odd weights of each dword)
  float s;
  int nsum32[2];  // -32 * (sum of the quantised activations) of sub-block k
};

constexpr float kQ16Max = 32639.0f;     // |q| bound: hi = (q + 128) >> 8 stays in int8
constexpr float kQ16Magic = 12583040.0f;  // 1.5 * 2^23 + 128
constexpr uint32_t kQ16MagicBits = 0x4B400080u;

// Limbs of four rounded values (bits of x / s + kQ16Magic): hi = byte 1,
// lo = byte 0 xor 0x80, packed in the order a, b, c, d.
__device__ __forceinline__ void limbs4(float a, float b, float c, float d, uint32_t& hi,
                                       uint32_t& lo) {
  const uint32_t ab = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b),
                                            __builtin_bit_cast(uint32_t, a), 0x05010400u);
  const uint32_t cd = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, d),
                                            __builtin_bit_cast(uint32_t, c), 0x05010400u);
  lo = __builtin_amdgcn_perm(cd, ab, 0x05040100u) ^ 0x80808080u;
  hi = __builtin_amdgcn_perm(cd, ab, 0x07060302u);
}

// Quantise N values (N = 64 for Q2_K, 32 for Q4_K, 16 for Q8_0) in slice
// order.
template <int FMT, int N>
__device__ __forceinline__ void quantize_slice(XSlice<FMT>& xs, const float (&v)[N]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float inv = amax > 0.f ? kQ16Max * __builtin_amdgcn_rcpf(amax) : 0.f;
  xs.s = amax > 0.f ? __builtin_amdgcn_rcpf(inv) : 0.f;
  float y[N];
  uint32_t bsum = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    y[i] = fmaf(v[i], inv, kQ16Magic);
    bsum += __builtin_bit_cast(uint32_t, y[i]);
  }
  if constexpr (FMT == kQ4_K || FMT == kQ6_K) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float* g = y + 8 * k;
      limbs4(g[0], g[2], g[4], g[6], xs.h[2 * k], xs.l[2 * k]);
      limbs4(g[1], g[3], g[5], g[7], xs.h[2 * k + 1], xs.l[2 * k + 1]);
    }
    if constexpr (FMT == kQ4_K) {
      xs.sum = xs.s * (float)(int32_t)(bsum - (uint32_t)N * kQ16MagicBits);
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint32_t b = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) b += __builtin_bit_cast(uint32_t, y[16 * k + i]);
        xs.nsum32[k] = -32 * (int32_t)(b - 16u * kQ16MagicBits);
      }
    }
  } else if constexpr (FMT == kQ2_K) {
#pragma unroll
    for (int k = 0; k < 16; ++k) limbs4(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3], xs.h[k], xs.l[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) b += __builtin_bit_cast(uint32_t, y[16 * k + i]);
      xs.sum[k] = xs.s * (float)(int32_t)(b - 16u * kQ16MagicBits);
    }
    (void)bsum;
  } else if constexpr (FMT == kQ3_K) {
#pragma unroll
    for (int k = 0; k < 16; ++k) limbs4(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3], xs.h[k], xs.l[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) b += __builtin_bit_cast(uint32_t, y[16 * k + i]);
      xs.nsum4[k] = -4 * (int32_t)(b - 16u * kQ16MagicBits);
    }
    (void)bsum;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) limbs4(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3], xs.h[k], xs.l[k]);
    xs.sum = 0.f;
  }
}

// Every activation slice of a pass at once: slice (t, ci) is chunk
// j + lpr * ci of activation row xrow[t] (K values per row).  All loads are
// issued before the first slice is quantised, so the pass waits for one
// memory round trip, not one per slice.  A chunk at or past `nchunks` reads
// at an offset beyond the buffer resource, which returns zeros, and an
// all-zero slice quantises to zero limbs, scale and sums.  XCOH: the
// activations were written earlier in this launch by other workgroups (with
// write-through stores), so the loads read past the per-XCD L2.
template <int FMT, int NT, int CPL, bool XCOH = false>
__device__ __forceinline__ void load_slices(XSlice<FMT> (&xs)[NT][CPL], const float* act,
                                            const int (&xrow)[NT], int K, int j, int lpr,
                                            int nchunks) {
  constexpr int W = QTraits<FMT>::kWpc;
  constexpr uint32_t kOutside = 0x7FFFFFF0u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(act, kOutside);
  f32x4 v[NT][CPL][W / 4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
      const int c = j + lpr * ci;
      const uint32_t off = c < nchunks ? 4u * (uint32_t)(xrow[t] * K + W * c) : kOutside;
#pragma unroll
      for (int i = 0; i < W / 4; ++i)
        v[t][ci][i] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * i, 0,
                                                            XCOH ? kCpolSc1 : 0);
    }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
      float f[W];
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        f[4 * i + 0] = v[t][ci][i].x;
        f[4 * i + 1] = v[t][ci][i].y;
        f[4 * i + 2] = v[t][ci][i].z;
        f[4 * i + 3] = v[t][ci][i].w;
      }
      quantize_slice<FMT, W>(xs[t][ci], f);
    }
}

// The same slices for a wave of 64 / LPR lane groups, which all need the
// same LPR * CPL chunk slices (lane j of every group: chunks j + LPR ci).
// Each of those slices is quantised once, chunk c by lane c % 64 (in its
// own slot c / 64), and every lane then gathers its CPL slices from the
// lanes that made them, one ds_bpermute per dword.  The slices are the
// ones load_slices gives, bit for bit: only the lane that computes them
// differs.
template <int FMT, int NT, int CPL, int LPR, bool XCOH = false>
__device__ __forceinline__ void load_slices_once(XSlice<FMT> (&xs)[NT][CPL], const float* act,
                                                 const int (&xrow)[NT], int K, int j,
                                                 int nchunks) {
  static_assert(LPR > 0 && LPR < kWave && kWave % LPR == 0, "lane groups of a wave");
  constexpr int NQ = (LPR * CPL + kWave - 1) / kWave;  // slices each lane makes
  constexpr int ND = (int)(sizeof(XSlice<FMT>) / 4);
  const int lane = threadIdx.x & (kWave - 1);
  XSlice<FMT> own[NT][NQ];
  load_slices<FMT, NT, NQ, XCOH>(own, act, xrow, K, lane, kWave, nchunks);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
      // Chunk j + LPR ci: LPR ci % 64 is a multiple of LPR and j < LPR, so
      // its slot (LPR ci) / 64 is the same for every lane.
      const int src = ((j + LPR * ci) & (kWave - 1)) * 4;
      uint32_t d[ND];
      __builtin_memcpy(d, &own[t][(LPR * ci) / kWave], sizeof(d));
#pragma unroll
      for (int i = 0; i < ND; ++i) d[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)d[i]);
      __builtin_memcpy(&xs[t][ci], d, sizeof(d));
    }
}

// acc += a * dot - b * xs.sum for one chunk: the chunk's contribution,
// with dot = sum_i q_i x16_i and a carrying the activation scale.
struct ChunkScale {
  float a, b;
};

__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ8_0>& ch, int /*sub*/) {
  return {f16_to_f32(ch.d), 0.f};
}

// Sub-block `sub` of a Q4_K header: a = d sc, b = dmin m.  The six-bit
// field at stream bit f (sc: f = 6 sub, m: f = 48 + 6 sub) lies in stream
// bytes f/8 and f/8 + 1; a byte permute with a lane-constant selector
// gathers those two bytes (sc from words y, z; m from z, w) and a
// bit-field extract takes the six bits.  `sub` is fixed per lane, so the
// selectors and offsets are computed once.
struct Q4kSel {
  uint32_t ssel, msel;  // v_perm selectors: the two bytes into bits 0..15
  uint32_t soff, moff;  // bit offsets of the fields in them
};
__device__ __forceinline__ Q4kSel q4k_sel(int sub) {
  // v_perm byte numbering: 0..3 = second operand (lower word), 4..7 = first.
  const int sb = (6 * sub) >> 3;            // stream byte of sc, in (y, z) = bytes 0..7
  const int mb = ((48 + 6 * sub) >> 3) - 4;  // stream byte of m, in (z, w) = bytes 0..7
  Q4kSel q;
  q.ssel = (uint32_t)sb | ((uint32_t)(sb + 1) << 8) | 0x0C0C0000u;  // 0x0C: zero byte
  // The last m field (stream bits 90..95) sits wholly in byte mb = 7.
  q.msel = (uint32_t)mb | ((uint32_t)(mb < 7 ? mb + 1 : 7) << 8) | 0x0C0C0000u;
  q.soff = (uint32_t)((6 * sub) & 7);
  q.moff = (uint32_t)((48 + 6 * sub) & 7);
  return q;
}
__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ4_K>& ch, const Q4kSel& q) {
  const uint4& h = ch.h;
  const uint32_t sc = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.z, h.y, q.ssel), q.soff, 6);
  const uint32_t m = __builtin_amdgcn_ubfe(__builtin_amdgcn_perm(h.w, h.z, q.msel), q.moff, 6);
  // fma with a zero addend rather than a product, so that each fp16 field
  // enters a mixed-precision FMA without a separate conversion.
  return {fmaf(f16_lo(h.x), (float)sc, 0.0f), fmaf(f16_hi(h.x), (float)m, 0.0f)};
}
__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ4_K>& ch, int sub) {
  return decode_scale(ch, q4k_sel(sub));
}

// Q2_K: a = d, b = dmin of the super-block (sub-block scales and mins are
// applied inside chunk_fma).
__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ2_K>& ch, int /*sub*/) {
  return {f16_lo(ch.dd), f16_hi(ch.dd)};
}

// Q3_K: a = d (the 6-bit scales are applied inside chunk_fma).
__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ3_K>& ch, int /*sub*/) {
  return {f16_lo(ch.d), 0.f};
}
// Q6_K: a = d (the 8-bit scales are applied inside chunk_fma).
__device__ __forceinline__ ChunkScale decode_scale(const Chunk<kQ6_K>& ch, int /*sub*/) {
  return {f16_lo(ch.d), 0.f};
}

// sum_i q_i x16_i over the chunk (exact in int32; converted with at most one
// rounding).
__device__ __forceinline__ float chunk_dot(const Chunk<kQ8_0>& ch, const XSlice<kQ8_0>& xs) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  int ah = 0, al = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ah = __builtin_amdgcn_sdot4((int)w[k], (int)xs.h[k], ah, false);
    al = __builtin_amdgcn_sdot4((int)w[k], (int)xs.l[k], al, false);
  }
  return fmaf((float)ah, 256.0f, (float)al);
}

__device__ __forceinline__ float chunk_dot(const Chunk<kQ4_K>& ch, const XSlice<kQ4_K>& xs) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  int ah = 0, al = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = (int)(w[k] & 0x0F0F0F0Fu), o = (int)((w[k] >> 4) & 0x0F0F0F0Fu);
    ah = __builtin_amdgcn_sdot4(e, (int)xs.h[2 * k], ah, false);
    ah = __builtin_amdgcn_sdot4(o, (int)xs.h[2 * k + 1], ah, false);
    al = __builtin_amdgcn_sdot4(e, (int)xs.l[2 * k], al, false);
    al = __builtin_amdgcn_sdot4(o, (int)xs.l[2 * k + 1], al, false);
  }
  return (float)(ah * 256 + al);  // |.| < 2^24: exact
}

// acc + the chunk's contribution sum_i w_i x_i.
__device__ __forceinline__ float chunk_fma(const Chunk<kQ8_0>& ch, const ChunkScale& k,
                                           const XSlice<kQ8_0>& xs, float acc) {
  return fmaf(k.a, chunk_dot(ch, xs) * xs.s, acc);
}
__device__ __forceinline__ float chunk_fma(const Chunk<kQ4_K>& ch, const ChunkScale& k,
                                           const XSlice<kQ4_K>& xs, float acc) {
  return fmaf(k.a, chunk_dot(ch, xs) * xs.s, fmaf(-k.b, xs.sum, acc));
}

// Q2_K: for sub-block k of the chunk, four v_dot4 per limb give the exact
// dot of its 16 quants with the 16-bit activations; the 4-bit scales then
// weight the four sub-block dots in int32 (|dot| <= 16*3*128 per limb, so
// each product fits the 24-bit multiply), and the mins weight the
// sub-block activation sums: contribution = d*s*(256 H + L) - dmin*sum_k
// m_k*sum_k.  The plane extractions and scale fields depend only on the
// chunk, so they are shared by every token of a pass.
__device__ __forceinline__ float chunk_fma(const Chunk<kQ2_K>& ch, const ChunkScale& k,
                                           const XSlice<kQ2_K>& xs, float acc) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  int ah = 0, al = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    int h = 0, l = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = (int)((w[b] >> (2 * j)) & 0x03030303u);
      h = __builtin_amdgcn_sdot4(p, (int)xs.h[4 * b + j], h, false);
      l = __builtin_amdgcn_sdot4(p, (int)xs.l[4 * b + j], l, false);
    }
    const int sc = (int)__builtin_amdgcn_ubfe(ch.sc, 8 * b, 4);
    // The sign extension from bit 23 is the identity on these values and
    // tells the compiler that a 24-bit multiply-add suffices.
    ah += __builtin_amdgcn_sbfe(h, 0, 24) * sc;
    al += __builtin_amdgcn_sbfe(l, 0, 24) * sc;
  }
  const uint32_t mv = (ch.sc >> 4) & 0x0F0F0F0Fu;
  float mn = (float)(mv & 0xFFu) * xs.sum[0];
  mn = fmaf((float)((mv >> 8) & 0xFFu), xs.sum[1], mn);
  mn = fmaf((float)((mv >> 16) & 0xFFu), xs.sum[2], mn);
  mn = fmaf((float)(mv >> 24), xs.sum[3], mn);
  return fmaf(k.a, fmaf((float)ah, 256.0f, (float)al) * xs.s, fmaf(-k.b, mn, acc));
}

// Q3_K: plane j of sub-block k is (w_k >> 2j) & 0x03030303 with the high
// bits (bit 4 (k % 2) + j of each byte of high dword k / 2) moved to bit 2
// of each byte, so one v_dot4 per limb takes four 3-bit quants Q.  Per
// sub-block the exact integer sum of (Q - 4) x16 is 256 H + L - 4 sum x16
// (|.| <= 16*4*32639 < 2^21), weighted by S - 32 in int32 with 24-bit
// multiply-adds; contribution = d*s*(that total).
__device__ __forceinline__ float chunk_fma(const Chunk<kQ3_K>& ch, const ChunkScale& k,
                                           const XSlice<kQ3_K>& xs, float acc) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  const uint32_t hw[2] = {ch.hb.x, ch.hb.y};
  const uint32_t sx = ch.sc ^ 0x20202020u;  // S - 32 as a signed 6-bit field
  int tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t H = hw[b >> 1];
    int h = 0, l = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * (b & 1) + j;
      const uint32_t hi = (i >= 2 ? (H >> (i - 2)) : (H << (2 - i))) & 0x04040404u;
      const int p = (int)(((w[b] >> (2 * j)) & 0x03030303u) | hi);
      h = __builtin_amdgcn_sdot4(p, (int)xs.h[4 * b + j], h, false);
      l = __builtin_amdgcn_sdot4(p, (int)xs.l[4 * b + j], l, false);
    }
    const int dsub = h * 256 + l + xs.nsum4[b];
    const int sc = __builtin_amdgcn_sbfe((int)sx, 8 * b, 6);
    tot += __builtin_amdgcn_sbfe(dsub, 0, 24) * sc;
  }
  return fmaf(k.a * xs.s, (float)tot, acc);
}

// Q6_K: dword k of the group's low nibbles gives its even / odd weights as
// Q4_K does; their high bit pairs sit at bits 4 (k % 2) / 4 (k % 2) + 2 of
// every byte of high dword k / 2 and move to bits 4..5 with one shift and
// one AND-OR, so one v_dot4 per limb takes four 6-bit quants Q.  Per
// sub-block (dwords 2t, 2t + 1) the exact integer sum of (Q - 32) x16 is
// 256 H + L - 32 sum x16 (|.| <= 16*32*32639 < 2^24, exact in fp32); the
// signed scales weight the two sub-blocks in fp32 and d*s the chunk.
__device__ __forceinline__ float chunk_fma(const Chunk<kQ6_K>& ch, const ChunkScale& k,
                                           const XSlice<kQ6_K>& xs, float acc) {
  const uint32_t w[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
  const uint32_t hw[2] = {ch.hb.x, ch.hb.y};
  float v = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t H = hw[t];
    int h = 0, l = 0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int d = 2 * t + kk;
      const uint32_t he = (kk == 0 ? (H << 4) : H) & 0x30303030u;
      const uint32_t ho = (kk == 0 ? (H << 2) : (H >> 2)) & 0x30303030u;
      const int e = (int)((w[d] & 0x0F0F0F0Fu) | he);
      const int o = (int)(((w[d] >> 4) & 0x0F0F0F0Fu) | ho);
      h = __builtin_amdgcn_sdot4(e, (int)xs.h[2 * d], h, false);
      h = __builtin_amdgcn_sdot4(o, (int)xs.h[2 * d + 1], h, false);
      l = __builtin_amdgcn_sdot4(e, (int)xs.l[2 * d], l, false);
      l = __builtin_amdgcn_sdot4(o, (int)xs.l[2 * d + 1], l, false);
    }
    const int dsub = h * 256 + l + xs.nsum32[t];
    const int sc = __builtin_amdgcn_sbfe((int)ch.sc, 8 * t, 8);
    v = fmaf((float)sc, (float)dsub, v);
  }
  return fmaf(k.a * xs.s, v, acc);
}

}  // namespace svr
