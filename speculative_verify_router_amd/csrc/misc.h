// Weighted combine of expert outputs, and the block-decoder test hook.
#pragma once

#include "common.h"

namespace svr {

// y[t][h] = s[t][h] + sum_{j=0..k-1} w[t][j] * o[t*k + j][h], in slot order.
// One thread per 4 consecutive outputs (float4 loads/stores).
static __global__ __launch_bounds__(kBlock) void k_combine(const float* __restrict__ o,
                                                    const float* __restrict__ s,
                                                    const float* __restrict__ w,
                                                    float* __restrict__ y, int M, int H, int k) {
  const int64_t i4 = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int H4 = H >> 2;
  if (i4 >= (int64_t)M * H4) return;
  const int t = (int)(i4 / H4);
  const int c = (int)(i4 - (int64_t)t * H4);
  float4 acc = s ? ldf4(s + (int64_t)t * H + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(int64_t)t * k + j];
    const float4 v = ldf4(o + ((int64_t)t * k + j) * H + 4 * c);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  *reinterpret_cast<float4*>(y + (int64_t)t * H + 4 * c) = acc;
}

// Dequantise rows [r0, r0 + n) of a planar tensor into out[n][cols].
// Q8_0: d*q.  Q4_K and Q2_K: fma(d*sc, q, -(dmin*m)); d*sc and dmin*m are
// exact in fp32, so the result is the correctly rounded block value.  Q3_K:
// (d*(S-32))*(Q-4), exact (at most 20 significant bits).  Q6_K:
// (d*sc)*(Q-32), exact (d*sc has at most 18 significant bits and
// |Q-32| <= 32 adds at most 5).
static __global__ __launch_bounds__(kBlock) void k_dequant(int fmt, const uint8_t* __restrict__ base,
                                                    int64_t rows, int cols, int64_t r0, int64_t n,
                                                    float* __restrict__ out) {
  const int64_t total = n * cols;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kBlock) {
    const int64_t r = r0 + i / cols;
    const int c = (int)(i % cols);
    float v;
    if (fmt == MOE_Q8_0) {
      const int64_t nb = cols >> 5;
      const int64_t qoff = ((2 * rows * nb) + 255) & ~(int64_t)255;
      const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(base + 2 * (r * nb + (c >> 5))));
      const int q = (int)(int8_t)base[qoff + r * cols + c];
      v = d * (float)q;
    } else if (fmt == MOE_Q2_K) {
      const int64_t n_sb = rows * (cols >> 8);
      const int64_t soff = (4 * n_sb + 255) & ~(int64_t)255;
      const int64_t qoff = (soff + 16 * n_sb + 255) & ~(int64_t)255;
      const int64_t rec = r * (cols >> 8) + (c >> 8);
      const uint8_t* dd = base + 4 * rec;
      const float d = f16_to_f32((uint32_t)dd[0] | ((uint32_t)dd[1] << 8));
      const float dmin = f16_to_f32((uint32_t)dd[2] | ((uint32_t)dd[3] << 8));
      const int s = (c >> 4) & 15, wi = c & 15;
      const uint32_t sm = base[soff + 16 * rec + s];
      const uint32_t qb = base[qoff + 64 * rec + 4 * s + (wi & 3)];
      const float q = (float)((qb >> (2 * (wi >> 2))) & 3u);
      v = fmaf(d * (float)(sm & 15u), q, -(dmin * (float)(sm >> 4)));
    } else if (fmt == MOE_Q3_K) {
      const int64_t n_sb = rows * (cols >> 8);
      const int64_t soff = (2 * n_sb + 255) & ~(int64_t)255;
      const int64_t loff = (soff + 16 * n_sb + 255) & ~(int64_t)255;
      const int64_t hoff = (loff + 64 * n_sb + 255) & ~(int64_t)255;
      const int64_t rec = r * (cols >> 8) + (c >> 8);
      const float d = f16_to_f32((uint32_t)base[2 * rec] | ((uint32_t)base[2 * rec + 1] << 8));
      const int s = (c >> 4) & 15, wi = c & 15;
      const int S = (int)(base[soff + 16 * rec + s] & 63u) - 32;
      const uint32_t lo = (base[loff + 64 * rec + 4 * s + (wi & 3)] >> (2 * (wi >> 2))) & 3u;
      const uint32_t hi = (base[hoff + 32 * rec + 4 * (s >> 1) + (wi & 3)] >> (4 * (s & 1) + (wi >> 2))) & 1u;
      v = (d * (float)S) * (float)((int)(lo | (hi << 2)) - 4);
    } else if (fmt == MOE_Q6_K) {
      const int64_t n_sb = rows * (cols >> 8);
      const int64_t soff = (2 * n_sb + 255) & ~(int64_t)255;
      const int64_t loff = (soff + 16 * n_sb + 255) & ~(int64_t)255;
      const int64_t hoff = (loff + 128 * n_sb + 255) & ~(int64_t)255;
      const int64_t rec = r * (cols >> 8) + (c >> 8);
      const float d = f16_to_f32((uint32_t)base[2 * rec] | ((uint32_t)base[2 * rec + 1] << 8));
      const int g = (c >> 5) & 7, wi = c & 31;
      const int sc = (int)(int8_t)base[soff + 16 * rec + 2 * g + (wi >> 4)];
      const uint32_t lo = (base[loff + 128 * rec + 16 * g + (wi >> 1)] >> (4 * (wi & 1))) & 15u;
      const uint32_t hi = (base[hoff + 64 * rec + 8 * g + 4 * (wi >> 4) + ((wi & 7) >> 1)] >>
                           (4 * ((wi >> 3) & 1) + 2 * (wi & 1))) & 3u;
      v = (d * (float)sc) * (float)((int)(lo | (hi << 4)) - 32);
    } else {
      const int64_t ns = cols >> 8;
      const int64_t rec = r * ns + (c >> 8);
      const uint8_t* h = base + 16 * rec;
      const float d = f16_to_f32((uint32_t)h[0] | ((uint32_t)h[1] << 8));
      const float dmin = f16_to_f32((uint32_t)h[2] | ((uint32_t)h[3] << 8));
      const int s = (c >> 5) & 7;
      const int wi = c & 31;
      const int sb = 6 * s, mb = 48 + 6 * s;  // bit offsets in the 96-bit stream
      const uint32_t sc = (((uint32_t)h[4 + (sb >> 3)] | ((uint32_t)h[4 + min((sb >> 3) + 1, 11)] << 8)) >> (sb & 7)) & 63u;
      const uint32_t m = (((uint32_t)h[4 + (mb >> 3)] | ((uint32_t)h[4 + min((mb >> 3) + 1, 11)] << 8)) >> (mb & 7)) & 63u;
      const uint8_t qb = base[16 * rows * ns + 128 * rec + 16 * s + (wi >> 1)];
      const float q = (float)((wi & 1) ? (qb >> 4) : (qb & 15));
      v = fmaf(d * (float)sc, q, -(dmin * (float)m));
    }
    out[i] = v;
  }
}

}  // namespace svr
