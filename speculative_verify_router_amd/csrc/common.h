// Device helpers shared by the gfx950 kernels of the routed-MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_layer.h"

namespace svr {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kBlock = 256;        // threads per workgroup (4 waves)
constexpr int kMaxExperts = 1024;  // experts per layer
constexpr int kMaxTopK = 64;       // selected experts per token
constexpr int kMaxChunksPerLane = 8;

// fp16 bit pattern -> float (v_cvt_f32_f16; subnormals kept).
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// Sum over an aligned group of `lpr` consecutive lanes (lpr a power of two
// <= 64); every lane of the group receives the total.
__device__ __forceinline__ float group_sum(float v, int lpr) {
  for (int off = lpr >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, kWave); }

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float4 ldf4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

// Byte b of a dword as float (v_cvt_f32_ubyte{0..3}).
template <int B>
__device__ __forceinline__ float ubyte_f(uint32_t v) {
  return (float)((v >> (8 * B)) & 0xFFu);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace svr
