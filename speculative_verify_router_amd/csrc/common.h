// Device helpers shared by the gfx950 kernels of the routed-MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_layer.h"

namespace svr {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kBlock = 256;        // threads per workgroup (4 waves)
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxExperts = 1024;  // experts per layer
constexpr int kMaxTopK = 64;       // selected experts per token
// Batches up to this size give every (token, slot) pair its own workgroups
// (equal work per workgroup) instead of grouping them by expert.
constexpr int kPairTokens = 4;
constexpr int kMaxChunksPerLane = 8;
// Hand-off counters at the start of the workspace (zero between calls).
constexpr int kCounterBytes = 16384;

// fp16 bit pattern -> float (v_cvt_f32_f16; subnormals kept: the kernels run
// with fp16/fp64 denormals enabled).
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}
__device__ __forceinline__ float f16_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// DPP lane moves.  update_dpp(old, src, ...) returns `old` in lanes whose
// source is outside the row (row_shr) or whose row is masked off.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Sum over each aligned group of `lpr` lanes (lpr a power of two <= 64),
// delivered in the group's LAST lane (other lanes hold partial sums).  Only
// DPP moves: an inclusive scan inside 16-lane rows, then row broadcasts.
__device__ __forceinline__ float group_sum_last(float v, int lpr) {
  if (lpr >= 2) v += dpp<kDppShr1>(0.f, v);
  if (lpr >= 4) v += dpp<kDppShr2>(0.f, v);
  if (lpr >= 8) v += dpp<kDppShr4>(0.f, v);
  if (lpr >= 16) v += dpp<kDppShr8>(0.f, v);
  if (lpr >= 32) v += dpp<kDppBcast15, 0xA>(0.f, v);
  if (lpr >= 64) v += dpp<kDppBcast31, 0xC>(0.f, v);
  return v;
}

// Sum over the whole wave, returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, group_sum_last(v, kWave)), kWave - 1));
}

// Maximum / minimum of a u32 over the wave, returned to every lane.  Lanes
// without a DPP source take the operation's identity (0 for max, ~0 for
// min), which lets each step fold into one DPP-modified max / min.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppShr1>(0u, v));
  v = max(v, dpp_u<kDppShr2>(0u, v));
  v = max(v, dpp_u<kDppShr4>(0u, v));
  v = max(v, dpp_u<kDppShr8>(0u, v));
  v = max(v, dpp_u<kDppBcast15, 0xA>(0u, v));
  v = max(v, dpp_u<kDppBcast31, 0xC>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<kDppShr1>(~0u, v));
  v = min(v, dpp_u<kDppShr2>(~0u, v));
  v = min(v, dpp_u<kDppShr4>(~0u, v));
  v = min(v, dpp_u<kDppShr8>(~0u, v));
  v = min(v, dpp_u<kDppBcast15, 0xA>(~0u, v));
  v = min(v, dpp_u<kDppBcast31, 0xC>(~0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Hand-off stores and loads for data that another workgroup, possibly on
// another XCD, reads in the same launch: agent-scope relaxed atomics write
// through and read past the per-XCD L2, so no cache-wide release or
// acquire fence is needed.
template <typename T>
__device__ __forceinline__ void store_shared(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_shared(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// silu(g) = g / (1 + e^-g) with the hardware reciprocal (1 ulp); e^-g
// overflowing to inf gives -0 for very negative g, as the limit requires.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Order-preserving 32-bit key of a float: a larger value gives a larger
// key; -0 maps to +0's key and NaN to -inf's.  Every finite or infinite
// value has a key of at least 0x007FFFFF, so 0 is below all of them.
__device__ __forceinline__ uint32_t order_key(float v) {
  v = (v != v) ? -INFINITY : v + 0.0f;
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Buffer resource over [base, base + bytes): 16-byte loads with 32-bit
// offsets; reads past `bytes` return zero.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}
// 16-byte load that reads past the per-XCD L2 (sc1), for data another
// workgroup of the same launch wrote with store_shared.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ f32x4 bload16_shared(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
}

// "Last workgroup done" hand-off.  Every wave of the workgroup must have
// waited for its hand-off stores (store_shared) to complete -- wait_stores()
// -- before the barrier that precedes this call by one thread.  Returns the
// counter's previous value.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ unsigned arrive(unsigned* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace svr
