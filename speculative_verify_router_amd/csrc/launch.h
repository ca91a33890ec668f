// Host-side launch helpers shared by the library's translation units:
// tensor-type properties, lane shapes, occupancy-sized work splits and the
// kernel-family launchers that live in their own translation units (so the
// families compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <unordered_map>

#include "ffn.h"
#include "moe_layer.h"
#include "phases.h"

namespace svr {
namespace host {

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline int wpc_of(int dtype) {
  return dtype == MOE_Q8_0 ? 16 : (dtype == MOE_Q4_K || dtype == MOE_Q6_K) ? 32 : 64;
}
inline int blk_of(int dtype) { return dtype == MOE_Q8_0 ? 32 : 256; }
// Types of the shared expert, and of the routed experts (also Q2_K, Q3_K,
// Q6_K).
inline bool quant_type(int dtype) { return dtype == MOE_Q8_0 || dtype == MOE_Q4_K; }
inline bool gemv_only_type(int dtype) {
  return dtype == MOE_Q2_K || dtype == MOE_Q3_K || dtype == MOE_Q6_K;
}
inline bool routed_type(int dtype) { return quant_type(dtype) || gemv_only_type(dtype); }
inline int qfmt(int dtype) {
  switch (dtype) {
    case MOE_Q8_0: return kQ8_0;
    case MOE_Q4_K: return kQ4_K;
    case MOE_Q2_K: return kQ2_K;
    case MOE_Q3_K: return kQ3_K;
    default: return kQ6_K;
  }
}

// Lanes per row and 16-byte chunks per lane for a row of K columns.  The
// shape keeps the per-lane activation slice within 96 floats (Q4_K: 3
// chunks of 32, Q8_0: 6 chunks of 16, Q2_K and Q3_K: 1 chunk of 64, Q6_K: 3
// chunks of 32) where possible and wastes the fewest
// lane positions (chunk positions past the row's end load the row's last
// chunk against a zero activation); among equal shapes the fewest chunks
// per lane.  Rows too long for that take 64 lanes and up to 8 chunks.
struct FfnShape {
  int lpr, cpl;
};
inline bool ffn_shape(int dtype, int K, FfnShape* s) {
  if (K <= 0 || K % blk_of(dtype)) return false;
  const int chunks = K / wpc_of(dtype);
  const int cap = 96 / wpc_of(dtype);
  double best = 0.0;
  for (int lpr = 64; lpr >= 1; lpr >>= 1) {
    const int cpl = (chunks + lpr - 1) / lpr;
    if (cpl > cap) continue;
    const double eff = (double)chunks / (double)(lpr * cpl);
    if (eff > best + 1e-12) {
      best = eff;
      s->lpr = lpr;
      s->cpl = cpl;
    }
  }
  if (best > 0.0) return true;
  const int cpl = (chunks + kWave - 1) / kWave;
  if (cpl > kMaxChunksPerLane) return false;
  s->lpr = kWave;
  s->cpl = cpl;
  return true;
}

// --------------------------------------------------------------------------
// Work split.  Every launch is sized to about one round of resident
// workgroups (CUs x workgroups per CU for that kernel), since a partial
// second round costs a whole extra pass of latency.  A role's rows are cut
// into tiles of a whole number of wave steps.
// --------------------------------------------------------------------------
inline int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Workgroups of `kernel` resident at once on the device: CUs x the
// occupancy query, cached per kernel.
template <typename K>
inline int resident_blocks(K kernel) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> per_cu;
  const void* key = reinterpret_cast<const void*>(kernel);
  int v = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = per_cu.find(key);
    if (it != per_cu.end()) v = it->second;
  }
  if (!v) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, kBlock, 0) != hipSuccess || v < 1)
      v = 1;
    std::lock_guard<std::mutex> lock(mu);
    per_cu[key] = v;
  }
  return v * device_cus();
}

// Rows per workgroup for `blocks` workgroups over `slots` experts.
inline void size_role(FfnArgs& a, int dtype, int slots, int64_t blocks) {
  FfnShape s;
  ffn_shape(dtype, a.K, &s);
  a.lpr = s.lpr;
  const int G = kWave / s.lpr;  // rows per wave step
  const int unit_step = a.split_tokens ? G : kWavesPerBlock * G;
  int64_t tiles = blocks / (slots > 0 ? slots : 1);
  // Workgroups go to the 8 XCDs round-robin by linear index (tile fastest):
  // with a multiple of 8 tiles, every slot's tile t runs on XCD t % 8, so
  // slots that stream the same expert share that XCD's L2.  Rounded down
  // only where that leaves at most 1/8 of the round idle.
  if (tiles >= 8 && tiles % 8 <= tiles / 8) tiles -= tiles % 8;
  if (tiles < 1) tiles = 1;
  int64_t upb = (a.rows_per_expert + tiles - 1) / tiles;
  upb = (upb + unit_step - 1) / unit_step * unit_step;
  if (a.max_rows > 0 && upb > a.max_rows)
    upb = std::max<int64_t>(unit_step, a.max_rows / unit_step * unit_step);
  a.units_per_block = (int)upb;
}

// Shared-expert tiles of phase 1: the workgroup slots of one resident round
// that the router rows leave free (at least a quarter of the round), each
// taking an equal share of the rows.  A wave's token group of 4 / M waves
// shares a tile's rows (see ffn_tile_tokens), so a tile is a whole number
// of that group's steps.
inline void size_shared_tiles(FfnArgs& a, int dtype, int64_t blocks) {
  FfnShape s;
  ffn_shape(dtype, a.K, &s);
  a.lpr = s.lpr;
  const int G = kWave / s.lpr;
  const int rg = a.n_tokens < kWavesPerBlock ? kWavesPerBlock / a.n_tokens : 1;
  const int unit = rg * G;
  if (blocks < 1) blocks = 1;
  int64_t rows = (a.rows_per_expert + blocks - 1) / blocks;
  rows = (rows + unit - 1) / unit * unit;
  a.units_per_block = (int)rows;
}

inline int tiles_of(const FfnArgs& a) {
  return (a.rows_per_expert + a.units_per_block - 1) / a.units_per_block;
}

// Bytes per weight row of K columns.
inline double row_bytes(int dtype, int K) {
  if (dtype == MOE_Q8_0) return K / 32 * 34.0;
  return K / 256 * (dtype == MOE_Q4_K ? 144.0 : dtype == MOE_Q2_K ? 84.0 : dtype == MOE_Q3_K ? 114.0 : 210.0);
}

// Fused instantiations.  A key packs (format, shape code); each launcher
// tries the exact lane shape first (lanes per row fixed at compile time),
// then a generic instantiation with the same chunks per lane that reads the
// lanes per row at run time.
constexpr int key(int fmt, int code) { return fmt * 65536 + code; }
inline int exact_key(int dtype, const FfnShape& s) { return key(qfmt(dtype), shape_code(s.cpl, s.lpr)); }
inline int generic_key(int dtype, const FfnShape& s) { return key(qfmt(dtype), shape_code(s.cpl, 0)); }


// Phase 2 split of one resident round between its two roles.
struct DualPlan {
  int64_t a_work, b_work;  // bytes streamed by all waves of each side
  int slots;               // routed expert slots
  int adtype, bdtype;
};

// Kernel-family launchers (launch_ffn.hip, launch_expert.hip).  Each
// returns false when no instantiation matches the shape.
bool launch_ffn(int dtype, bool gateup, FfnArgs a, int slots_max, hipStream_t st);
bool launch_dual(int adtype, const FfnShape& as, int bdtype, const FfnShape& bs, hipStream_t st,
                 const FfnArgs& a, const FfnArgs& b, const DualPlan& d);
bool launch_down_tok(int dtype, const FfnShape& ds, hipStream_t st, const FfnArgs& a,
                     const CombineArgs& c);
bool launch_down_combine(int dtype, const FfnShape& ds, hipStream_t st, const FfnArgs& a,
                         const CombineArgs& c, int slots);

}  // namespace host
}  // namespace svr
