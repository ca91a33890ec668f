// Fused expert launches of the staged path: routed gate/up with the shared
// down (k_dual), and the routed down with its combine (k_down_tok for pair
// slots, k_down_combine otherwise), one instantiation per known shape.
#include "launch.h"

namespace svr {
namespace host {

// Phase 2: routed gate/up (A) + shared down (B) in one grid.  The resident
// round is split in proportion to the bytes each side's waves stream: the
// shared side's waves each take one token over the same rows.
//
// The round is one workgroup per CU for Q4_K gate/up over 32 or more
// (token, slot) pairs (per-pair tiles, four tokens of top-8): a second
// wave per SIMD buys it no bandwidth, and half as many tiles of twice the
// rows spend less on per-tile start-up and activation quantisation (about
// 1 us per layer at four tokens).  The other formats do more arithmetic
// per byte and need the second wave to cover it (Q2_K: 4 us slower at one
// workgroup per CU; Q8_0 at one token: 1 us slower).
template <int FA, int SA, int FB, int SB>
void launch_dual_t(hipStream_t st, FfnArgs a, FfnArgs b, const DualPlan& d) {
  auto k = k_dual<FA, SA, true, FB, SB, false>;
  const bool one_per_cu = FA == kQ4_K && a.pair_expert && d.slots >= 32;
  const int64_t cap = one_per_cu ? device_cus() : resident_blocks(k);
  int64_t bb = (int64_t)((double)cap * d.b_work / (double)(d.a_work + d.b_work) + 0.5);
  if (bb < 1) bb = 1;
  if (bb > cap / 2) bb = cap / 2;
  size_role(a, d.adtype, d.slots, cap - bb);
  size_role(b, d.bdtype, 1, bb);
  const int at = tiles_of(a), na = at * d.slots;
  hipLaunchKernelGGL(k, dim3(na + tiles_of(b)), dim3(kBlock), 0, st, a, at, na, b);
}

bool launch_dual_keys(int akey, int bkey, hipStream_t st, const FfnArgs& a, const FfnArgs& b,
                      const DualPlan& d) {
#define SVR_D(FA, CA, LA, FB, CB, LB)                                                   \
  if (akey == key(FA, shape_code(CA, LA)) && bkey == key(FB, shape_code(CB, LB))) {    \
    launch_dual_t<FA, shape_code(CA, LA), FB, shape_code(CB, LB)>(st, a, b, d);        \
    return true;                                                                         \
  }
#define SVR_DG(FA, CA)                                                                  \
  SVR_D(FA, CA, 0, kQ8_0, 1, 0) SVR_D(FA, CA, 0, kQ8_0, 2, 0) SVR_D(FA, CA, 0, kQ8_0, 3, 0) \
  SVR_D(FA, CA, 0, kQ8_0, 5, 0)
  SVR_D(kQ4_K, 2, 64, kQ8_0, 5, 16) SVR_D(kQ4_K, 2, 64, kQ8_0, 3, 32)
  SVR_D(kQ8_0, 4, 64, kQ8_0, 5, 16) SVR_D(kQ8_0, 4, 64, kQ8_0, 3, 32)
  SVR_D(kQ2_K, 1, 64, kQ8_0, 5, 16) SVR_D(kQ2_K, 1, 64, kQ8_0, 3, 32)
  SVR_D(kQ6_K, 2, 64, kQ8_0, 5, 16)
  SVR_DG(kQ4_K, 1) SVR_DG(kQ4_K, 2) SVR_DG(kQ4_K, 3) SVR_DG(kQ8_0, 4) SVR_DG(kQ2_K, 1)
  SVR_DG(kQ3_K, 1) SVR_DG(kQ6_K, 2)
#undef SVR_DG
#undef SVR_D
  return false;
}

bool launch_dual(int adtype, const FfnShape& as, int bdtype, const FfnShape& bs, hipStream_t st,
                 const FfnArgs& a, const FfnArgs& b, const DualPlan& d) {
  return launch_dual_keys(exact_key(adtype, as), exact_key(bdtype, bs), st, a, b, d) ||
         launch_dual_keys(generic_key(adtype, as), generic_key(bdtype, bs), st, a, b, d);
}

// Phase 3 with pair slots: one workgroup per (token, row tile), one
// resident round of them (the rows of a tile a whole number of wave steps,
// at most one per thread).
template <int F, int S>
bool launch_down_tok_t(hipStream_t st, FfnArgs a, const CombineArgs& c, int dtype) {
  auto k = k_down_tok<F, S>;
  FfnShape s;
  ffn_shape(dtype, a.K, &s);
  a.lpr = s.lpr;
  const int G = kWave / s.lpr;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kDownTokThreads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int64_t tiles = (int64_t)per_cu * device_cus() / (c.M > 0 ? c.M : 1);
  if (tiles < 1) tiles = 1;
  int64_t upb = (a.rows_per_expert + tiles - 1) / tiles;
  upb = (upb + G - 1) / G * G;
  if (upb > kDownTokRows) upb = kDownTokRows / G * G;
  a.units_per_block = (int)upb;
  const int nt = (a.rows_per_expert + a.units_per_block - 1) / a.units_per_block;
  hipLaunchKernelGGL(k, dim3((unsigned)(nt * c.M)), dim3(kDownTokThreads), 0, st, a, c, nt);
  return true;
}

bool launch_down_tok(int dtype, const FfnShape& ds, hipStream_t st, const FfnArgs& a,
                     const CombineArgs& c) {
#define SVR_DT(F, C, L) \
  if (key(F, shape_code(C, L)) == kk) return launch_down_tok_t<F, shape_code(C, L)>(st, a, c, dtype);
  for (int kk : {exact_key(dtype, ds), generic_key(dtype, ds)}) {
    SVR_DT(kQ4_K, 3, 16) SVR_DT(kQ8_0, 5, 16) SVR_DT(kQ8_0, 3, 32)
    SVR_DT(kQ4_K, 1, 0) SVR_DT(kQ4_K, 2, 0) SVR_DT(kQ4_K, 3, 0) SVR_DT(kQ8_0, 1, 0)
    SVR_DT(kQ8_0, 2, 0) SVR_DT(kQ8_0, 3, 0) SVR_DT(kQ8_0, 4, 0) SVR_DT(kQ8_0, 5, 0)
    SVR_DT(kQ8_0, 6, 0) SVR_DT(kQ2_K, 1, 32) SVR_DT(kQ2_K, 1, 0) SVR_DT(kQ3_K, 1, 32)
    SVR_DT(kQ3_K, 1, 0) SVR_DT(kQ6_K, 3, 16) SVR_DT(kQ6_K, 3, 0) SVR_DT(kQ6_K, 1, 0)
  }
#undef SVR_DT
  return false;
}

// Phase 3: routed down + combine, one resident round of row tiles x slots.
template <int F, int S>
bool launch_down_combine_t(hipStream_t st, FfnArgs a, const CombineArgs& c, int dtype, int slots) {
  auto k = k_down_combine<F, S>;
  size_role(a, dtype, slots, resident_blocks(k));
  const int tiles = tiles_of(a);
  if (tiles > kMaxTiles) return false;
  hipLaunchKernelGGL(k, dim3(tiles, slots), dim3(kBlock), 0, st, a, c);
  return true;
}

bool launch_down_combine_key(int k, hipStream_t st, const FfnArgs& a, const CombineArgs& c,
                             int dtype, int slots) {
#define SVR_DC(F, C, L) \
  if (k == key(F, shape_code(C, L))) return launch_down_combine_t<F, shape_code(C, L)>(st, a, c, dtype, slots);
  SVR_DC(kQ4_K, 3, 16) SVR_DC(kQ8_0, 5, 16)
  SVR_DC(kQ4_K, 1, 0) SVR_DC(kQ4_K, 2, 0) SVR_DC(kQ4_K, 3, 0) SVR_DC(kQ8_0, 1, 0) SVR_DC(kQ8_0, 2, 0)
  SVR_DC(kQ8_0, 3, 0) SVR_DC(kQ8_0, 4, 0) SVR_DC(kQ8_0, 5, 0) SVR_DC(kQ8_0, 6, 0)
  SVR_DC(kQ2_K, 1, 32) SVR_DC(kQ2_K, 1, 0) SVR_DC(kQ3_K, 1, 32) SVR_DC(kQ3_K, 1, 0)
  SVR_DC(kQ6_K, 3, 16) SVR_DC(kQ6_K, 3, 0)
#undef SVR_DC
  return false;
}

bool launch_down_combine(int dtype, const FfnShape& ds, hipStream_t st, const FfnArgs& a,
                         const CombineArgs& c, int slots) {
  return launch_down_combine_key(exact_key(dtype, ds), st, a, c, dtype, slots) ||
         launch_down_combine_key(generic_key(dtype, ds), st, a, c, dtype, slots);
}

}  // namespace host
}  // namespace svr
