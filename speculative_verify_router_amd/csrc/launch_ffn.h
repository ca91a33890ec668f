// Single-role expert GEMV launches (k_ffn) for one tensor type: every
// chunks-per-lane count, for shapes and batch sizes without a fused
// instantiation.  Each type is its own translation unit (launch_ffn_*.hip)
// so that the families compile in parallel.
#pragma once

#include "launch.h"

namespace svr {
namespace host {

template <int FMT, bool GU>
bool launch_ffn_c(int cpl, FfnArgs a, int dtype, int slots, hipStream_t st) {
  switch (cpl) {
#define SVR_CASE(C)                                                                   \
  case C: {                                                                           \
    auto k = k_ffn<FMT, C, GU>;                                                       \
    size_role(a, dtype, slots, resident_blocks(k));                                   \
    hipLaunchKernelGGL(k, dim3(tiles_of(a), slots), dim3(kBlock), 0, st, a);          \
    return true;                                                                      \
  }
    SVR_CASE(1) SVR_CASE(2) SVR_CASE(3) SVR_CASE(4) SVR_CASE(5) SVR_CASE(6) SVR_CASE(7) SVR_CASE(8)
#undef SVR_CASE
    default: return false;
  }
}

template <int FMT>
bool launch_ffn_fmt(int dtype, bool gateup, FfnArgs a, int slots_max, hipStream_t st) {
  FfnShape s;
  ffn_shape(dtype, a.K, &s);
  return gateup ? launch_ffn_c<FMT, true>(s.cpl, a, dtype, slots_max, st)
                : launch_ffn_c<FMT, false>(s.cpl, a, dtype, slots_max, st);
}

}  // namespace host
}  // namespace svr
