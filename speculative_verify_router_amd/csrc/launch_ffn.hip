// Single-role expert GEMV launches (k_ffn): every (format, chunks per lane)
// pair, for shapes and batch sizes without a fused instantiation.
#include "launch.h"

namespace svr {
namespace host {

// Single-role launches, every (format, chunks-per-lane) pair.
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

bool launch_ffn(int dtype, bool gateup, FfnArgs a, int slots_max, hipStream_t st) {
  FfnShape s;
  ffn_shape(dtype, a.K, &s);
  if (dtype == MOE_Q8_0)
    return gateup ? launch_ffn_c<kQ8_0, true>(s.cpl, a, dtype, slots_max, st)
                  : launch_ffn_c<kQ8_0, false>(s.cpl, a, dtype, slots_max, st);
  if (dtype == MOE_Q2_K)
    return gateup ? launch_ffn_c<kQ2_K, true>(s.cpl, a, dtype, slots_max, st)
                  : launch_ffn_c<kQ2_K, false>(s.cpl, a, dtype, slots_max, st);
  if (dtype == MOE_Q3_K)
    return gateup ? launch_ffn_c<kQ3_K, true>(s.cpl, a, dtype, slots_max, st)
                  : launch_ffn_c<kQ3_K, false>(s.cpl, a, dtype, slots_max, st);
  if (dtype == MOE_Q6_K)
    return gateup ? launch_ffn_c<kQ6_K, true>(s.cpl, a, dtype, slots_max, st)
                  : launch_ffn_c<kQ6_K, false>(s.cpl, a, dtype, slots_max, st);
  return gateup ? launch_ffn_c<kQ4_K, true>(s.cpl, a, dtype, slots_max, st)
                : launch_ffn_c<kQ4_K, false>(s.cpl, a, dtype, slots_max, st);
}

}  // namespace host
}  // namespace svr
