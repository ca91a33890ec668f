// Single-role expert GEMV launches (k_ffn): dispatch on the tensor type to
// the per-type translation units.
#include "launch.h"

namespace svr {
namespace host {

template <int FMT>
bool launch_ffn_fmt(int dtype, bool gateup, FfnArgs a, int slots_max, hipStream_t st);

bool launch_ffn(int dtype, bool gateup, FfnArgs a, int slots_max, hipStream_t st) {
  switch (dtype) {
    case MOE_Q8_0: return launch_ffn_fmt<kQ8_0>(dtype, gateup, a, slots_max, st);
    case MOE_Q4_K: return launch_ffn_fmt<kQ4_K>(dtype, gateup, a, slots_max, st);
    case MOE_Q2_K: return launch_ffn_fmt<kQ2_K>(dtype, gateup, a, slots_max, st);
    case MOE_Q3_K: return launch_ffn_fmt<kQ3_K>(dtype, gateup, a, slots_max, st);
    case MOE_Q6_K: return launch_ffn_fmt<kQ6_K>(dtype, gateup, a, slots_max, st);
    default: return false;
  }
}

}  // namespace host
}  // namespace svr
