// k_ffn launches for Q8_0 tensors (see launch_ffn.h).
#include "launch_ffn.h"

namespace svr {
namespace host {
template bool launch_ffn_fmt<kQ8_0>(int, bool, FfnArgs, int, hipStream_t);
}  // namespace host
}  // namespace svr
