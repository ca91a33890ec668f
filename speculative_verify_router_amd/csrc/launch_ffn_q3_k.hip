// k_ffn launches for Q3_K tensors (see launch_ffn.h).
#include "launch_ffn.h"

namespace svr {
namespace host {
template bool launch_ffn_fmt<kQ3_K>(int, bool, FfnArgs, int, hipStream_t);
}  // namespace host
}  // namespace svr
