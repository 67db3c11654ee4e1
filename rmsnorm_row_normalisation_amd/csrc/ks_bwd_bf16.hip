// RMSNorm backward kernels for bfloat16: vector and generic paths and the
// dw reduction.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_bwd_bf16(const BwdLaunch &l) { return launch_bwd_typed<bf16>(l); }

}  // namespace ks
