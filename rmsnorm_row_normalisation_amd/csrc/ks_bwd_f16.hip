// RMSNorm backward kernels for float16: vector and generic paths and the
// dw reduction.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_bwd_f16(const BwdLaunch &l) { return launch_bwd_typed<f16>(l); }

}  // namespace ks
