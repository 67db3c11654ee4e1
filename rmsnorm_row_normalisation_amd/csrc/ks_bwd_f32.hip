// RMSNorm backward kernels for float32: vector and generic paths and the
// dw reduction.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_bwd_f32(const BwdLaunch &l) { return launch_bwd_typed<f32>(l); }

}  // namespace ks
