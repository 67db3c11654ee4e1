// SwiGLU kernels for float32.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_swiglu_f32(const SwigluLaunch &l) { return launch_swiglu_typed<f32>(l); }

}  // namespace ks
