// SwiGLU kernels for float16.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_swiglu_f16(const SwigluLaunch &l) { return launch_swiglu_typed<f16>(l); }

}  // namespace ks
