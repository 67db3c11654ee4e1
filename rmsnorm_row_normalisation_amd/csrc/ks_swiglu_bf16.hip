// SwiGLU kernels for bfloat16.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_swiglu_bf16(const SwigluLaunch &l) { return launch_swiglu_typed<bf16>(l); }

}  // namespace ks
