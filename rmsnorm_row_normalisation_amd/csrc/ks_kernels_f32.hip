// Kernels and plan dispatch for one storage dtype (float).
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_f32(const Launch &l) { return launch_typed<float>(l); }

}  // namespace ks
