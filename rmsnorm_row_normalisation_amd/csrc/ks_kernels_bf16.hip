// Kernels and plan dispatch for one storage dtype (__bf16).
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_bf16(const Launch &l) { return launch_typed<__bf16>(l); }

}  // namespace ks
