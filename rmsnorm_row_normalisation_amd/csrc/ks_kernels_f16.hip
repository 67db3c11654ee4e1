// Kernels and plan dispatch for one storage dtype (_Float16).
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_f16(const Launch &l) { return launch_typed<_Float16>(l); }

}  // namespace ks
