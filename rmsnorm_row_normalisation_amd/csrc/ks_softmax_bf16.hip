// Softmax kernels for bfloat16: vector, generic and split paths.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_softmax_bf16(const Launch &l) { return launch_softmax_typed<bf16>(l); }

}  // namespace ks
