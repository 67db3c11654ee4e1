// Softmax kernels for float16: vector, generic and split paths.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_softmax_f16(const Launch &l) { return launch_softmax_typed<f16>(l); }

}  // namespace ks
