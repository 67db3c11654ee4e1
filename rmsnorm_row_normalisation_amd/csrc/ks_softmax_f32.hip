// Softmax kernels for float32: vector, generic and split paths.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_softmax_f32(const Launch &l) { return launch_softmax_typed<f32>(l); }

}  // namespace ks
