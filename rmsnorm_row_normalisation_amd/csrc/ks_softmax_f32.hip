// Softmax kernels for float32: vector and generic paths.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_softmax_f32(const Launch &l)
{
    if (l.plan.path == KS_PATH_GENERIC)
        return launch_generic_typed<f32, KS_OP_SOFTMAX>(l);
    return vec_by_tpr<f32, KS_OP_SOFTMAX>(l);
}

}  // namespace ks
