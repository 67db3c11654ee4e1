// Softmax kernels for float16: vector and generic paths.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_softmax_f16(const Launch &l)
{
    if (l.plan.path == KS_PATH_GENERIC)
        return launch_generic_typed<f16, KS_OP_SOFTMAX>(l);
    return vec_by_tpr<f16, KS_OP_SOFTMAX>(l);
}

}  // namespace ks
