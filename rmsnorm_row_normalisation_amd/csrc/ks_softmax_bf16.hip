// Softmax kernels for bfloat16: vector and generic paths.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_softmax_bf16(const Launch &l)
{
    if (l.plan.path == KS_PATH_GENERIC)
        return launch_generic_typed<bf16, KS_OP_SOFTMAX>(l);
    return vec_by_tpr<bf16, KS_OP_SOFTMAX>(l);
}

}  // namespace ks
