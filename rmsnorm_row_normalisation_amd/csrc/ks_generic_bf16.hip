// Generic-path kernels for bfloat16, both operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_bf16(const Launch &l)
{
    return l.op == KS_OP_FUSED_ADD_RMS_NORM ? launch_generic_typed<bf16, KS_OP_FUSED_ADD_RMS_NORM>(l)
                                           : launch_generic_typed<bf16, KS_OP_RMS_NORM>(l);
}

}  // namespace ks
