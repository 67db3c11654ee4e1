// Generic-path kernels for bfloat16, the three normalisation operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_bf16(const Launch &l)
{
    switch (l.op) {
    case KS_OP_FUSED_ADD_RMS_NORM: return launch_generic_typed<bf16, KS_OP_FUSED_ADD_RMS_NORM>(l);
    case KS_OP_RMS_NORM_RESIDUAL: return launch_generic_typed<bf16, KS_OP_RMS_NORM_RESIDUAL>(l);
    default: return launch_generic_typed<bf16, KS_OP_RMS_NORM>(l);
    }
}

}  // namespace ks
