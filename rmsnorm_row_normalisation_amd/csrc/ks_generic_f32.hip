// Generic-path kernels for float32, both operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_f32(const Launch &l)
{
    return l.op == KS_OP_FUSED_ADD_RMS_NORM ? launch_generic_typed<f32, KS_OP_FUSED_ADD_RMS_NORM>(l)
                                           : launch_generic_typed<f32, KS_OP_RMS_NORM>(l);
}

}  // namespace ks
