// Vector-path kernels for float16, fused residual-add RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f16_fused(const Launch &l) { return vec_by_tpr<f16, KS_OP_FUSED_ADD_RMS_NORM>(l); }

}  // namespace ks
