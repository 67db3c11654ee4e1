// Vector-path kernels for float32, fused residual-add RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f32_fused(const Launch &l) { return vec_by_tpr<f32, KS_OP_FUSED_ADD_RMS_NORM>(l); }

}  // namespace ks
