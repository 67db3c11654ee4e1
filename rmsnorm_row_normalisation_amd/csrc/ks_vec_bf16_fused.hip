// Vector-path kernels for bfloat16, fused residual-add RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_bf16_fused(const Launch &l) { return vec_by_tpr<bf16, KS_OP_FUSED_ADD_RMS_NORM>(l); }

}  // namespace ks
