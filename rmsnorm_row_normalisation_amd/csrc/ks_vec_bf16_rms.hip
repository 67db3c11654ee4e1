// Vector-path kernels for bfloat16, RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_bf16_rms(const Launch &l) { return vec_by_tpr<bf16, KS_OP_RMS_NORM>(l); }

}  // namespace ks
