// Vector-path kernels for float32, RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f32_rms(const Launch &l) { return vec_by_tpr<f32, KS_OP_RMS_NORM>(l); }

}  // namespace ks
