// Vector-path kernels for float32, out-of-place RMSNorm(x + residual) * w.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f32_residual(const Launch &l) { return vec_by_tpr<f32, KS_OP_RMS_NORM_RESIDUAL>(l); }

}  // namespace ks
