// Vector-path kernels for float16, out-of-place RMSNorm(x + residual) * w.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f16_residual(const Launch &l) { return vec_by_tpr<f16, KS_OP_RMS_NORM_RESIDUAL>(l); }

}  // namespace ks
