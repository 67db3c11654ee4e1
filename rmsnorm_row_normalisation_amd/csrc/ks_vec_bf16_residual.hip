// Vector-path kernels for bfloat16, out-of-place RMSNorm(x + residual) * w.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_bf16_residual(const Launch &l) { return vec_by_tpr<bf16, KS_OP_RMS_NORM_RESIDUAL>(l); }

}  // namespace ks
