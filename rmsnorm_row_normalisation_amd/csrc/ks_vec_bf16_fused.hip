// Vector-path kernels for bfloat16, fused residual-add RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_bf16_fused(const Launch &l) { return vec_by_tpr<bf16, true>(l); }

}  // namespace ks
