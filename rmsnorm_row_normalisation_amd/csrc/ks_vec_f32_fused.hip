// Vector-path kernels for float, fused residual-add RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f32_fused(const Launch &l) { return vec_by_tpr<float, true>(l); }

}  // namespace ks
