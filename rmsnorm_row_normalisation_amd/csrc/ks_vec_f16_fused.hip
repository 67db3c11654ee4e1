// Vector-path kernels for _Float16, fused residual-add RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f16_fused(const Launch &l) { return vec_by_tpr<_Float16, true>(l); }

}  // namespace ks
