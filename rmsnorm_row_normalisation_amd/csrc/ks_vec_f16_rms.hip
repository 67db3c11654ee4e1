// Vector-path kernels for _Float16, RMSNorm.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_vec_f16_rms(const Launch &l) { return vec_by_tpr<_Float16, false>(l); }

}  // namespace ks
