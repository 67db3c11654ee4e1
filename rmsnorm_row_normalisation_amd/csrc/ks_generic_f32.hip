// Generic-path kernels for float32, both operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_f32(const Launch &l)
{
    return l.fused ? launch_generic_typed<f32, true>(l) : launch_generic_typed<f32, false>(l);
}

}  // namespace ks
