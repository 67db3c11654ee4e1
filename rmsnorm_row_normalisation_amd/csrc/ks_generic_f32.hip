// Generic-path kernels for float, both operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_f32(const Launch &l)
{
    return l.fused ? launch_generic_typed<float, true>(l) : launch_generic_typed<float, false>(l);
}

}  // namespace ks
