// Generic-path kernels for float16, both operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_f16(const Launch &l)
{
    return l.fused ? launch_generic_typed<f16, true>(l) : launch_generic_typed<f16, false>(l);
}

}  // namespace ks
