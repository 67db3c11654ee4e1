// Generic-path kernels for _Float16, both operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_f16(const Launch &l)
{
    return l.fused ? launch_generic_typed<_Float16, true>(l) : launch_generic_typed<_Float16, false>(l);
}

}  // namespace ks
