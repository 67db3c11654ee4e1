// Generic-path kernels for bfloat16, both operations.
#include "ks_launch.hpp"

namespace ks {

hipError_t launch_generic_bf16(const Launch &l)
{
    return l.fused ? launch_generic_typed<bf16, true>(l) : launch_generic_typed<bf16, false>(l);
}

}  // namespace ks
