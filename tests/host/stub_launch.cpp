// Stand-ins for the kernel launch functions, so that the host side of the C
// ABI (validation, overlap checks, the launch policy, plan checks) can be
// built with the host compiler's sanitizers and driven on a machine without
// a GPU.  Each stand-in only counts the calls that reached it.
#include <stdlib.h>

#include "ks_internal.h"

namespace ks {

long g_launches = 0;

#define KS_STUB(name, arg)                 \
    hipError_t name(const arg &)           \
    {                                      \
        ++g_launches;                      \
        return hipSuccess;                 \
    }

KS_STUB(launch_vec_f32_rms, Launch)
KS_STUB(launch_vec_f32_fused, Launch)
KS_STUB(launch_vec_f32_residual, Launch)
KS_STUB(launch_generic_f32, Launch)
KS_STUB(launch_vec_f16_rms, Launch)
KS_STUB(launch_vec_f16_fused, Launch)
KS_STUB(launch_vec_f16_residual, Launch)
KS_STUB(launch_generic_f16, Launch)
KS_STUB(launch_vec_bf16_rms, Launch)
KS_STUB(launch_vec_bf16_fused, Launch)
KS_STUB(launch_vec_bf16_residual, Launch)
KS_STUB(launch_generic_bf16, Launch)
// Softmax: a split plan must arrive with a workspace.
static hipError_t softmax_stub(const Launch &l)
{
    ++g_launches;
    if (l.plan.path == KS_PATH_SPLIT && l.work == nullptr)
        abort();
    return hipSuccess;
}
hipError_t launch_softmax_f32(const Launch &l) { return softmax_stub(l); }
hipError_t launch_softmax_f16(const Launch &l) { return softmax_stub(l); }
hipError_t launch_softmax_bf16(const Launch &l) { return softmax_stub(l); }
KS_STUB(launch_swiglu_f32, SwigluLaunch)
KS_STUB(launch_swiglu_f16, SwigluLaunch)
KS_STUB(launch_swiglu_bf16, SwigluLaunch)
KS_STUB(launch_bwd_f32, BwdLaunch)
KS_STUB(launch_bwd_f16, BwdLaunch)
KS_STUB(launch_bwd_bf16, BwdLaunch)

}  // namespace ks
