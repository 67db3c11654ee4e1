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

// The RMSNorm forms: an accepted plan names a compiled shape (one row per
// team, so rows_per_block is the workgroup's team count).
static hipError_t vec_stub(const Launch &l)
{
    ++g_launches;
    const ks_plan_t &p = l.plan;
    if (p.threads_per_row <= 0 || p.rows_per_block != p.block_threads / p.threads_per_row)
        abort();
    return hipSuccess;
}
#define KS_VEC_STUB(name) \
    hipError_t name(const Launch &l) { return vec_stub(l); }

KS_VEC_STUB(launch_vec_f32_rms)
KS_VEC_STUB(launch_vec_f32_fused)
KS_VEC_STUB(launch_vec_f32_residual)
KS_STUB(launch_generic_f32, Launch)
KS_VEC_STUB(launch_vec_f16_rms)
KS_VEC_STUB(launch_vec_f16_fused)
KS_VEC_STUB(launch_vec_f16_residual)
KS_STUB(launch_generic_f16, Launch)
KS_VEC_STUB(launch_vec_bf16_rms)
KS_VEC_STUB(launch_vec_bf16_fused)
KS_VEC_STUB(launch_vec_bf16_residual)
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
// The backward: an accepted vector plan names a compiled shape (1024-thread
// workgroups with up to 3 (fp32) or 2 pieces per lane, 512-thread ones with up
// to 4, one row per team).
static hipError_t bwd_stub(const BwdLaunch &l, int elem_bytes)
{
    ++g_launches;
    const ks_plan_t &p = l.plan;
    if (p.path == KS_PATH_VECTOR &&
        ((p.block_threads != kBwdBlock && p.block_threads != kBwdBlockHalf) || p.threads_per_row <= 0 ||
         p.threads_per_row > p.block_threads || p.rows_per_block != p.block_threads / p.threads_per_row ||
         p.vectors_per_thread < 1 || p.vectors_per_thread > bwd_max_vpt(elem_bytes, p.block_threads)))
        abort();
    return hipSuccess;
}
hipError_t launch_bwd_f32(const BwdLaunch &l) { return bwd_stub(l, 4); }
hipError_t launch_bwd_f16(const BwdLaunch &l) { return bwd_stub(l, 2); }
hipError_t launch_bwd_bf16(const BwdLaunch &l) { return bwd_stub(l, 2); }

}  // namespace ks

namespace ks {
// The sweep runs without a device: the whole-MI355X compute-unit count.
int device_compute_units() { return kDefaultComputeUnits; }
}  // namespace ks
