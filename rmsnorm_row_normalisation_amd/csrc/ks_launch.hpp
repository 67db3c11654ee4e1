// Host-side dispatch from a plan to a compiled kernel, for one dtype.  Each
// per-dtype translation unit includes this once and defines its launch_*.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "ks_device.hpp"
#include "ks_internal.h"

namespace ks {

template <typename Kernel>
hipError_t run(Kernel kernel, const Launch &l, int block)
{
    Params p{l.y, l.x, l.res, l.w, l.rows, l.hidden, l.eps};
    const int64_t rpb = block / l.plan.threads_per_row;
    const dim3 grid((unsigned)((l.rows + rpb - 1) / rpb));
    if (l.start != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, dim3(block), 0, l.stream, l.start, l.stop, 0, p);
    else
        hipLaunchKernelGGL(kernel, grid, dim3(block), 0, l.stream, p);
    return hipGetLastError();
}

template <typename T, bool F, int TPR>
hipError_t vec_by_vpt(const Launch &l)
{
    constexpr int B = TPR < 256 ? 256 : TPR;
    constexpr int C = kStreamCpol;
    switch (l.plan.vectors_per_thread) {
    case 1: return run(vec_kernel<T, F, TPR, 1, B, C>, l, B);
    case 2: return run(vec_kernel<T, F, TPR, 2, B, C>, l, B);
    case 3: return run(vec_kernel<T, F, TPR, 3, B, C>, l, B);
    case 4: return run(vec_kernel<T, F, TPR, 4, B, C>, l, B);
    default: break;
    }
    if constexpr (TPR < kMaxTpr) {
        switch (l.plan.vectors_per_thread) {
        case 5: return run(vec_kernel<T, F, TPR, 5, B, C>, l, B);
        case 6: return run(vec_kernel<T, F, TPR, 6, B, C>, l, B);
        case 7: return run(vec_kernel<T, F, TPR, 7, B, C>, l, B);
        case 8: return run(vec_kernel<T, F, TPR, 8, B, C>, l, B);
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <typename T, bool F>
hipError_t vec_by_tpr(const Launch &l)
{
    switch (l.plan.threads_per_row) {
    case 8: return vec_by_vpt<T, F, 8>(l);
    case 16: return vec_by_vpt<T, F, 16>(l);
    case 32: return vec_by_vpt<T, F, 32>(l);
    case 64: return vec_by_vpt<T, F, 64>(l);
    case 128: return vec_by_vpt<T, F, 128>(l);
    case 256: return vec_by_vpt<T, F, 256>(l);
    case 512: return vec_by_vpt<T, F, 512>(l);
    case 1024: return vec_by_vpt<T, F, 1024>(l);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, bool F, int EPA>
hipError_t generic_by_tpr(const Launch &l)
{
    switch (l.plan.threads_per_row) {
    case 8: return run(generic_kernel<T, F, 8, EPA, 256>, l, 256);
    case 64: return run(generic_kernel<T, F, 64, EPA, 256>, l, 256);
    case 256: return run(generic_kernel<T, F, 256, EPA, 256>, l, 256);
    case 1024: return run(generic_kernel<T, F, 1024, EPA, 1024>, l, 1024);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_typed(const Launch &l)
{
    constexpr int kVecElems = Pack<T>::kElems;
    if (l.plan.path == KS_PATH_VECTOR)
        return l.fused ? vec_by_tpr<T, true>(l) : vec_by_tpr<T, false>(l);
    if (l.plan.path == KS_PATH_GENERIC) {
        if (l.plan.elems_per_access == 1)
            return l.fused ? generic_by_tpr<T, true, 1>(l) : generic_by_tpr<T, false, 1>(l);
        if (l.plan.elems_per_access == kVecElems)
            return l.fused ? generic_by_tpr<T, true, kVecElems>(l) : generic_by_tpr<T, false, kVecElems>(l);
    }
    return hipErrorInvalidValue;
}

}  // namespace ks
