// Host-side dispatch from a plan to a compiled kernel, for one dtype.  Each
// per-dtype translation unit includes this once and defines its launch_*.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "ks_device.hpp"
#include "ks_internal.h"

namespace ks {

// Launch one kernel on `stream`.  With a timing request pending
// (ks_time_next_call) the launch goes through the runtime's kernel-dispatch
// events: the start event marks the beginning of the call's first kernel,
// the stop event the end of each kernel (so of the last one).
template <typename Kernel, typename... Args>
hipError_t dispatch(Kernel kernel, dim3 grid, dim3 block, size_t lds_bytes, hipStream_t stream, Args... args)
{
    TimingRequest &t = timing_request();
    if (t.start == nullptr && t.stop == nullptr) {
        hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
    } else {
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds_bytes, stream, t.start, t.stop, 0u, args...);
        t.start = nullptr;
    }
    return hipGetLastError();
}

// A kernel launch with the fields of its parameter struct as the kernel's
// scalar arguments (the kernel entry points rebuild the struct; scalar
// arguments are preloaded into SGPRs at wave launch, up to 14 SGPRs).
template <typename Kernel>
hipError_t dispatch_fields(Kernel k, dim3 g, dim3 b, size_t lds, hipStream_t s, const Params &p)
{
    return dispatch(k, g, b, lds, s, p.y, p.x, p.res, p.w, p.rows, p.hidden, p.eps);
}
template <typename Kernel>
hipError_t dispatch_fields(Kernel k, dim3 g, dim3 b, size_t lds, hipStream_t s, const SwigluParams &p)
{
    return dispatch(k, g, b, lds, s, p.out, p.x, p.rows, p.d);
}
template <typename Kernel>
hipError_t dispatch_fields(Kernel k, dim3 g, dim3 b, size_t lds, hipStream_t s, const SplitParams &p)
{
    return dispatch(k, g, b, lds, s, p.y, p.x, p.stats, p.rows, p.hidden, p.chunks);
}
template <typename Kernel>
hipError_t dispatch_fields(Kernel k, dim3 g, dim3 b, size_t lds, hipStream_t s, const BwdParams &p)
{
    // the sizes before the partial-row pointers: 14 SGPRs of arguments are
    // preloaded, and the sizes are needed before the first load, the
    // pointers only at the end
    return dispatch(k, g, b, lds, s, p.dx, p.dy, p.x, p.w, p.rows, p.hidden, p.eps, p.part, p.rho, p.part_nt);
}
template <typename Kernel>
hipError_t dispatch_fields(Kernel k, dim3 g, dim3 b, size_t lds, hipStream_t s, const DwParams &p)
{
    return dispatch(k, g, b, lds, s, p.dw, p.part, p.nparts, p.hidden);
}

// Rows one launch of a row kernel may cover: its grid stays within 2^31
// work-items (a dispatch counts work-items in 32 bits); larger batches go out
// in consecutive slices of rows, each a launch of the same kernel.
inline int64_t rows_per_launch(int64_t rows_per_block, int block)
{
    return (kMaxLaunchItems / block) * rows_per_block;
}

template <typename T, typename Kernel>
hipError_t run(Kernel kernel, const Launch &l, int block, size_t lds_bytes = 0)
{
    const int64_t rpb = block / l.plan.threads_per_row;
    const int64_t slice = rows_per_launch(rpb, block);
    const size_t row_bytes = (size_t)l.hidden * Pack<T>::kBytes;
    for (int64_t r0 = 0; r0 < l.rows; r0 += slice) {
        const int64_t n = l.rows - r0 < slice ? l.rows - r0 : slice;
        const size_t off = (size_t)r0 * row_bytes;
        Params p{(char *)l.y + off, (const char *)l.x + off, l.res ? (char *)l.res + off : nullptr, l.w, n,
                 l.hidden, l.eps};
        const hipError_t err =
            dispatch_fields(kernel, dim3((unsigned)((n + rpb - 1) / rpb)), dim3(block), lds_bytes, l.stream, p);
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

// The kernel entry point of one op (OP is a ks_op_t: RMSNorm, fused in place,
// out-of-place residual, or softmax).
template <int OP, typename T, int TPR, int V, int B, int LC, int SC, bool WL>
constexpr auto vec_entry()
{
    if constexpr (OP == KS_OP_FUSED_ADD_RMS_NORM)
        return fused_add_rms_norm_vec<T, TPR, V, B, LC, SC, WL>;
    else if constexpr (OP == KS_OP_RMS_NORM_RESIDUAL)
        return rms_norm_residual_vec<T, TPR, V, B, LC, SC, WL>;
    else if constexpr (OP == KS_OP_SOFTMAX)
        return softmax_vec<T, TPR, V, B, LC, SC>;
    else
        return rms_norm_vec<T, TPR, V, B, LC, SC, WL>;
}

template <int OP, typename T, int TPR, int EPA, int B>
constexpr auto generic_entry()
{
    if constexpr (OP == KS_OP_FUSED_ADD_RMS_NORM)
        return fused_add_rms_norm_generic<T, TPR, EPA, B>;
    else if constexpr (OP == KS_OP_RMS_NORM_RESIDUAL)
        return rms_norm_residual_generic<T, TPR, EPA, B>;
    else if constexpr (OP == KS_OP_SOFTMAX)
        return softmax_generic<T, TPR, EPA, B>;
    else
        return rms_norm_generic<T, TPR, EPA, B>;
}

// The compiled memory-hint variants of one launch shape (softmax has no
// weight, so no LDS-staged variant).
template <typename T, int OP, int TPR, int V>
hipError_t vec_one(const Launch &l)
{
    constexpr int B = TPR < 256 ? 256 : TPR;
    constexpr int NT = kNonTemporal;
    const ks_plan_t &p = l.plan;
    if (!p.load_nt && !p.store_nt && !p.weight_lds)
        return run<T>(vec_entry<OP, T, TPR, V, B, 0, 0, false>(), l, B);
    if (p.load_nt && p.store_nt && !p.weight_lds)
        return run<T>(vec_entry<OP, T, TPR, V, B, NT, NT, false>(), l, B);
    if (!p.load_nt && p.store_nt && !p.weight_lds)
        return run<T>(vec_entry<OP, T, TPR, V, B, 0, NT, false>(), l, B);
    if constexpr (OP != KS_OP_SOFTMAX) {
        if (p.load_nt && p.store_nt && p.weight_lds)
            return run<T>(vec_entry<OP, T, TPR, V, B, NT, NT, true>(), l, B, (size_t)V * TPR * 16);
    }
    return hipErrorInvalidValue;
}

template <typename T, int OP, int TPR>
hipError_t vec_by_vpt(const Launch &l)
{
    switch (l.plan.vectors_per_thread) {
    case 1: return vec_one<T, OP, TPR, 1>(l);
    case 2: return vec_one<T, OP, TPR, 2>(l);
    case 3: return vec_one<T, OP, TPR, 3>(l);
    case 4: return vec_one<T, OP, TPR, 4>(l);
    case 5: return vec_one<T, OP, TPR, 5>(l);
    case 6: return vec_one<T, OP, TPR, 6>(l);
    case 7: return vec_one<T, OP, TPR, 7>(l);
    case 8: return vec_one<T, OP, TPR, 8>(l);
    case kWideVpt:
        if constexpr (wide_vpt_compiled(OP, TPR))
            return vec_one<T, OP, TPR, kWideVpt>(l);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int OP>
hipError_t vec_by_tpr(const Launch &l)
{
    switch (l.plan.threads_per_row) {
    case 8: return vec_by_vpt<T, OP, 8>(l);
    case 16: return vec_by_vpt<T, OP, 16>(l);
    case 32: return vec_by_vpt<T, OP, 32>(l);
    case 64: return vec_by_vpt<T, OP, 64>(l);
    case 128: return vec_by_vpt<T, OP, 128>(l);
    case 256: return vec_by_vpt<T, OP, 256>(l);
    case 512: return vec_by_vpt<T, OP, 512>(l);
    case 1024: return vec_by_vpt<T, OP, 1024>(l);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int OP, int EPA>
hipError_t generic_by_tpr(const Launch &l)
{
    switch (l.plan.threads_per_row) {
    case 8: return run<T>(generic_entry<OP, T, 8, EPA, 256>(), l, 256);
    case 64: return run<T>(generic_entry<OP, T, 64, EPA, 256>(), l, 256);
    case 256: return run<T>(generic_entry<OP, T, 256, EPA, 256>(), l, 256);
    case 1024: return run<T>(generic_entry<OP, T, 1024, EPA, 1024>(), l, 1024);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int OP>
hipError_t launch_generic_typed(const Launch &l)
{
    constexpr int kVecElems = Pack<T>::kElems;
    if (l.plan.elems_per_access == 1)
        return generic_by_tpr<T, OP, 1>(l);
    if (l.plan.elems_per_access == kVecElems)
        return generic_by_tpr<T, OP, kVecElems>(l);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Split-row softmax: the statistics kernel, then the normalising kernel, on
// one stream (the second reads what the first wrote).
// ---------------------------------------------------------------------------
template <typename T, int V>
hipError_t softmax_split_one(const Launch &l)
{
    const int64_t chunks = split_chunks((int64_t)l.hidden * Pack<T>::kBytes, V);
    SplitParams p{l.y, l.x, l.work, l.rows, l.hidden, (int32_t)chunks};
    const dim3 grid((unsigned)chunks, (unsigned)l.rows);
    const hipError_t err = dispatch_fields(softmax_split_stats<T, V>, grid, dim3(kSplitBlock), 0, l.stream, p);
    if (err != hipSuccess)
        return err;
    return dispatch_fields(softmax_split_norm<T, V>, grid, dim3(kSplitBlock), 0, l.stream, p);
}

template <typename T>
hipError_t launch_softmax_typed(const Launch &l)
{
    if (l.plan.path == KS_PATH_GENERIC)
        return launch_generic_typed<T, KS_OP_SOFTMAX>(l);
    if (l.plan.path == KS_PATH_SPLIT) {
        switch (l.plan.vectors_per_thread) {
        case 1: return softmax_split_one<T, 1>(l);
        case 2: return softmax_split_one<T, 2>(l);
        case 4: return softmax_split_one<T, 4>(l);
        default: return hipErrorInvalidValue;
        }
    }
    return vec_by_tpr<T, KS_OP_SOFTMAX>(l);
}

// ---------------------------------------------------------------------------
// SwiGLU
// ---------------------------------------------------------------------------
template <typename T, typename Kernel>
hipError_t run_swiglu(Kernel kernel, const SwigluLaunch &l, int block)
{
    const int64_t rpb = block / l.plan.threads_per_row;
    const int64_t slice = rows_per_launch(rpb, block);
    const size_t out_bytes = (size_t)l.d * Pack<T>::kBytes;   // per row; x rows are twice as long
    for (int64_t r0 = 0; r0 < l.rows; r0 += slice) {
        const int64_t n = l.rows - r0 < slice ? l.rows - r0 : slice;
        SwigluParams p{(char *)l.out + (size_t)r0 * out_bytes, (const char *)l.x + (size_t)r0 * 2 * out_bytes, n,
                       l.d};
        const hipError_t err = dispatch_fields(kernel, dim3((unsigned)((n + rpb - 1) / rpb)), dim3(block), 0, l.stream, p);
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

template <typename T, int TPR, int V>
hipError_t swiglu_one(const SwigluLaunch &l)
{
    constexpr int B = TPR < 256 ? 256 : TPR;
    constexpr int NT = kNonTemporal;
    const ks_plan_t &p = l.plan;
    if (!p.load_nt && !p.store_nt)
        return run_swiglu<T>(silu_and_mul_vec<T, TPR, V, B, 0, 0>, l, B);
    if (p.load_nt && p.store_nt)
        return run_swiglu<T>(silu_and_mul_vec<T, TPR, V, B, NT, NT>, l, B);
    if (!p.load_nt && p.store_nt)
        return run_swiglu<T>(silu_and_mul_vec<T, TPR, V, B, 0, NT>, l, B);
    return hipErrorInvalidValue;
}

template <typename T, int TPR>
hipError_t swiglu_by_vpt(const SwigluLaunch &l)
{
    switch (l.plan.vectors_per_thread) {
    case 1: return swiglu_one<T, TPR, 1>(l);
    case 2: return swiglu_one<T, TPR, 2>(l);
    case 3: return swiglu_one<T, TPR, 3>(l);
    case 4: return swiglu_one<T, TPR, 4>(l);
    case 5: return swiglu_one<T, TPR, 5>(l);
    case 6: return swiglu_one<T, TPR, 6>(l);
    case 7: return swiglu_one<T, TPR, 7>(l);
    case 8: return swiglu_one<T, TPR, 8>(l);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_swiglu_typed(const SwigluLaunch &l)
{
    if (l.plan.path == KS_PATH_GENERIC) {
        SwigluParams p{l.out, l.x, l.rows, l.d};
        const int64_t total = l.rows * (int64_t)l.d;
        int64_t blocks = (total + kSwigluGenericBlock - 1) / kSwigluGenericBlock;
        blocks = blocks > 8192 ? 8192 : blocks;   // grid-stride beyond 2M threads
        return dispatch_fields(silu_and_mul_generic<T>, dim3((unsigned)blocks), dim3(kSwigluGenericBlock), 0, l.stream, p);
    }
    switch (l.plan.threads_per_row) {
    case 8: return swiglu_by_vpt<T, 8>(l);
    case 16: return swiglu_by_vpt<T, 16>(l);
    case 32: return swiglu_by_vpt<T, 32>(l);
    case 64: return swiglu_by_vpt<T, 64>(l);
    case 128: return swiglu_by_vpt<T, 128>(l);
    case 256: return swiglu_by_vpt<T, 256>(l);
    case 512: return swiglu_by_vpt<T, 512>(l);
    case 1024: return swiglu_by_vpt<T, 1024>(l);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// RMSNorm backward
// ---------------------------------------------------------------------------
template <typename T, int TPR, int V, int B>
hipError_t bwd_vec_one(const BwdParams &p, unsigned grid, hipStream_t stream)
{
    return dispatch_fields(rms_norm_backward_vec<T, TPR, V, B>, dim3(grid), dim3(B), 0, stream, p);
}

// The compiled backward plans: 1024-thread workgroups with 1..3 (fp32) or 1..2
// pieces per lane, 512-thread workgroups (teams up to 512 lanes) with 1..4.
template <typename T, int TPR>
hipError_t bwd_vec_by_vpt(const BwdParams &p, int vpt, int block, unsigned grid, hipStream_t stream)
{
    if (block == kBwdBlockHalf) {
        if constexpr (TPR <= kBwdBlockHalf) {
            switch (vpt) {
            case 1: return bwd_vec_one<T, TPR, 1, kBwdBlockHalf>(p, grid, stream);
            case 2: return bwd_vec_one<T, TPR, 2, kBwdBlockHalf>(p, grid, stream);
            case 3: return bwd_vec_one<T, TPR, 3, kBwdBlockHalf>(p, grid, stream);
            case 4: return bwd_vec_one<T, TPR, 4, kBwdBlockHalf>(p, grid, stream);
            default: break;
            }
        }
        return hipErrorInvalidValue;
    }
    if (block != kBwdBlock)
        return hipErrorInvalidValue;
    switch (vpt) {
    case 1: return bwd_vec_one<T, TPR, 1, kBwdBlock>(p, grid, stream);
    case 2: return bwd_vec_one<T, TPR, 2, kBwdBlock>(p, grid, stream);
    default: break;
    }
    if constexpr (Pack<T>::kBytes == 4) {
        if (vpt == 3)
            return bwd_vec_one<T, TPR, 3, kBwdBlock>(p, grid, stream);
    }
    return hipErrorInvalidValue;
}

// Generic plans: 256-thread workgroups, 1024 for 1024-lane teams.
template <typename T, int TPR, int EPA>
hipError_t bwd_generic_one(const BwdParams &p, unsigned grid, hipStream_t stream)
{
    constexpr int B = TPR == 1024 ? 1024 : 256;
    return dispatch_fields(rms_norm_backward_generic<T, TPR, EPA, B>, dim3(grid), dim3(B), 0, stream, p);
}

template <typename T, int EPA>
hipError_t bwd_generic_by_tpr(const BwdParams &p, int tpr, unsigned grid, hipStream_t stream)
{
    switch (tpr) {
    case 8: return bwd_generic_one<T, 8, EPA>(p, grid, stream);
    case 64: return bwd_generic_one<T, 64, EPA>(p, grid, stream);
    case 256: return bwd_generic_one<T, 256, EPA>(p, grid, stream);
    case 1024: return bwd_generic_one<T, 1024, EPA>(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

// Whether nparts fp32 partial rows of dw are written and read non-temporal.
inline int32_t part_nt(int64_t nparts, int64_t hidden)
{
    return nparts * hidden * (int64_t)sizeof(float) >= kBwdPartNtBytes ? 1 : 0;
}

template <typename T>
hipError_t launch_bwd_typed(const BwdLaunch &l)
{
    const ks_plan_t &pl = l.plan;
    const int64_t rpb = pl.block_threads / pl.threads_per_row;
    int32_t nparts = 0;
    hipError_t err = hipSuccess;
    if (l.rows > 0) {
        BwdParams p{l.dx, l.dy, l.x, l.w, l.dw ? l.work : nullptr, nullptr, l.rows, l.hidden, l.eps, 0};
        if (pl.path == KS_PATH_VECTOR) {
            const int64_t groups = (l.rows + rpb - 1) / rpb;
            const unsigned grid = (unsigned)(groups < kBwdMaxParts ? groups : kBwdMaxParts);
            nparts = (int32_t)grid;
            p.part_nt = part_nt(nparts, l.hidden);
            switch (pl.threads_per_row) {
            case 8: err = bwd_vec_by_vpt<T, 8>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            case 16: err = bwd_vec_by_vpt<T, 16>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            case 32: err = bwd_vec_by_vpt<T, 32>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            case 64: err = bwd_vec_by_vpt<T, 64>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            case 128: err = bwd_vec_by_vpt<T, 128>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            case 256: err = bwd_vec_by_vpt<T, 256>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            case 512: err = bwd_vec_by_vpt<T, 512>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            case 1024: err = bwd_vec_by_vpt<T, 1024>(p, pl.vectors_per_thread, pl.block_threads, grid, l.stream); break;
            default: return hipErrorInvalidValue;
            }
        } else {
            nparts = (int32_t)(l.rows < kBwdMaxParts ? l.rows : kBwdMaxParts);
            p.part_nt = part_nt(nparts, l.hidden);
            if (l.dw)
                p.rho = l.work + (size_t)nparts * (size_t)l.hidden;
            if (pl.elems_per_access != 1 && pl.elems_per_access != Pack<T>::kElems)
                return hipErrorInvalidValue;
            const int64_t slice = rows_per_launch(rpb, pl.block_threads);
            const size_t row_bytes = (size_t)l.hidden * Pack<T>::kBytes;
            for (int64_t r0 = 0; r0 < l.rows && err == hipSuccess; r0 += slice) {
                const int64_t n = l.rows - r0 < slice ? l.rows - r0 : slice;
                const size_t off = (size_t)r0 * row_bytes;
                BwdParams ps = p;
                ps.dx = (char *)p.dx + off;
                ps.dy = (const char *)p.dy + off;
                ps.x = (const char *)p.x + off;
                ps.rho = p.rho ? p.rho + r0 : nullptr;
                ps.rows = n;
                const unsigned grid = (unsigned)((n + rpb - 1) / rpb);
                err = pl.elems_per_access == 1
                          ? bwd_generic_by_tpr<T, 1>(ps, pl.threads_per_row, grid, l.stream)
                          : bwd_generic_by_tpr<T, Pack<T>::kElems>(ps, pl.threads_per_row, grid, l.stream);
            }
            if (err == hipSuccess && l.dw) {
                const dim3 cgrid((unsigned)((l.hidden + 255) / 256), (unsigned)nparts);
                err = dispatch_fields(rms_norm_backward_colsum<T>, cgrid, dim3(256), 0, l.stream, p);
            }
        }
    }
    if (err != hipSuccess || l.dw == nullptr)
        return err;
    DwParams d{l.dw, l.work, nparts, l.hidden};
    const dim3 dgrid((unsigned)((l.hidden + kDwCols - 1) / kDwCols));
    return part_nt(nparts, l.hidden)
               ? dispatch_fields(rms_norm_backward_dw<T, true>, dgrid, dim3(kDwBlock), 0, l.stream, d)
               : dispatch_fields(rms_norm_backward_dw<T, false>, dgrid, dim3(kDwBlock), 0, l.stream, d);
}

}  // namespace ks
