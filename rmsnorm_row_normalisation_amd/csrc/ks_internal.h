// Host-side declarations shared by the C-ABI layer and the per-dtype kernel
// translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "ks_norm.h"

namespace ks {

// Everything one launch of a row operation needs (softmax uses y = out and x
// only).  `plan` has been validated against the buffers (plan_fits in
// ks_api.cpp) before a launch function sees it.
struct Launch {
    void *y;
    const void *x;
    void *res;
    const void *w;
    int64_t rows;
    int32_t hidden;
    float eps;
    ks_op_t op;         // KS_OP_RMS_NORM, KS_OP_FUSED_ADD_RMS_NORM, KS_OP_RMS_NORM_RESIDUAL or KS_OP_SOFTMAX
    ks_plan_t plan;
    hipStream_t stream;
    float *work = nullptr;   // split softmax: the caller's workspace (split_workspace_floats)
};

// One SwiGLU launch (out [rows, d], x [rows, 2 d]).
struct SwigluLaunch {
    void *out;
    const void *x;
    int64_t rows;
    int32_t d;
    ks_plan_t plan;
    hipStream_t stream;
};

// One RMSNorm backward call (dx, and dw unless dw is null).  `work` is the
// caller's fp32 workspace (see bwd_workspace_floats).
struct BwdLaunch {
    void *dx;
    void *dw;
    const void *dy;
    const void *x;
    const void *w;
    float *work;
    int64_t rows;
    int32_t hidden;
    float eps;
    ks_plan_t plan;
    hipStream_t stream;
};

// Backward: at most this many fp32 partial rows of dw (vector path: one per
// workgroup; generic path: one per chunk of rows).  The vector path runs
// 1024- or 512-thread workgroups, where x, dy, the next group's x and dy, the
// weight and the dw sums of a lane's pieces stay in VGPRs: with 1024 threads
// (128 VGPRs per lane) at most 3 pieces per lane for fp32 and 2 for 16-bit
// dtypes (whose pieces hold 8 sums each), one more spills; with 512 threads
// (256 VGPRs per lane) up to 4 pieces for every dtype.
constexpr int kBwdMaxParts = 256;
// Partial-row arrays of at least this many bytes are written and read
// non-temporal: from 2 MiB (a 2048-wide row's 256 partial rows) a graph-timed
// sweep of bf16 and fp32, 1024..8192 wide, 64..2048 rows, measured 0..19%
// faster calls; below it, plain stores and loads were 3..5% faster (the
// column sum then finds the rows in the caches).
constexpr int64_t kBwdPartNtBytes = 2 << 20;
constexpr int kBwdBlock = 1024;
constexpr int kBwdBlockHalf = 512;
constexpr int kBwdMaxVpt32 = 3;
constexpr int kBwdMaxVpt16 = 2;
constexpr int kBwdMaxVptHalf = 4;
inline int bwd_max_vpt(int elem_bytes, int block = kBwdBlock)
{
    return block == kBwdBlockHalf ? kBwdMaxVptHalf : elem_bytes == 4 ? kBwdMaxVpt32 : kBwdMaxVpt16;
}

// fp32 elements of workspace a backward call needs: the partial rows and, on
// the generic path, one rho per row.
inline int64_t bwd_workspace_floats(int64_t rows, int64_t hidden)
{
    const int64_t parts = rows < kBwdMaxParts ? rows : kBwdMaxParts;
    return parts * hidden + rows;
}

// Work-items one launch of a row kernel may hold (its grid counts work-items
// in 32 bits); the launch code covers larger batches in slices of rows.
constexpr int64_t kMaxLaunchItems = int64_t(1) << 31;

// Cache-policy bits of a buffer instruction that marks it non-temporal.
constexpr int kNonTemporal = 2;

// Launch the kernel the plan names, one function per path, dtype and op (each
// in its own translation unit so they compile in parallel).  Return
// hipErrorInvalidValue when no kernel was compiled for the plan (plan_fits
// rules that out before a launch).
#define KS_DECLARE_LAUNCH(dt)                             \
    hipError_t launch_vec_##dt##_rms(const Launch &l);      \
    hipError_t launch_vec_##dt##_fused(const Launch &l);    \
    hipError_t launch_vec_##dt##_residual(const Launch &l); \
    hipError_t launch_generic_##dt(const Launch &l);
KS_DECLARE_LAUNCH(f32)
KS_DECLARE_LAUNCH(f16)
KS_DECLARE_LAUNCH(bf16)
#undef KS_DECLARE_LAUNCH
hipError_t launch_swiglu_f32(const SwigluLaunch &l);
hipError_t launch_swiglu_f16(const SwigluLaunch &l);
hipError_t launch_swiglu_bf16(const SwigluLaunch &l);
hipError_t launch_bwd_f32(const BwdLaunch &l);
hipError_t launch_bwd_f16(const BwdLaunch &l);
hipError_t launch_bwd_bf16(const BwdLaunch &l);
hipError_t launch_softmax_f32(const Launch &l);
hipError_t launch_softmax_f16(const Launch &l);
hipError_t launch_softmax_bf16(const Launch &l);

// Split softmax plans: 256-lane workgroups, each over one chunk of
// 256 * vectors_per_thread 16-byte pieces of one row (grid: chunks x rows,
// so at most 65535 rows); the workspace holds an fp32 (maximum, sum) pair per
// chunk.
constexpr int kSplitBlock = 256;
constexpr int64_t kSplitMaxRows = 65535;
inline int64_t split_chunks(int64_t row_bytes, int vpt)
{
    const int64_t pieces = row_bytes / 16;
    const int64_t per_chunk = (int64_t)kSplitBlock * vpt;
    return (pieces + per_chunk - 1) / per_chunk;
}
inline int64_t split_workspace_floats(int64_t rows, int64_t row_bytes, int vpt)
{
    return rows * split_chunks(row_bytes, vpt) * 2;
}

// A pending request for per-call kernel timing (ks_time_next_call): the
// runtime's kernel-dispatch events for the calling thread's next call.  The
// launch code attaches `start` to the call's first kernel and `stop` to every
// kernel of the call (the last record stands); the entry point clears the
// request when it returns.
struct TimingRequest {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
TimingRequest &timing_request();   // the calling thread's request (ks_api.cpp)

// Compute units of the current device, queried once per device and cached
// (ks_device_info.cpp); 0 when no device is visible.  The launch policy scales
// its batch-size thresholds with it; kDefaultComputeUnits (a whole MI355X)
// stands in when it is unknown.
int device_compute_units();
constexpr int kDefaultComputeUnits = 256;
constexpr int kMaxComputeUnits = 4096;

// ks_api.cpp: the pre-HIP checks of ks_softmax_ws and the workspace bytes of
// its plan for these buffers; the per-thread HIP error behind KS_ERROR_HIP.
ks_status_t softmax_ws_need(const void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                            size_t *need);
void record_hip_error(int err);

// The one generic SwiGLU plan: a grid-stride loop over elements.
constexpr int kSwigluGenericBlock = 256;

// Vector path limits: threads per row 8..1024 (powers of two), vectors per
// thread 1..8, so rows of up to 128 KiB.  A 1024-thread workgroup leaves 128
// VGPRs per lane; the forward kernels use at most 122 at 8 pieces (the
// out-of-place residual form spills 8 at exactly 7 pieces and 1024 lanes, so
// the policy gives it 8 pieces there).
constexpr int kMinTpr = 8;
constexpr int kMaxTpr = 1024;
constexpr int kMaxVpt = 8;
// Besides 1..kMaxVpt, RMSNorm and its two residual forms compile 16 pieces
// per lane for teams of 32..128 lanes: a 16 KiB row on one wave (fp32 4096,
// 16-bit 8192 wide) instead of two joined by an LDS exchange and a barrier.
constexpr int kWideVpt = 16;
constexpr bool wide_vpt_compiled(int op, int tpr)
{
    return op != KS_OP_SOFTMAX && op != KS_OP_SILU_AND_MUL && op != KS_OP_RMS_NORM_BACKWARD && tpr >= 32 &&
           tpr <= 128;
}

inline int block_threads_for(int tpr) { return tpr < 256 ? 256 : tpr; }

}  // namespace ks
