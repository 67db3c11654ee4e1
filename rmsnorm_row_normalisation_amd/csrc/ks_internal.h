// Host-side declarations shared by the C-ABI layer and the per-dtype kernel
// translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "ks_norm.h"

namespace ks {

// Everything one launch needs.  `plan` has been validated against the
// buffers (see plan_fits in ks_api.cpp) before a launch function sees it.
struct Launch {
    void *y;
    const void *x;
    void *res;
    const void *w;
    int64_t rows;
    int32_t hidden;
    float eps;
    bool fused;
    ks_plan_t plan;
    hipEvent_t start;
    hipEvent_t stop;
    hipStream_t stream;
};

// Cache-policy bits for the streamed (x, residual, out) buffer accesses.
// 0 = default; 2 = non-temporal.  Weight accesses always use the default.
constexpr int kStreamCpol = 0;

// Launch the kernel the plan names for one dtype.  Returns hipErrorInvalidValue
// when no kernel was compiled for the plan (plan_fits rules that out).
hipError_t launch_f32(const Launch &l);
hipError_t launch_f16(const Launch &l);
hipError_t launch_bf16(const Launch &l);

// Vector path limits: threads per row 8..1024 (powers of two), vectors per
// thread 1..8 (1..4 when a row spans 1024 threads, to stay within the VGPR
// budget of a 1024-thread workgroup).
constexpr int kMinTpr = 8;
constexpr int kMaxTpr = 1024;
constexpr int kMaxVpt = 8;
constexpr int kMaxVptAt1024 = 4;

inline int block_threads_for(int tpr) { return tpr < 256 ? 256 : tpr; }

}  // namespace ks
