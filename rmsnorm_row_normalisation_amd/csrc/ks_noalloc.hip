// ks_softmax_noalloc: softmax whose split plans keep their per-chunk
// statistics in a device array the library holds, for callers that cannot
// allocate device memory (graph capture, serving loops, harnesses that forbid
// allocation).  The kernels are the split softmax kernels of ks_softmax_ws;
// only the home of the statistics differs.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "ks_internal.h"
#include "ks_norm.h"

namespace {

// The statistics array: one copy per GPU, at that GPU's own address.  In host
// code `scratch` names a host-side stand-in, never the device memory: host
// code uses only the address hipGetSymbolAddress returns for the current
// device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[KS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device (under a lock, so concurrent first calls look
// it up once) and kept for the rest of the process.
hipError_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess)
                return err;
            if (p == nullptr)
                return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// A timing request (ks_time_next_call) applies to this call alone, also when
// it returns before reaching ks_softmax_ws.
struct ClearTimingOnReturn {
    ~ClearTimingOnReturn() { ks::timing_request() = ks::TimingRequest{}; }
};

}  // namespace

extern "C" ks_status_t ks_softmax_noalloc(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                                          hipStream_t stream)
{
    const ClearTimingOnReturn timing;
    size_t need = 0;
    const ks_status_t st = ks::softmax_ws_need(out, x, rows, hidden, dtype, &need);
    if (st != KS_SUCCESS)
        return st;
    if (need > KS_NOALLOC_SCRATCH_BYTES)
        return KS_ERROR_SCRATCH_LIMIT;
    if (rows == 0)
        return KS_SUCCESS;
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t err = scratch_address(&ws);
        if (err != hipSuccess) {
            ks::record_hip_error((int)err);
            return KS_ERROR_HIP;
        }
    }
    // the same plan, checks and kernels as a call with a caller workspace of
    // the array's size (a one-pass plan gets no workspace and touches none)
    return ks_softmax_ws(out, x, rows, hidden, dtype, ws, need > 0 ? (size_t)KS_NOALLOC_SCRATCH_BYTES : 0, stream);
}
