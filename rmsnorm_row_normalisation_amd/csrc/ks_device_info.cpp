// Device properties the launch policy reads: the current device's compute
// units, queried once per device (hipDeviceGetAttribute) and cached for the
// life of the process.
#include <atomic>

#include <hip/hip_runtime_api.h>

#include "ks_internal.h"

namespace {

constexpr int kMaxDevices = 256;
std::atomic<int> g_cus[kMaxDevices];   // 0: not queried yet

}  // namespace

namespace ks {

int device_compute_units()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 0;
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus > 0)
        return cus;
    // concurrent first calls on one device may both query; they store the same value
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    if (cus > kMaxComputeUnits)
        cus = kMaxComputeUnits;
    g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace ks
