// Reference HBM streams for the measurements: what a kernel that only reads,
// only writes, or copies reaches on this device, next to which the
// normalisation kernels' bandwidth is read.  Not part of the operator
// library (libks_norm.so); built into libks_streamref.so and used by the
// benchmark only.
//
// Every kernel moves 16-byte pieces with raw buffer instructions:
//   ksref_read      one load per lane (256-thread workgroups, one per 4 KiB)
//   ksref_write     one store per lane
//   ksref_copy      one load and one store per lane
//   ksref_copy_rows the normalisation kernels' pattern: a wave owns
//                   `pieces` KiB, lane l holds pieces l + 64 k, all loads come
//                   first, then a wave-wide sum and a double-precision
//                   reciprocal square root (the dependency a row reduction
//                   puts between a row's loads and its stores), then the
//                   stores
//   ksref_inplace4  the fused form's four streams: read x and r, write both
//                   back in place, with the ksref_copy_rows layout
//   ksref_timeline  ksref_copy_rows (layout 0) or ksref_inplace4 (layout 1)
//                   with 8 pieces per lane, or no loads and stores at all
//                   (layout 2), where lane 0 of each wave records
//                   the wall clock at the wave's start, when its first load
//                   has arrived, when all its loads have arrived, when the scale is ready, when its last
//                   store has issued and when its stores are acknowledged,
//                   with the wave's hardware and XCD ids: where the time of a
//                   16 MiB row kernel goes
//   ksref_empty     a kernel that does nothing: the per-launch floor
//   ksref_spin      one wave that waits a given number of microseconds on the
//                   device's constant-rate wall clock, then exits (at most
//                   100 ms): queued ahead of a run of timed calls, it lets the
//                   host enqueue them before the first one starts, so they
//                   run back to back
// `policy` selects the cache bits of the stores: 0 default, 1 non-temporal,
// 2 sc0 sc1 (system scope).  Loads are non-temporal.
//
// Each entry point returns 0, 1 for a size that is not a whole number of
// workgroup blocks (4096 * pieces bytes, at most 2^31 bytes per buffer) or an
// unknown variant, or the hipError_t of the launch.  With start/stop events
// the launch records them at the kernel's start and end (hipExtLaunchKernel).
#include <stdint.h>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr int kNt = 2;                 // non-temporal
constexpr int kScope[3] = {0, 2, 17};  // store policy -> cache bits (default, nt, sc0|sc1)

// (each buffer descriptor spans exactly the caller's buffer, so the hardware
// range check drops any access past it)
template <int SC> __global__ __launch_bounds__(256) void write_one(char *dst, uint32_t bytes)
{
    const uint32_t off = (blockIdx.x * 256u + threadIdx.x) * 16u;
    const auto b = rsrc(dst, bytes);
    const u32x4 v = {off, off ^ 0x55555555u, ~off, 0x3f800000u};
    __builtin_amdgcn_raw_buffer_store_b128(v, b, off, 0, SC);
}

__global__ __launch_bounds__(256) void read_one(const char *src, uint32_t bytes, unsigned *sink)
{
    const uint32_t off = (blockIdx.x * 256u + threadIdx.x) * 16u;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc(src, bytes), off, 0, kNt);
    const unsigned x = v.x ^ v.y ^ v.z ^ v.w;
    if (x == 0x9e3779b9u)              // keeps the load; the store practically never happens
        sink[threadIdx.x] = x;
}

template <int SC> __global__ __launch_bounds__(256) void copy_one(const char *src, char *dst, uint32_t bytes)
{
    const uint32_t off = (blockIdx.x * 256u + threadIdx.x) * 16u;
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc(src, bytes), off, 0, kNt);
    v.x ^= 1u;
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(dst, bytes), off, 0, SC);
}

// the wave's V loads, then the reduction a row imposes, then its V stores
template <int V> __device__ __forceinline__ unsigned wave_scale(const u32x4 (&v)[V])
{
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < V; ++k)
        s += __uint_as_float(v[k].x & 0x3fffffffu);
#pragma unroll
    for (int o = 32; o >= 1; o /= 2)
        s += __shfl_xor(s, o, 64);
    return (unsigned)(float)(1.0 / __builtin_sqrt((double)s + 1.0)) | 1u;
}

template <int V> __global__ __launch_bounds__(256) void copy_rows(const char *src, char *dst)
{
    const uint32_t base = (blockIdx.x * 4u + threadIdx.x / 64u) * (uint32_t)V * 1024u;
    const uint32_t lane = threadIdx.x % 64u;
    const auto a = rsrc(src + base, V * 1024u), b = rsrc(dst + base, V * 1024u);
    u32x4 v[V];
#pragma unroll
    for (int k = 0; k < V; ++k)
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(a, (k * 64u + lane) * 16u, 0, kNt);
    const unsigned m = wave_scale<V>(v);
#pragma unroll
    for (int k = 0; k < V; ++k) {
        u32x4 t = v[k];
        t.x ^= m;
        __builtin_amdgcn_raw_buffer_store_b128(t, b, (k * 64u + lane) * 16u, 0, kNt);
    }
}

template <int V> __global__ __launch_bounds__(256) void inplace4(char *x, char *r)
{
    const uint32_t base = (blockIdx.x * 4u + threadIdx.x / 64u) * (uint32_t)V * 1024u;
    const uint32_t lane = threadIdx.x % 64u;
    const auto ax = rsrc(x + base, V * 1024u), ar = rsrc(r + base, V * 1024u);
    u32x4 a[V], c[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        a[k] = __builtin_amdgcn_raw_buffer_load_b128(ax, (k * 64u + lane) * 16u, 0, kNt);
        c[k] = __builtin_amdgcn_raw_buffer_load_b128(ar, (k * 64u + lane) * 16u, 0, kNt);
    }
#pragma unroll
    for (int k = 0; k < V; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(a[k] ^ c[k], ar, (k * 64u + lane) * 16u, 0, kNt);
    const unsigned m = wave_scale<V>(a);
#pragma unroll
    for (int k = 0; k < V; ++k) {
        u32x4 t = a[k];
        t.x ^= m;
        __builtin_amdgcn_raw_buffer_store_b128(t, ax, (k * 64u + lane) * 16u, 0, kNt);
    }
}

// Wave records of ksref_timeline: 8 words per wave, wave w = 4 * block + wave
// of the block.  Stamps are ticks of the constant-rate wall clock.
enum Stamp { kStart, kFirst, kLoaded, kScaled, kIssued, kAcked, kHwId, kXccId, kStampWords };

// The clock reads are inline asm so that the compiler keeps them in program
// order: after the value they take as input (and so after the loads that value
// came from), or after the stores issued before them.
__device__ __forceinline__ uint64_t clock_now()
{
    uint64_t t;
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
    return t;
}

__device__ __forceinline__ uint64_t clock_after(unsigned dep)
{
    uint64_t t;
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) : "v"(dep) : "memory");
    return t;
}

// the same, and `next` passes through the asm, so work that uses it comes after the clock read
__device__ __forceinline__ uint64_t clock_between(unsigned dep, unsigned &next)
{
    uint64_t t;
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t), "+v"(next) : "v"(dep) : "memory");
    return t;
}

template <int kLayout, int SC> __global__ __launch_bounds__(256) void timeline(char *x, char *y, uint64_t *stamps)
{
    constexpr int V = 8;
    constexpr bool kInplace = kLayout == 1;
    const uint64_t t0 = clock_now();
    const uint32_t wave = blockIdx.x * 4u + threadIdx.x / 64u;
    const uint32_t base = wave * (uint32_t)V * 1024u;
    const uint32_t lane = threadIdx.x % 64u;
    uint64_t tf, t1, t2;
    if constexpr (kLayout == 2) {
        tf = t1 = t2 = clock_now();
    } else {
        const auto ax = rsrc(x + base, V * 1024u), ay = rsrc(y + base, V * 1024u);
        u32x4 a[V], c[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            a[k] = __builtin_amdgcn_raw_buffer_load_b128(ax, (k * 64u + lane) * 16u, 0, kNt);
            if constexpr (kInplace)
                c[k] = __builtin_amdgcn_raw_buffer_load_b128(ay, (k * 64u + lane) * 16u, 0, kNt);
        }
        // loads complete in the order they were issued: with all but V - 1 (or
        // 2V - 1) of them done, the first is back
        unsigned dep = 0;                  // passes through the asm: the sum over all loads comes after it
        if constexpr (kInplace)
            asm volatile("s_waitcnt vmcnt(15)\n\ts_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(tf), "+v"(dep)::"memory");
        else
            asm volatile("s_waitcnt vmcnt(7)\n\ts_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(tf), "+v"(dep)::"memory");
#pragma unroll
        for (int k = 0; k < V; ++k)
            dep ^= a[k].x ^ a[k].w ^ (kInplace ? c[k].x ^ c[k].w : 0u);
        unsigned first = a[0].x;           // the row sum starts from a[0].x
        t1 = clock_between(dep, first);
        a[0].x = first;
        if constexpr (kInplace)
#pragma unroll
            for (int k = 0; k < V; ++k)
                __builtin_amdgcn_raw_buffer_store_b128(a[k] ^ c[k], ay, (k * 64u + lane) * 16u, 0, SC);
        const unsigned m = wave_scale<V>(a);
        t2 = clock_after(m);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            u32x4 t = a[k];
            t.x ^= m;
            __builtin_amdgcn_raw_buffer_store_b128(t, kInplace ? ax : ay, (k * 64u + lane) * 16u, 0, SC);
        }
    }
    const uint64_t t3 = clock_now();
    __builtin_amdgcn_s_waitcnt(0);     // every counter at zero: the stores are acknowledged
    const uint64_t t4 = clock_now();
    if (lane == 0) {
        unsigned hw, xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        uint64_t *r = stamps + (size_t)wave * kStampWords;
        r[kStart] = t0;
        r[kFirst] = tf;
        r[kLoaded] = t1;
        r[kScaled] = t2;
        r[kIssued] = t3;
        r[kAcked] = t4;
        r[kHwId] = hw;
        r[kXccId] = xcc;
    }
}

__global__ __launch_bounds__(256) void empty_kernel() {}

// waits `ticks` of the constant-rate wall clock (every wave of the one
// workgroup leaves when the clock has moved that far)
__global__ __launch_bounds__(64) void spin_kernel(uint64_t ticks)
{
    const uint64_t t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks)
        __builtin_amdgcn_s_sleep(8);
}

template <typename Kernel, typename... Args>
int go(Kernel k, unsigned groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, Args... args)
{
    if (e0 != nullptr || e1 != nullptr)
        hipExtLaunchKernelGGL(k, dim3(groups), dim3(256), 0u, s, e0, e1, 0u, args...);
    else
        hipLaunchKernelGGL(k, dim3(groups), dim3(256), 0, s, args...);
    return (int)hipGetLastError();
}

// workgroups for `bytes` in blocks of 4096 * pieces bytes, or 0 if it is not a whole number of them
unsigned groups_for(uint64_t bytes, int pieces)
{
    const uint64_t block = 4096ull * (uint64_t)pieces;
    if (bytes == 0 || bytes > (1ull << 31) || bytes % block != 0)
        return 0;
    return (unsigned)(bytes / block);
}

// the timeline kernel of layout L with the given store cache bits
template <int L>
int timeline_policy(int policy, unsigned g, hipStream_t s, hipEvent_t e0, hipEvent_t e1, char *x, char *y, uint64_t *st)
{
    switch (policy) {
    case 0: return go(timeline<L, kScope[0]>, g, s, e0, e1, x, y, st);
    case 1: return go(timeline<L, kScope[1]>, g, s, e0, e1, x, y, st);
    case 2: return go(timeline<L, kScope[2]>, g, s, e0, e1, x, y, st);
    default: return 1;
    }
}

}  // namespace

extern "C" {

int ksref_read(const void *src, uint64_t bytes, void *sink, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const unsigned g = groups_for(bytes, 1);
    return g == 0 ? 1 : go(read_one, g, s, e0, e1, (const char *)src, (uint32_t)bytes, (unsigned *)sink);
}

int ksref_write(void *dst, uint64_t bytes, int policy, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const unsigned g = groups_for(bytes, 1);
    if (g == 0)
        return 1;
    switch (policy) {
    case 0: return go(write_one<kScope[0]>, g, s, e0, e1, (char *)dst, (uint32_t)bytes);
    case 1: return go(write_one<kScope[1]>, g, s, e0, e1, (char *)dst, (uint32_t)bytes);
    case 2: return go(write_one<kScope[2]>, g, s, e0, e1, (char *)dst, (uint32_t)bytes);
    default: return 1;
    }
}

int ksref_copy(const void *src, void *dst, uint64_t bytes, int policy, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const unsigned g = groups_for(bytes, 1);
    if (g == 0)
        return 1;
    switch (policy) {
    case 0: return go(copy_one<kScope[0]>, g, s, e0, e1, (const char *)src, (char *)dst, (uint32_t)bytes);
    case 1: return go(copy_one<kScope[1]>, g, s, e0, e1, (const char *)src, (char *)dst, (uint32_t)bytes);
    case 2: return go(copy_one<kScope[2]>, g, s, e0, e1, (const char *)src, (char *)dst, (uint32_t)bytes);
    default: return 1;
    }
}

int ksref_copy_rows(const void *src, void *dst, uint64_t bytes, int pieces, hipStream_t s, hipEvent_t e0,
                    hipEvent_t e1)
{
    const unsigned g = groups_for(bytes, pieces);
    if (g == 0)
        return 1;
    switch (pieces) {
    case 1: return go(copy_rows<1>, g, s, e0, e1, (const char *)src, (char *)dst);
    case 2: return go(copy_rows<2>, g, s, e0, e1, (const char *)src, (char *)dst);
    case 4: return go(copy_rows<4>, g, s, e0, e1, (const char *)src, (char *)dst);
    case 8: return go(copy_rows<8>, g, s, e0, e1, (const char *)src, (char *)dst);
    default: return 1;
    }
}

int ksref_inplace4(void *x, void *r, uint64_t bytes, int pieces, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const unsigned g = groups_for(bytes, pieces);
    if (g == 0)
        return 1;
    switch (pieces) {
    case 1: return go(inplace4<1>, g, s, e0, e1, (char *)x, (char *)r);
    case 2: return go(inplace4<2>, g, s, e0, e1, (char *)x, (char *)r);
    case 4: return go(inplace4<4>, g, s, e0, e1, (char *)x, (char *)r);
    case 8: return go(inplace4<8>, g, s, e0, e1, (char *)x, (char *)r);
    default: return 1;
    }
}

// x and y of `bytes` each (a whole number of 32 KiB blocks; layout 2 touches
// neither); stamps of at least 64 bytes per wave (bytes / 8 KiB waves).
// layout 0: y = x with the rows pattern; 1: the fused form's streams on x and
// y in place; 2: the waves only take their stamps.  policy: the stores' cache
// bits as for ksref_write.
int ksref_timeline(void *x, void *y, uint64_t bytes, int layout, int policy, void *stamps, uint64_t stamps_bytes,
                   hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const unsigned g = groups_for(bytes, 8);
    if (g == 0 || stamps == nullptr || stamps_bytes < (uint64_t)g * 4u * kStampWords * sizeof(uint64_t) ||
        ((uintptr_t)stamps & 7u) != 0)
        return 1;
    char *cx = (char *)x, *cy = (char *)y;
    uint64_t *st = (uint64_t *)stamps;
    switch (layout) {
    case 0: return timeline_policy<0>(policy, g, s, e0, e1, cx, cy, st);
    case 1: return timeline_policy<1>(policy, g, s, e0, e1, cx, cy, st);
    case 2: return timeline_policy<2>(policy, g, s, e0, e1, cx, cy, st);
    default: return 1;
    }
}

// the wall clock's rate (kHz) of the current device
int ksref_wall_clock_khz(int *khz)
{
    if (khz == nullptr)
        return 1;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
    return (int)err;
}

int ksref_empty(unsigned groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return groups == 0 ? 1 : go(empty_kernel, groups, s, e0, e1);
}

int ksref_spin(unsigned microseconds, hipStream_t s)
{
    if (microseconds == 0 || microseconds > 100000)
        return 1;
    int dev = 0, khz = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (err != hipSuccess)
        return (int)err;
    if (khz <= 0)
        return 1;
    const uint64_t ticks = (uint64_t)microseconds * (uint64_t)khz / 1000u;
    hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, s, ticks);
    return (int)hipGetLastError();
}

}  // extern "C"
