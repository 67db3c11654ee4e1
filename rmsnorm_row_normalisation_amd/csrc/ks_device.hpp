// Device code for RMSNorm (forward and backward), fused residual-add RMSNorm
// (in place, and the out-of-place RMSNorm(x + residual) * w), the SwiGLU
// activation and softmax on gfx950 (CDNA4).
//
// Operation (kernscope README, "Numerical contract"): per row, widen to fp32,
// sum of squares in fp32, scale = rsqrt(sum / H + eps), y = (v * scale) *
// fp32(w), round to the storage dtype.  The fused form first forms the fp32
// sum s = x + residual, stores cast(s) to residual, and normalises the
// unrounded s into x; the out-of-place form normalises s into out and writes
// nothing else.  SwiGLU, softmax and the backward are described in their own
// sections below.
//
// Kernel families (one entry point per operation and family, at the end):
//   *_vec           a team of kTpr lanes owns a row; each lane keeps kVpt
//                   16-byte pieces of it in VGPRs, so every byte of the
//                   inputs is read from HBM once and every output byte
//                   written once.  Loads and stores are raw buffer
//                   instructions on one descriptor per group of rows; pieces
//                   past the end of the row get an out-of-range offset, so
//                   they read as zero and their stores are dropped by the
//                   hardware range check.  The backward's vector kernel walks
//                   several row groups per workgroup.
//   *_generic       a team of kTpr lanes strides over the row with kEpa
//                   elements per access, in passes (normalisation: sum, then
//                   normalise and store; softmax: maximum, sum, store).
//                   Serves unaligned buffers, rows whose byte size is not a
//                   multiple of 16, and rows wider than the vector kernels
//                   hold in registers.
//   rms_norm_backward_colsum / _dw   the weight gradient's column sums.
//   softmax_split_stats / _norm      softmax with a row cut into chunks, one
//                   workgroup per chunk (wide rows in small batches), with
//                   per-chunk statistics in a caller workspace.
//
// Reduction: the vector kernels sum every row in one canonical order that is
// the same for every launch shape (see "Reductions" below), so their results
// do not depend on the plan or on the batch a row is in.  The generic
// kernels' order depends on the plan, which depends only on (op, dtype,
// hidden); the split softmax sums in its own order (chunk sums, rescaled).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace ks {

using u32x4 = unsigned int __attribute__((ext_vector_type(4)));

// Word 3 of a raw (unswizzled, stride 0) buffer descriptor on gfx9-family
// parts, gfx950 included: 32-bit data format.
constexpr int kBufferWord3 = 0x00020000;
// A byte offset past every buffer this library builds (all are < 2^31 bytes):
// loads there return zero and stores there are discarded.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Arguments of the row kernels (normalisation forms and softmax).
struct Params {
    void *y;          // output: rms_norm, out-of-place residual and softmax: out; fused in place: x
    const void *x;    // input x (fused in place: the same buffer as y)
    void *res;        // residual (fused in place: read, then written; out of place: read); else unused
    const void *w;    // weight [hidden] (softmax: unused)
    int64_t rows;
    int32_t hidden;
    float eps;        // softmax: unused
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}

// Two-lane vectors for paired conversions.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Storage dtype tags (kernel names carry them, e.g. rms_norm_vec<ks::bf16, ...>).
struct f32 {};
struct f16 {};
struct bf16 {};

// ---------------------------------------------------------------------------
// Element packing: a 16-byte piece holds kElems values of T.
// ---------------------------------------------------------------------------
template <typename T> struct Pack;

template <> struct Pack<f32> {
    static constexpr int kBytes = 4;
    static constexpr int kElems = 4;
    __device__ static __forceinline__ float get(const u32x4 &v, int e) { return __uint_as_float(v[e]); }
    __device__ static __forceinline__ u32x4 put(const float *f)
    {
        u32x4 r;
        r.x = __float_as_uint(f[0]);
        r.y = __float_as_uint(f[1]);
        r.z = __float_as_uint(f[2]);
        r.w = __float_as_uint(f[3]);
        return r;
    }
};

// bfloat16 is the upper half of binary32: widening is a 16-bit shift, exact.
template <> struct Pack<bf16> {
    static constexpr int kBytes = 2;
    static constexpr int kElems = 8;
    __device__ static __forceinline__ float get(const u32x4 &v, int e)
    {
        unsigned w = v[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    // round to nearest even; a two-lane conversion becomes one
    // v_cvt_pk_bf16_f32 (two scalar conversions would need a third
    // instruction to merge the halves)
    __device__ static __forceinline__ unsigned two(float a, float b)
    {
        const f32x2 v = {a, b};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
    }
    __device__ static __forceinline__ u32x4 put(const float *f)
    {
        u32x4 r;
        r.x = two(f[0], f[1]);
        r.y = two(f[2], f[3]);
        r.z = two(f[4], f[5]);
        r.w = two(f[6], f[7]);
        return r;
    }
};

// The compiler may fuse "fp32 multiply, then convert to fp16" into one
// v_fma_mixlo_f16, which rounds the exact product straight to fp16 (measured:
// it differs from rounding to fp32 first on about 6e-5 of products).  The
// contract rounds to fp32 first, so every value converted to fp16 passes
// through this empty asm, which keeps it an fp32 value (no instruction).
__device__ __forceinline__ float as_fp32(float v)
{
    asm("" : "+v"(v));
    return v;
}

template <> struct Pack<f16> {
    static constexpr int kBytes = 2;
    static constexpr int kElems = 8;
    __device__ static __forceinline__ float get(const u32x4 &v, int e)
    {
        unsigned w = v[e >> 1];
        unsigned short h = (unsigned short)((e & 1) ? (w >> 16) : (w & 0xffffu));
        return (float)__builtin_bit_cast(_Float16, h);   // exact widening
    }
    // round to nearest even; one v_cvt_pk_f16_f32 for the pair
    __device__ static __forceinline__ unsigned two(float a, float b)
    {
        const f32x2 v = {as_fp32(a), as_fp32(b)};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
    }
    __device__ static __forceinline__ u32x4 put(const float *f)
    {
        u32x4 r;
        r.x = two(f[0], f[1]);
        r.y = two(f[2], f[3]);
        r.z = two(f[4], f[5]);
        r.w = two(f[6], f[7]);
        return r;
    }
};

// Scalar element access for the unaligned generic path.
template <typename T> struct Scalar;
template <> struct Scalar<f32> {
    __device__ static __forceinline__ float get(const void *p, int64_t i) { return ((const float *)p)[i]; }
    __device__ static __forceinline__ void put(void *p, int64_t i, float v) { ((float *)p)[i] = v; }
};
template <> struct Scalar<bf16> {
    __device__ static __forceinline__ float get(const void *p, int64_t i)
    {
        return __uint_as_float((unsigned)((const unsigned short *)p)[i] << 16);
    }
    __device__ static __forceinline__ void put(void *p, int64_t i, float v) { ((__bf16 *)p)[i] = (__bf16)v; }
};
template <> struct Scalar<f16> {
    __device__ static __forceinline__ float get(const void *p, int64_t i) { return (float)((const _Float16 *)p)[i]; }
    __device__ static __forceinline__ void put(void *p, int64_t i, float v)
    {
        ((_Float16 *)p)[i] = (_Float16)as_fp32(v);
    }
};

// ---------------------------------------------------------------------------
// Reductions.
//
// The vector kernel sums a row in one canonical order that does not depend on
// the launch shape: each 16-byte piece p (bytes [16p, 16p + 16) of the row) is
// summed element by element in index order (an FMA chain), then the piece
// sums are combined by folding in half: with n the row's piece count rounded
// up to a power of two (missing pieces are zero), s[p] += s[p + n/2] for all
// p < n/2, then n /= 2, until one value is left.  A lane holding pieces
// lane + k * kTpr performs the levels with n/2 >= kTpr locally (k with
// k + n/(2 kTpr)), the levels 64 <= n/2 < kTpr across waves through LDS, and
// the last levels as an XOR butterfly inside the wave.  Every power-of-two
// team size therefore produces the bitwise same sum, so plans may differ
// between batch sizes without changing any result.  Each step adds two
// values; fp32 addition is commutative, so partner lanes agree bitwise.
// ---------------------------------------------------------------------------
// The value of lane ^ kMask, kMask a power of two below 64.
template <int kMask> __device__ __forceinline__ float xor_partner(float v)
{
    if constexpr (kMask == 1)                        // quad_perm [1,0,3,2]
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    else if constexpr (kMask == 2)                   // quad_perm [2,3,0,1]
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    else if constexpr (kMask <= 16)                  // ds_swizzle bit mode: lane ^ kMask within 32 lanes
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (kMask << 10)));
    else
        return __shfl_xor(v, kMask, 64);
}

// Reduction operators.  Max is exact, so its order never matters; the sum's
// order is the canonical fold described above.
struct SumOp {
    __device__ static __forceinline__ float apply(float a, float b) { return a + b; }
};
struct MaxOp {
    __device__ static __forceinline__ float apply(float a, float b) { return fmaxf(a, b); }
};

// Butterfly over aligned groups of kWidth lanes, masks kWidth/2 down to 1.
template <int kWidth, typename Op = SumOp> __device__ __forceinline__ float butterfly(float v)
{
    if constexpr (kWidth >= 2) {
        v = Op::apply(v, xor_partner<kWidth / 2>(v));
        v = butterfly<kWidth / 2, Op>(v);
    }
    return v;
}

// Local folding of kSlots partial sums (kSlots rounded up to a power of two,
// missing slots count as zero); returns the fold of all of them.
template <int kSlots> __device__ __forceinline__ float local_fold(float *part)
{
    constexpr int kP2 = kSlots <= 1 ? 1 : kSlots <= 2 ? 2 : kSlots <= 4 ? 4 : kSlots <= 8 ? 8 : 16;
    static_assert(kSlots <= 16, "at most 16 slots per lane");
#pragma unroll
    for (int n = kP2; n > 1; n /= 2)
#pragma unroll
        for (int k = 0; k < n / 2; ++k)
            if (k + n / 2 < kSlots)
                part[k] = part[k] + part[k + n / 2];
    return part[0];
}

// Finish the canonical fold across a team of kTpr lanes (kTpr a power of two)
// in a block of kBlock threads.  Every thread of the block must call this.
// Each operator has its own LDS slots, so a kernel may reduce once per
// operator without a barrier in between.
template <int kTpr, int kBlock, typename Op = SumOp> __device__ __forceinline__ float team_fold(float v)
{
    if constexpr (kTpr <= 64) {
        return butterfly<kTpr, Op>(v);
    } else {
        constexpr int kWaves = kTpr / 64;            // waves per row
        __shared__ float lanes[kBlock];
        lanes[threadIdx.x] = v;
        __syncthreads();
        const int lane = threadIdx.x & 63;
        const int first = (threadIdx.x / kTpr) * kTpr;
        float a[kWaves];
#pragma unroll
        for (int j = 0; j < kWaves; ++j)
            a[j] = lanes[first + j * 64 + lane];
#pragma unroll
        for (int n = kWaves; n > 1; n /= 2)
#pragma unroll
            for (int j = 0; j < n / 2; ++j)
                a[j] = Op::apply(a[j], a[j + n / 2]);
        return butterfly<64, Op>(a[0]);
    }
}

// Sum over a team of kTpr lanes (generic path: any order that depends only on
// the plan).  Every thread of the block must call this.
template <int kTpr, int kBlock> __device__ __forceinline__ float team_sum(float v)
{
    return team_fold<kTpr, kBlock>(v);
}

// rsqrt(sum / H + eps) with fp32 mean and add, and the reciprocal square root
// evaluated in double (IEEE sqrt, IEEE divide) and rounded once to fp32: the
// correctly rounded value except within about 2^-52 of an fp32 rounding
// boundary, and the same operations the CPU oracle performs.
__device__ __forceinline__ float row_scale(float sum_sq, int32_t hidden, float eps)
{
    const float mean = sum_sq / (float)hidden;
    const float d = mean + eps;
    return (float)(1.0 / __builtin_sqrt((double)d));
}

// ---------------------------------------------------------------------------
// Vector kernel: row held in VGPRs.
//
// kFused: the row is s = x + residual (fp32), else x.  kStoreSum: the
// rounded s is written back to residual (the in-place fused form; without it
// the out-of-place residual form writes only y).
// kLoadCpol / kStoreCpol: cache-policy bits of the streamed x / residual /
// out accesses (0 = default, 2 = non-temporal).  kWeightLds: the workgroup
// first stages the weight row in LDS (one HBM/L2 read per workgroup instead
// of one per row); needs row_bytes of dynamic LDS.
// ---------------------------------------------------------------------------
template <typename T, bool kFused, bool kStoreSum, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol,
          bool kWeightLds>
__device__ __forceinline__ void vec_body(const Params &p)
{
    constexpr int kE = Pack<T>::kElems;
    constexpr int kRpb = kBlock / kTpr;
    const int tid = threadIdx.x;
    const int lane = tid % kTpr;   // position inside the row's team
    const int team = tid / kTpr;   // row inside the block
    const int64_t row0 = (int64_t)blockIdx.x * kRpb;
    const int64_t left = p.rows - row0;
    const uint32_t nrows = left < kRpb ? (uint32_t)left : (uint32_t)kRpb;
    const uint32_t row_bytes = (uint32_t)p.hidden * (uint32_t)Pack<T>::kBytes;
    const uint32_t blk_bytes = nrows * row_bytes;          // rows past the batch are out of range
    const size_t base = (size_t)row0 * row_bytes;

    const auto rx = make_rsrc((const char *)p.x + base, blk_bytes);
    const auto ry = make_rsrc((char *)p.y + base, blk_bytes);
    const auto rw = make_rsrc(p.w, row_bytes);

    uint32_t off[kVpt];
    bool in_row[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        const uint32_t c = (uint32_t)(k * kTpr + lane) * 16u;
        in_row[k] = c < row_bytes;
        off[k] = in_row[k] ? (uint32_t)team * row_bytes + c : kOutOfRange;
    }

    // weight staging loads go out first, so waiting for them does not wait for x
    constexpr int kStage = kWeightLds ? 1 : 0;
    extern __shared__ u32x4 wlds[];
    u32x4 wst[kStage ? (kVpt * kTpr + kBlock - 1) / kBlock : 1];
    if constexpr (kWeightLds) {
#pragma unroll
        for (int i = 0; i < (kVpt * kTpr + kBlock - 1) / kBlock; ++i) {
            const uint32_t c = (uint32_t)(i * kBlock + tid) * 16u;
            wst[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, c < row_bytes ? c : kOutOfRange, 0, 0);
        }
    }

    u32x4 xv[kVpt], wv[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
        xv[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off[k], 0, kLoadCpol);
    u32x4 rv[kFused ? kVpt : 1];
    const auto rr = make_rsrc((char *)p.res + base, kFused ? blk_bytes : 0u);
    if constexpr (kFused) {
#pragma unroll
        for (int k = 0; k < kVpt; ++k)
            rv[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, off[k], 0, kLoadCpol);
    }

    if constexpr (kWeightLds) {
#pragma unroll
        for (int i = 0; i < (kVpt * kTpr + kBlock - 1) / kBlock; ++i) {
            const int v = i * kBlock + tid;
            if (v < kVpt * kTpr)
                wlds[v] = wst[i];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kVpt; ++k)
            wv[k] = wlds[k * kTpr + lane];     // pieces past the row hold zeros
    } else {
#pragma unroll
        for (int k = 0; k < kVpt; ++k)
            wv[k] = __builtin_amdgcn_raw_buffer_load_b128(rw, in_row[k] ? (uint32_t)(k * kTpr + lane) * 16u
                                                                          : kOutOfRange, 0, 0);
    }

    float part[kVpt];   // per-piece sums of squares, elements in index order
    if constexpr (!kFused) {
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                const float v = Pack<T>::get(xv[k], e);
                a = __builtin_fmaf(v, v, a);
            }
            part[k] = a;
        }
        const float scale = row_scale(team_fold<kTpr, kBlock>(local_fold<kVpt>(part)), p.hidden, p.eps);
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            float o[kE];
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                const float t = Pack<T>::get(xv[k], e) * scale;
                o[e] = t * Pack<T>::get(wv[k], e);
            }
            __builtin_amdgcn_raw_buffer_store_b128(Pack<T>::put(o), ry, off[k], 0, kStoreCpol);
        }
    } else {
        float s[kVpt][kE];
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                s[k][e] = Pack<T>::get(xv[k], e) + Pack<T>::get(rv[k], e);
                a = __builtin_fmaf(s[k][e], s[k][e], a);
            }
            part[k] = a;
            // this lane has read every element it will write: store the
            // rounded residual now, so the writes start before the reduction
            if constexpr (kStoreSum)
                __builtin_amdgcn_raw_buffer_store_b128(Pack<T>::put(s[k]), rr, off[k], 0, kStoreCpol);
        }
        const float scale = row_scale(team_fold<kTpr, kBlock>(local_fold<kVpt>(part)), p.hidden, p.eps);
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            float o[kE];
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                const float t = s[k][e] * scale;
                o[e] = t * Pack<T>::get(wv[k], e);
            }
            __builtin_amdgcn_raw_buffer_store_b128(Pack<T>::put(o), ry, off[k], 0, kStoreCpol);
        }
    }
}

// ---------------------------------------------------------------------------
// Element groups of the generic kernels: kEpa == 1 is one scalar element (any
// alignment), kEpa == Pack<T>::kElems one 16-byte piece.  The generic loops
// visit a lane's accesses kGenericBatch at a time, issuing all their loads
// before using any, so the loads' latencies overlap (one access per
// iteration left these kernels latency-bound); the element order of every
// sum is unchanged.
// ---------------------------------------------------------------------------
constexpr int kGenericBatch = 4;

template <typename T, int kEpa> struct Access {
    using V = u32x4;
    __device__ static __forceinline__ V load(const void *p, int64_t i)
    {
        return *(const u32x4 *)((const char *)p + i * Pack<T>::kBytes);
    }
    __device__ static __forceinline__ float get(const V &v, int e) { return Pack<T>::get(v, e); }
    __device__ static __forceinline__ void store(void *p, int64_t i, const float *f)
    {
        *(u32x4 *)((char *)p + i * Pack<T>::kBytes) = Pack<T>::put(f);
    }
};
template <typename T> struct Access<T, 1> {
    using V = float;
    __device__ static __forceinline__ V load(const void *p, int64_t i) { return Scalar<T>::get(p, i); }
    __device__ static __forceinline__ float get(const V &v, int) { return v; }
    __device__ static __forceinline__ void store(void *p, int64_t i, const float *f) { Scalar<T>::put(p, i, f[0]); }
};

// A lane's running sum in the generic kernels, where one lane may add
// thousands of batches of a long row: each batch is summed on its own, then
// added with a compensation term (Neumaier's form of Kahan summation), so the
// lane's sum keeps about one rounding however many batches it takes.  (A
// plain running sum of positive terms drifts by up to one rounding per
// addition: about 1e-6 relative for 2^24-element fp32 rows.)  Non-finite
// sums pass through unchanged: the compensation is dropped once the sum is
// infinite, so +inf stays +inf instead of turning into NaN.
struct LaneSum {
    float s = 0.0f;
    float c = 0.0f;
    __device__ __forceinline__ void add(float v)
    {
        const float t = s + v;
        const float e = fabsf(s) >= fabsf(v) ? (s - t) + v : (v - t) + s;
        c = __builtin_isfinite(t) ? c + e : c;
        s = t;
    }
    __device__ __forceinline__ float value() const { return s + c; }
};

// ---------------------------------------------------------------------------
// Generic kernel: two passes over the row, kEpa elements per access.
// kEpa == 1: scalar accesses (any alignment); kEpa == 16 / sizeof(T): 16-byte
// accesses (aligned buffers, row bytes a multiple of 16).
// ---------------------------------------------------------------------------
template <typename T, bool kFused, bool kStoreSum, int kTpr, int kEpa, int kBlock>
__device__ __forceinline__ void generic_body(const Params &p)
{
    using A = Access<T, kEpa>;
    using V = typename A::V;
    constexpr int kU = kGenericBatch;
    constexpr int kRpb = kBlock / kTpr;
    const int tid = threadIdx.x;
    const int lane = tid % kTpr;
    const int team = tid / kTpr;
    const int64_t row = (int64_t)blockIdx.x * kRpb + team;
    const bool active = row < p.rows;   // no early return: team_sum may hold a barrier
    const int64_t H = p.hidden;
    const int64_t base = active ? row * H : 0;
    constexpr int64_t kStride = (int64_t)kTpr * kEpa;

    LaneSum sum_sq;
    if (active) {
        for (int64_t j0 = (int64_t)lane * kEpa; j0 < H; j0 += kU * kStride) {
            V xv[kU], rv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t j = j0 + u * kStride;
                if (j < H) {
                    xv[u] = A::load(p.x, base + j);
                    if constexpr (kFused)
                        rv[u] = A::load(p.res, base + j);
                }
            }
            float batch = 0.0f;
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (j0 + u * kStride < H) {
#pragma unroll
                    for (int e = 0; e < kEpa; ++e) {
                        float v = A::get(xv[u], e);
                        if constexpr (kFused)
                            v = v + A::get(rv[u], e);
                        batch = __builtin_fmaf(v, v, batch);
                    }
                }
            }
            sum_sq.add(batch);
        }
    }
    const float scale = row_scale(team_sum<kTpr, kBlock>(sum_sq.value()), p.hidden, p.eps);
    if (!active)
        return;
    // Second pass: each element is read again and written by the same lane that
    // read it in the first pass (a batch's loads all precede its stores), so
    // in-place updates are safe.
    for (int64_t j0 = (int64_t)lane * kEpa; j0 < H; j0 += kU * kStride) {
        V xv[kU], rv[kU], wv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = j0 + u * kStride;
            if (j < H) {
                xv[u] = A::load(p.x, base + j);
                wv[u] = A::load(p.w, j);
                if constexpr (kFused)
                    rv[u] = A::load(p.res, base + j);
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = j0 + u * kStride;
            if (j < H) {
                float v[kEpa], o[kEpa];
#pragma unroll
                for (int e = 0; e < kEpa; ++e) {
                    v[e] = A::get(xv[u], e);
                    if constexpr (kFused)
                        v[e] = v[e] + A::get(rv[u], e);
                }
                if constexpr (kFused && kStoreSum)
                    A::store(p.res, base + j, v);
#pragma unroll
                for (int e = 0; e < kEpa; ++e) {
                    const float t = v[e] * scale;
                    o[e] = t * A::get(wv[u], e);
                }
                A::store(p.y, base + j, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// SwiGLU activation: out[r, j] = (g * sigmoid(g)) * u with g = x[r, j] and
// u = x[r, d + j] widened to fp32, rounded once to the storage dtype.
// Elementwise: every launch shape gives the same result.
// ---------------------------------------------------------------------------
struct SwigluParams {
    void *out;        // [rows, d]
    const void *x;    // [rows, 2 d]: gate half, then up half
    int64_t rows;
    int32_t d;
};

// sigmoid(g) for outputs rounded to 16 bits.  e^-g comes from the hardware
// base-2 exponential, with -g * log2(e) carried as hi + lo (log2(e) split into
// an fp32 head and tail, as in Cody and Waite's argument reduction, and the
// head product's rounding error recovered exactly by an FMA, the error-free
// product of Ogita, Rump and Oishi) and 2^lo applied to first order; 1 / (1 + e) is the hardware reciprocal with one
// Newton step.  Within a few fp32 ulps of the exact value, far below half an
// ulp of bf16 or fp16.  -g is clamped to [-20, 88]: from g >= 20 the result is
// exactly 1, as the exact value rounds to 1 in fp32; below g = -88 (exact
// value under 2^-126) it is 0.  NaN stays NaN in the product with g.
__device__ __forceinline__ float sigmoid_fast(float g)
{
    constexpr float kLog2e = 1.44269502f;       // fp32 nearest to log2(e)
    constexpr float kLog2eTail = 1.925963e-8f;  // log2(e) - kLog2e
    constexpr float kLn2 = 0.693147182f;
    const float x = fminf(fmaxf(-g, -20.0f), 88.0f);
    const float hi = x * kLog2e;
    const float lo = __builtin_fmaf(x, kLog2eTail, __builtin_fmaf(x, kLog2e, -hi));
    const float e2 = __builtin_amdgcn_exp2f(hi);
    const float e = __builtin_fmaf(e2, lo * kLn2, e2);
    const float d = 1.0f + e;
    float r = __builtin_amdgcn_rcpf(d);
    r = __builtin_fmaf(__builtin_fmaf(-d, r, 1.0f), r, r);
    return -g > 88.0f ? 0.0f : r;
}

// fp32 outputs (tolerance 1e-6 relative) use the device library's exp and an
// IEEE division; 16-bit outputs use sigmoid_fast.
template <typename T> __device__ __forceinline__ float swiglu_one(float g, float u)
{
    float s;
    if constexpr (Pack<T>::kBytes == 4)
        s = 1.0f / (1.0f + expf(-g));
    else
        s = sigmoid_fast(g);
    const float t = g * s;
    return t * u;
}

// A team of kTpr lanes owns a row; lane l handles output pieces l + k * kTpr
// (16 bytes each) and the matching gate and up pieces.
template <typename T, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol>
__device__ __forceinline__ void swiglu_vec_body(const SwigluParams &p)
{
    constexpr int kE = Pack<T>::kElems;
    constexpr int kRpb = kBlock / kTpr;
    const int tid = threadIdx.x;
    const int lane = tid % kTpr;
    const int team = tid / kTpr;
    const int64_t row0 = (int64_t)blockIdx.x * kRpb;
    const int64_t left = p.rows - row0;
    const uint32_t nrows = left < kRpb ? (uint32_t)left : (uint32_t)kRpb;
    const uint32_t out_row = (uint32_t)p.d * (uint32_t)Pack<T>::kBytes;   // bytes of one output row
    const uint32_t in_row = 2u * out_row;
    const auto rx = make_rsrc((const char *)p.x + (size_t)row0 * in_row, nrows * in_row);
    const auto ro = make_rsrc((char *)p.out + (size_t)row0 * out_row, nrows * out_row);

    uint32_t goff[kVpt], ooff[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        const uint32_t c = (uint32_t)(k * kTpr + lane) * 16u;
        const bool in = c < out_row;
        goff[k] = in ? (uint32_t)team * in_row + c : kOutOfRange;
        ooff[k] = in ? (uint32_t)team * out_row + c : kOutOfRange;
    }
    u32x4 gv[kVpt], uv[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
        gv[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, goff[k], 0, kLoadCpol);
#pragma unroll
    for (int k = 0; k < kVpt; ++k)   // the up piece sits one output row further on
        uv[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, goff[k] == kOutOfRange ? kOutOfRange : goff[k] + out_row,
                                                      0, kLoadCpol);
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        float o[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e)
            o[e] = swiglu_one<T>(Pack<T>::get(gv[k], e), Pack<T>::get(uv[k], e));
        __builtin_amdgcn_raw_buffer_store_b128(Pack<T>::put(o), ro, ooff[k], 0, kStoreCpol);
    }
}

// Any alignment and width: one element per thread per step, grid-stride.
template <typename T>
__device__ __forceinline__ void swiglu_generic_body(const SwigluParams &p)
{
    const int64_t total = p.rows * (int64_t)p.d;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / p.d;
        const int64_t j = i - r * p.d;
        const float g = Scalar<T>::get(p.x, r * 2 * (int64_t)p.d + j);
        const float u = Scalar<T>::get(p.x, r * 2 * (int64_t)p.d + p.d + j);
        Scalar<T>::put(p.out, i, swiglu_one<T>(g, u));
    }
}

// ---------------------------------------------------------------------------
// Softmax over the last dimension: z = x - max(x) over the row (fp32), out =
// exp(z) / sum(exp(z)), rounded once to the storage dtype.  The maximum is
// exact in any order; the sum follows the same canonical fold as the sum of
// squares above, so every vector plan gives the same bits.  A NaN or +inf
// anywhere in a row, or a row of only -inf, makes some z NaN and with it the
// sum and every output of that row; -inf entries of other rows give exp = 0.
// ---------------------------------------------------------------------------

// exp(z) for z <= 0, -inf or NaN.
//   fp32 outputs: the device library's expf (about 1 ulp).
//   fp16 outputs: the hardware base-2 exponential of z * log2(e) with the
//     product's rounding error carried to first order (as in sigmoid_fast):
//     within about 2 fp32 ulps.  z is clamped at -150, where the result is
//     0 anyway, so that -inf does not turn the correction into NaN.
//   bf16 outputs: the hardware exponential of the rounded product.  Its
//     relative error |z| * 2^-24 stays far below half a bf16 ulp (2^-9) for
//     every z whose result is not negligible next to the row's maximum (1).
template <typename T> __device__ __forceinline__ float softmax_exp(float z)
{
    constexpr float kLog2e = 1.44269502f;       // fp32 nearest to log2(e)
    constexpr float kLog2eTail = 1.925963e-8f;  // log2(e) - kLog2e
    constexpr float kLn2 = 0.693147182f;
    if constexpr (Pack<T>::kBytes == 4) {
        return expf(z);
    } else if constexpr (__is_same(T, bf16)) {
        return __builtin_amdgcn_exp2f(z * kLog2e);
    } else {
        const float x = z < -150.0f ? -150.0f : z;   // NaN passes through
        const float hi = x * kLog2e;
        const float lo = __builtin_fmaf(x, kLog2eTail, __builtin_fmaf(x, kLog2e, -hi));
        const float e2 = __builtin_amdgcn_exp2f(hi);
        return __builtin_fmaf(e2, lo * kLn2, e2);
    }
}

// e / sum with r = 1 / sum (IEEE division, once per row).  fp32 outputs add
// one remainder correction (q + (e - q sum) r), which brings the product
// e * r to within about half an ulp of the quotient; for 16-bit outputs the
// product alone is far inside the output's rounding.
template <typename T> __device__ __forceinline__ float softmax_div(float e, float sum, float r)
{
    const float q = e * r;
    if constexpr (Pack<T>::kBytes == 4)
        return __builtin_fmaf(__builtin_fmaf(-q, sum, e), r, q);
    else
        return q;
}

// Vector kernel: a team of kTpr lanes owns a row held in VGPRs (pieces
// lane + k * kTpr), read once from HBM and written once.
template <typename T, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol>
__device__ __forceinline__ void softmax_vec_body(const Params &p)
{
    constexpr int kE = Pack<T>::kElems;
    constexpr int kRpb = kBlock / kTpr;
    const int tid = threadIdx.x;
    const int lane = tid % kTpr;
    const int team = tid / kTpr;
    const int64_t row0 = (int64_t)blockIdx.x * kRpb;
    const int64_t left = p.rows - row0;
    const uint32_t nrows = left < kRpb ? (uint32_t)left : (uint32_t)kRpb;
    const uint32_t row_bytes = (uint32_t)p.hidden * (uint32_t)Pack<T>::kBytes;
    const uint32_t blk_bytes = nrows * row_bytes;
    const size_t base = (size_t)row0 * row_bytes;
    const auto rx = make_rsrc((const char *)p.x + base, blk_bytes);
    const auto ry = make_rsrc((char *)p.y + base, blk_bytes);

    uint32_t off[kVpt];
    bool in_row[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        const uint32_t c = (uint32_t)(k * kTpr + lane) * 16u;
        in_row[k] = c < row_bytes;
        off[k] = in_row[k] ? (uint32_t)team * row_bytes + c : kOutOfRange;
    }
    u32x4 xv[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
        xv[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off[k], 0, kLoadCpol);

    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        float pm = Pack<T>::get(xv[k], 0);
#pragma unroll
        for (int e = 1; e < kE; ++e)
            pm = fmaxf(pm, Pack<T>::get(xv[k], e));
        mx = in_row[k] ? fmaxf(mx, pm) : mx;   // pieces past the row read as zeros
    }
    const float m = team_fold<kTpr, kBlock, MaxOp>(mx);

    float ev[kVpt][kE];
    float part[kVpt];   // per-piece sums, elements in index order
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            ev[k][e] = softmax_exp<T>(Pack<T>::get(xv[k], e) - m);
            a = a + ev[k][e];
        }
        part[k] = in_row[k] ? a : 0.0f;
    }
    const float sum = team_fold<kTpr, kBlock>(local_fold<kVpt>(part));
    const float r = 1.0f / sum;
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        float o[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e)
            o[e] = softmax_div<T>(ev[k][e], sum, r);
        __builtin_amdgcn_raw_buffer_store_b128(Pack<T>::put(o), ry, off[k], 0, kStoreCpol);
    }
}

// Split-row softmax, for wide rows in small batches: a row is cut into
// chunks of kSplitLanes * kVpt consecutive 16-byte pieces, one 256-lane
// workgroup per (chunk, row), so that a batch of a few rows still spreads
// over the chip.  Two kernels:
//   stats:  each chunk's maximum m_c (NaN if the chunk holds one) and
//           s_c = sum of exp(x - m_c) over the chunk (canonical fold),
//           written to the workspace as (m_c, s_c); a chunk of only -inf has
//           s_c = 0;
//   norm:   each chunk's workgroup reads its row's (m_c, s_c), forms
//           M = max m_c and S = sum of s_c * exp(m_c - M) (lane l takes
//           chunks l, l + 256, ... in order, then the canonical fold), and
//           writes exp(x - M) / S for its chunk.
// exp(x - M) is the value the one-pass kernels compute; S is formed in
// another order, with the factors exp(m_c - M), so a result can differ from
// theirs in the last bit.  The page's non-finite rules hold: a NaN or +inf
// makes some s_c NaN (exp(NaN - m_c) or exp(inf - inf)), so S is NaN; a row
// of only -inf has M = -inf and every m_c - M is NaN.  M itself is a plain
// maximum (NaN m_c are skipped unless all are NaN); a NaN s_c still reaches
// S through s_c * exp(m_c - M).  Chunks never overlap, and a workgroup stores only the
// chunk it loaded, so out may be x.
constexpr int kSplitLanes = 256;
constexpr int kSplitCpol = 2;   // non-temporal loads and stores: streamed once

// Maximum that keeps NaN (fmaxf drops it): a chunk holding a NaN gets
// m_c = NaN, so its s_c is NaN and so is its row's sum.  Its own LDS slots
// (a distinct operator), apart from the MaxOp fold of the same kernels.
struct NanMaxOp {
    __device__ static __forceinline__ float apply(float a, float b) { return (a != a || b != b) ? a + b : fmaxf(a, b); }
};

struct SplitParams {
    void *y;          // out [rows, hidden]
    const void *x;    // [rows, hidden]
    float *stats;     // workspace [rows, chunks, 2]: (m_c, s_c)
    int64_t rows;
    int32_t hidden;
    int32_t chunks;   // ceil(row pieces / (kSplitLanes * kVpt))
};

// The lane's pieces of chunk blockIdx.x of row blockIdx.y (non-temporal
// loads; pieces past the row read as zero and are flagged).
template <typename T, int kVpt>
__device__ __forceinline__ void split_load(const SplitParams &p, u32x4 *xv, uint32_t *off, bool *in_row)
{
    const uint32_t row_bytes = (uint32_t)p.hidden * (uint32_t)Pack<T>::kBytes;
    const auto rx = make_rsrc((const char *)p.x + (size_t)blockIdx.y * row_bytes, row_bytes);
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        const uint32_t piece = (uint32_t)blockIdx.x * (kSplitLanes * kVpt) + (uint32_t)(k * kSplitLanes) + threadIdx.x;
        in_row[k] = piece * 16u < row_bytes;
        off[k] = in_row[k] ? piece * 16u : kOutOfRange;
        xv[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off[k], 0, kSplitCpol);
    }
}

template <typename T, int kVpt>
__device__ __forceinline__ void softmax_split_stats_body(const SplitParams &p)
{
    constexpr int kE = Pack<T>::kElems;
    u32x4 xv[kVpt];
    uint32_t off[kVpt];
    bool in_row[kVpt];
    split_load<T, kVpt>(p, xv, off, in_row);
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        float pm = Pack<T>::get(xv[k], 0);
#pragma unroll
        for (int e = 1; e < kE; ++e)
            pm = NanMaxOp::apply(pm, Pack<T>::get(xv[k], e));
        mx = in_row[k] ? NanMaxOp::apply(mx, pm) : mx;
    }
    const float m = team_fold<kSplitLanes, kSplitLanes, NanMaxOp>(mx);
    float part[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        float a = softmax_exp<T>(Pack<T>::get(xv[k], 0) - m);
#pragma unroll
        for (int e = 1; e < kE; ++e)
            a = a + softmax_exp<T>(Pack<T>::get(xv[k], e) - m);
        part[k] = in_row[k] ? a : 0.0f;
    }
    float sum = team_fold<kSplitLanes, kSplitLanes>(local_fold<kVpt>(part));
    if (m == -__builtin_inff())
        sum = 0.0f;                        // only -inf here: nothing to add
    if (threadIdx.x == 0) {
        float *st = p.stats + ((size_t)blockIdx.y * (size_t)p.chunks + blockIdx.x) * 2;
        st[0] = m;
        st[1] = sum;
    }
}

template <typename T, int kVpt>
__device__ __forceinline__ void softmax_split_norm_body(const SplitParams &p)
{
    constexpr int kE = Pack<T>::kElems;
    u32x4 xv[kVpt];
    uint32_t off[kVpt];
    bool in_row[kVpt];
    split_load<T, kVpt>(p, xv, off, in_row);      // in flight while the row's statistics combine
    const float *st = p.stats + (size_t)blockIdx.y * (size_t)p.chunks * 2;
    float mx = -__builtin_inff();
    for (int c = threadIdx.x; c < p.chunks; c += kSplitLanes)
        mx = fmaxf(mx, st[2 * c]);
    const float M = team_fold<kSplitLanes, kSplitLanes, MaxOp>(mx);
    float acc = 0.0f;
    for (int c = threadIdx.x; c < p.chunks; c += kSplitLanes)
        acc = acc + st[2 * c + 1] * softmax_exp<T>(st[2 * c] - M);
    const float S = team_fold<kSplitLanes, kSplitLanes>(acc);
    const float r = 1.0f / S;
    const uint32_t row_bytes = (uint32_t)p.hidden * (uint32_t)Pack<T>::kBytes;
    const auto ry = make_rsrc((char *)p.y + (size_t)blockIdx.y * row_bytes, row_bytes);
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        float o[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e)
            o[e] = softmax_div<T>(softmax_exp<T>(Pack<T>::get(xv[k], e) - M), S, r);
        __builtin_amdgcn_raw_buffer_store_b128(Pack<T>::put(o), ry, off[k], 0, kSplitCpol);
    }
}

// Generic kernel: three passes over the row (maximum, sum, store), kEpa
// elements per access as in generic_body.  Each lane reads and writes the
// same elements in the last pass, after the whole team has finished the
// first two, so out may be x.
template <typename T, int kTpr, int kEpa, int kBlock>
__device__ __forceinline__ void softmax_generic_body(const Params &p)
{
    using A = Access<T, kEpa>;
    using V = typename A::V;
    constexpr int kU = kGenericBatch;
    constexpr int kRpb = kBlock / kTpr;
    const int tid = threadIdx.x;
    const int lane = tid % kTpr;
    const int team = tid / kTpr;
    const int64_t row = (int64_t)blockIdx.x * kRpb + team;
    const bool active = row < p.rows;   // no early return before the reductions
    const int64_t H = p.hidden;
    const int64_t base = active ? row * H : 0;
    constexpr int64_t kStride = (int64_t)kTpr * kEpa;

    float mx = -__builtin_inff();
    LaneSum s;
    if (active) {
        for (int64_t j0 = (int64_t)lane * kEpa; j0 < H; j0 += kU * kStride) {
            V xv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (j0 + u * kStride < H)
                    xv[u] = A::load(p.x, base + j0 + u * kStride);
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (j0 + u * kStride < H)
#pragma unroll
                    for (int e = 0; e < kEpa; ++e)
                        mx = fmaxf(mx, A::get(xv[u], e));
        }
    }
    const float m = team_fold<kTpr, kBlock, MaxOp>(mx);
    if (active) {
        for (int64_t j0 = (int64_t)lane * kEpa; j0 < H; j0 += kU * kStride) {
            V xv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (j0 + u * kStride < H)
                    xv[u] = A::load(p.x, base + j0 + u * kStride);
            float batch = 0.0f;
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (j0 + u * kStride < H)
#pragma unroll
                    for (int e = 0; e < kEpa; ++e)
                        batch = batch + softmax_exp<T>(A::get(xv[u], e) - m);
            s.add(batch);
        }
    }
    const float sum = team_sum<kTpr, kBlock>(s.value());
    if (!active)
        return;
    const float r = 1.0f / sum;
    for (int64_t j0 = (int64_t)lane * kEpa; j0 < H; j0 += kU * kStride) {
        V xv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (j0 + u * kStride < H)
                xv[u] = A::load(p.x, base + j0 + u * kStride);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = j0 + u * kStride;
            if (j < H) {
                float o[kEpa];
#pragma unroll
                for (int e = 0; e < kEpa; ++e)
                    o[e] = softmax_div<T>(softmax_exp<T>(A::get(xv[u], e) - m), sum, r);
                A::store(p.y, base + j, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm backward: for y_j = x_j * rho * w_j with rho = rsqrt(mean(x^2) +
// eps), and an incoming gradient dy,
//   dx_j = rho * (g_j - c * x_j),  g_j = dy_j * w_j,  c = rho^2 * sum(g * x) / H,
//   dw_j = sum over rows of dy_j * (x_j * rho).
// rho is the forward's fp32 scale (row_scale, bit-identical to the forward).
// The two row sums (x^2 and g * x) use the canonical fold, so dx does not
// depend on the plan.  dw is summed without atomics, in a fixed order: each
// team accumulates its rows' terms in registers (rows in increasing order),
// each workgroup adds its teams' sums in team order into one fp32 partial
// row, and a second kernel adds the partial rows in a fixed order.
// ---------------------------------------------------------------------------
struct BwdParams {
    void *dx;           // [rows, hidden] output
    const void *dy;     // [rows, hidden]
    const void *x;      // [rows, hidden]
    const void *w;      // [hidden]
    float *part;        // [gridDim.x or chunks, hidden] fp32 partial sums of dw (null: no dw)
    float *rho;         // [rows] per-row scale (generic path, when dw is wanted)
    int64_t rows;
    int32_t hidden;
    float eps;
    int32_t part_nt;    // nonzero: the partial rows are stored non-temporal
};

// kN consecutive fp32 partial sums of dw from v to a, stored plainly or
// non-temporal.  The empty asm statements keep the two branches apart: a
// branch over two C++ stores that differ only in the hint is otherwise folded
// into one plain store.  (Buffer stores, whose hint is an immediate, measured
// 10% slower for the 32-byte pieces of 16-bit dtypes.)
template <int kN>
__device__ __forceinline__ void store_part(float *a, const float *v, int32_t nt)
{
    if (nt) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < kN; ++e)
            __builtin_nontemporal_store(v[e], a + e);
    } else {
#pragma unroll
        for (int e = 0; e < kN; ++e)
            a[e] = v[e];
        asm volatile("" ::: "memory");
    }
}

// Two team sums in the canonical fold, safe to call repeatedly in one kernel:
// barriers on both sides of the LDS exchange.  Every thread of the block
// must call this.
template <int kTpr, int kBlock> __device__ __forceinline__ void team_fold2(float &a, float &b)
{
    if constexpr (kTpr <= 64) {
        a = butterfly<kTpr>(a);
        b = butterfly<kTpr>(b);
    } else {
        constexpr int kWaves = kTpr / 64;
        __shared__ float la[kBlock], lb[kBlock];
        __syncthreads();                       // readers of the previous call are done
        la[threadIdx.x] = a;
        lb[threadIdx.x] = b;
        __syncthreads();
        const int lane = threadIdx.x & 63;
        const int first = (threadIdx.x / kTpr) * kTpr;
        float pa[kWaves], pb[kWaves];
#pragma unroll
        for (int j = 0; j < kWaves; ++j) {
            pa[j] = la[first + j * 64 + lane];
            pb[j] = lb[first + j * 64 + lane];
        }
#pragma unroll
        for (int n = kWaves; n > 1; n /= 2)
#pragma unroll
            for (int j = 0; j < n / 2; ++j) {
                pa[j] = pa[j] + pa[j + n / 2];
                pb[j] = pb[j] + pb[j + n / 2];
            }
        a = butterfly<64>(pa[0]);
        b = butterfly<64>(pb[0]);
    }
}

// Vector kernel: the weight pieces stay in VGPRs; the block walks row groups
// blockIdx.x, blockIdx.x + gridDim.x, ... (the same count for every thread,
// so the barriers inside team_fold2 are uniform), loading the next group
// while it finishes the current one.  x and dy are streamed once with
// non-temporal loads; dx is stored non-temporal.
template <typename T, int kTpr, int kVpt, int kBlock>
__device__ __forceinline__ void bwd_vec_body(const BwdParams &p)
{
    constexpr int kE = Pack<T>::kElems;
    constexpr int kRpb = kBlock / kTpr;
    constexpr int kNt = 2;
    const int tid = threadIdx.x;
    const int lane = tid % kTpr;
    const int team = tid / kTpr;
    const uint32_t row_bytes = (uint32_t)p.hidden * (uint32_t)Pack<T>::kBytes;
    const auto rw = make_rsrc(p.w, row_bytes);

    bool in_row[kVpt];
    u32x4 wv[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        const uint32_t c = (uint32_t)(k * kTpr + lane) * 16u;
        in_row[k] = c < row_bytes;
        wv[k] = __builtin_amdgcn_raw_buffer_load_b128(rw, in_row[k] ? c : kOutOfRange, 0, 0);
    }
    float acc[kVpt][kE];
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
#pragma unroll
        for (int e = 0; e < kE; ++e)
            acc[k][e] = 0.0f;

    // Row group g covers rows [g * kRpb, g * kRpb + kRpb); rows past the batch
    // fall outside the group's descriptors (zero reads, dropped stores).
    // A group past the batch has zero-size descriptors: its loads read zeros
    // and move no data.
    const int64_t ngroups = (p.rows + kRpb - 1) / kRpb;
    auto group_bytes = [&](int64_t grp) {
        const int64_t left = p.rows - grp * kRpb;
        return left <= 0 ? 0u : (left < kRpb ? (uint32_t)left : (uint32_t)kRpb) * row_bytes;
    };
    uint32_t off[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
        off[k] = in_row[k] ? (uint32_t)team * row_bytes + (uint32_t)(k * kTpr + lane) * 16u : kOutOfRange;
    auto load_group = [&](int64_t grp, u32x4 *xo, u32x4 *dyo) {
        const uint32_t bytes = group_bytes(grp);
        const size_t base = bytes == 0 ? 0 : (size_t)grp * kRpb * row_bytes;
        const auto rx = make_rsrc((const char *)p.x + base, bytes);
        const auto rdy = make_rsrc((const char *)p.dy + base, bytes);
#pragma unroll
        for (int k = 0; k < kVpt; ++k)
            xo[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off[k], 0, kNt);
#pragma unroll
        for (int k = 0; k < kVpt; ++k)
            dyo[k] = __builtin_amdgcn_raw_buffer_load_b128(rdy, off[k], 0, kNt);
    };

    // The two row sums of a group (per piece, elements in index order, then
    // the canonical fold within the lane).
    auto sums = [&](const u32x4 *xg, const u32x4 *dg, float &ss, float &dot) {
        float ps[kVpt], pc[kVpt];
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            float a = 0.0f, b = 0.0f;
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                const float xe = Pack<T>::get(xg[k], e);
                const float ge = Pack<T>::get(dg[k], e) * Pack<T>::get(wv[k], e);
                a = __builtin_fmaf(xe, xe, a);
                b = __builtin_fmaf(ge, xe, b);
            }
            ps[k] = a;
            pc[k] = b;
        }
        ss = local_fold<kVpt>(ps);
        dot = local_fold<kVpt>(pc);
    };
    // The team sums, dx of the group, and its dw terms added to acc.
    auto finish = [&](int64_t grp, const u32x4 *xg, const u32x4 *dg, float ss, float dot) {
        team_fold2<kTpr, kBlock>(ss, dot);
        const float rho = row_scale(ss, p.hidden, p.eps);
        const float c = ((dot / (float)p.hidden) * rho) * rho;
        const auto rdx = make_rsrc((char *)p.dx + (size_t)grp * kRpb * row_bytes, group_bytes(grp));
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            float o[kE];
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                const float xe = Pack<T>::get(xg[k], e);
                const float de = Pack<T>::get(dg[k], e);
                const float ge = de * Pack<T>::get(wv[k], e);
                o[e] = __builtin_fmaf(-c, xe, ge) * rho;
                acc[k][e] = __builtin_fmaf(de, xe * rho, acc[k][e]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(Pack<T>::put(o), rdx, off[k], 0, kNt);
        }
    };

    // Software pipeline: while a group is reduced and written, the next
    // group's loads are in flight.  They issue only once the group's own data
    // is back (its sums are formed), so that the memory system returns the
    // groups in turn and a group's dx stores overlap the next group's reads.
    // The first group is peeled off the loop and always issues the next
    // group's loads (a group past the batch has zero-size descriptors), so
    // the loop is entered, as it repeats, with one group's loads followed by
    // the previous group's stores outstanding: the wait for a group's data
    // then counts its loads only and leaves the stores in flight.  Any later
    // last group issues no loads.  g is the same for the whole workgroup, so every
    // thread reaches the barriers in team_fold2 equally often.
    int64_t g = blockIdx.x;
    if (g < ngroups) {
        u32x4 xv[kVpt], dv[kVpt], xn[kVpt], dn[kVpt];
        load_group(g, xv, dv);
        int64_t gn = g + gridDim.x;
        float ss, dot;
        sums(xv, dv, ss, dot);
        asm volatile("" ::"v"(ss), "v"(dot) : "memory");   // the loads below stay after the sums
        load_group(gn, xn, dn);
        finish(g, xv, dv, ss, dot);
        if (gn < ngroups) {
            for (g = gn, gn += gridDim.x; gn < ngroups; g = gn, gn += gridDim.x) {
#pragma unroll
                for (int k = 0; k < kVpt; ++k) {
                    xv[k] = xn[k];
                    dv[k] = dn[k];
                }
                sums(xv, dv, ss, dot);
                asm volatile("" ::"v"(ss), "v"(dot) : "memory");
                load_group(gn, xn, dn);
                finish(g, xv, dv, ss, dot);
            }
            sums(xn, dn, ss, dot);
            finish(g, xn, dn, ss, dot);
        }
    }
    if (p.part == nullptr)
        return;
    // this workgroup's partial row: the teams' sums added in team order
    float *prow = p.part + (size_t)blockIdx.x * (size_t)p.hidden;
    if constexpr (kRpb == 1) {
#pragma unroll
        for (int k = 0; k < kVpt; ++k)
            if (in_row[k])
                store_part<kE>(&prow[(k * kTpr + lane) * kE], acc[k], p.part_nt);
    } else {
        __shared__ float red[kBlock * kE];
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kE; ++e)
                red[(team * kTpr + lane) * kE + e] = acc[k][e];
            __syncthreads();
            for (int q = tid; q < kTpr * kE; q += kBlock) {    // q = lane' * kE + e'
                float sum = red[q];
                for (int t = 1; t < kRpb; ++t)
                    sum = sum + red[t * kTpr * kE + q];
                const int piece = k * kTpr + q / kE;
                if ((uint32_t)piece * 16u < row_bytes)
                    store_part<1>(&prow[piece * kE + q % kE], &sum, p.part_nt);
            }
        }
    }
}

// Generic kernel: one team per row, two passes (the two sums, then dx), kEpa
// elements per access; stores each row's rho when dw is wanted.
template <typename T, int kTpr, int kEpa, int kBlock>
__device__ __forceinline__ void bwd_generic_body(const BwdParams &p)
{
    using A = Access<T, kEpa>;
    using V = typename A::V;
    constexpr int kU = kGenericBatch;
    constexpr int kRpb = kBlock / kTpr;
    const int tid = threadIdx.x;
    const int lane = tid % kTpr;
    const int team = tid / kTpr;
    const int64_t row = (int64_t)blockIdx.x * kRpb + team;
    const bool active = row < p.rows;
    const int64_t H = p.hidden;
    const int64_t base = active ? row * H : 0;
    constexpr int64_t kStride = (int64_t)kTpr * kEpa;

    LaneSum ss_sum, dot_sum;
    if (active) {
        for (int64_t j0 = (int64_t)lane * kEpa; j0 < H; j0 += kU * kStride) {
            V xv[kU], dv[kU], wv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t j = j0 + u * kStride;
                if (j < H) {
                    xv[u] = A::load(p.x, base + j);
                    dv[u] = A::load(p.dy, base + j);
                    wv[u] = A::load(p.w, j);
                }
            }
            float bs = 0.0f, bd = 0.0f;
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (j0 + u * kStride < H)
#pragma unroll
                    for (int e = 0; e < kEpa; ++e) {
                        const float xe = A::get(xv[u], e);
                        const float ge = A::get(dv[u], e) * A::get(wv[u], e);
                        bs = __builtin_fmaf(xe, xe, bs);
                        bd = __builtin_fmaf(ge, xe, bd);
                    }
            ss_sum.add(bs);
            dot_sum.add(bd);
        }
    }
    float ss = ss_sum.value(), dot = dot_sum.value();
    team_fold2<kTpr, kBlock>(ss, dot);
    if (!active)
        return;
    const float rho = row_scale(ss, p.hidden, p.eps);
    const float c = ((dot / (float)p.hidden) * rho) * rho;
    if (p.rho != nullptr && lane == 0)
        p.rho[row] = rho;
    for (int64_t j0 = (int64_t)lane * kEpa; j0 < H; j0 += kU * kStride) {
        V xv[kU], dv[kU], wv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = j0 + u * kStride;
            if (j < H) {
                xv[u] = A::load(p.x, base + j);
                dv[u] = A::load(p.dy, base + j);
                wv[u] = A::load(p.w, j);
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = j0 + u * kStride;
            if (j < H) {
                float o[kEpa];
#pragma unroll
                for (int e = 0; e < kEpa; ++e) {
                    const float xe = A::get(xv[u], e);
                    const float ge = A::get(dv[u], e) * A::get(wv[u], e);
                    o[e] = __builtin_fmaf(-c, xe, ge) * rho;
                }
                A::store(p.dx, base + j, o);
            }
        }
    }
}

// Generic path, dw partials: block (blockIdx.x, blockIdx.y) sums the columns
// blockIdx.x * 256 + threadIdx.x over the rows of chunk blockIdx.y (chunks of
// ceil(rows / gridDim.y) consecutive rows), in row order, compensated
// (a chunk may hold thousands of rows).
template <typename T>
__device__ __forceinline__ void bwd_colsum_body(const BwdParams &p)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per = (p.rows + gridDim.y - 1) / gridDim.y;
    const int64_t r0 = (int64_t)blockIdx.y * per;
    const int64_t r1 = r0 + per < p.rows ? r0 + per : p.rows;
    if (j >= p.hidden)
        return;
    LaneSum acc;
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = r * p.hidden + j;
        acc.add(Scalar<T>::get(p.dy, i) * (Scalar<T>::get(p.x, i) * p.rho[r]));
    }
    const float v = acc.value();
    store_part<1>(&p.part[(size_t)blockIdx.y * (size_t)p.hidden + j], &v, p.part_nt);
}

// dw[j] = the nparts partial rows added in a fixed order.  A 256-thread block
// owns kDwCols consecutive columns; thread (slice v, column c) adds rows
// v, v + kDwSlices, v + 2 kDwSlices, ... of its column in turn (loads issued
// in batches, so their latencies overlap: with at most 256 partial rows, a
// thread waits for at most three rounds of loads), then the kDwSlices
// sums of a column are folded in half (v with v + 4, then v + 2, v + 1) and
// rounded to the dtype.  32-column blocks spread a 4096-wide dw over 128
// compute units (64-column, 1024-thread blocks measured 10% slower).  With
// kNt the partial rows are read non-temporal, as they were written.
constexpr int kDwCols = 32;
constexpr int kDwSlices = 8;
constexpr int kDwBlock = kDwCols * kDwSlices;
constexpr int kDwBatch = 32;

struct DwParams {
    void *dw;
    const float *part;
    int32_t nparts;
    int32_t hidden;
};

template <bool kNt>
__device__ __forceinline__ float load_part(const float *a)
{
    if constexpr (kNt)
        return __builtin_nontemporal_load(a);
    else
        return *a;
}

template <typename T, bool kNt>
__device__ __forceinline__ void bwd_dw_body(const DwParams &p)
{
    __shared__ float red[kDwSlices][kDwCols];
    const int c = threadIdx.x % kDwCols;
    const int v = threadIdx.x / kDwCols;
    const int64_t j = (int64_t)blockIdx.x * kDwCols + c;
    float s = 0.0f;
    if (j < p.hidden) {
        const float *col = p.part + j;
        const size_t step = (size_t)kDwSlices * (size_t)p.hidden;
        // kDwBatch, then kDwBatch / 2 rows of the column at a time, so their
        // loads are in flight together; the rows left after that (fewer than
        // kDwBatch / 2) go in one more batch of that size, whose loads past
        // the last partial row read the batch's first row again and whose
        // terms past it are not added (a plain loop over them waited for each
        // load in turn).  The rows are added in order either way.
        int q = v;
        auto batch = [&](auto n) {
            constexpr int kN = decltype(n)::value;
            for (; q + (kN - 1) * kDwSlices < p.nparts; q += kN * kDwSlices) {
                float t[kN];
#pragma unroll
                for (int u = 0; u < kN; ++u)
                    t[u] = load_part<kNt>(&col[(size_t)q * p.hidden + u * step]);
#pragma unroll
                for (int u = 0; u < kN; ++u)
                    s = s + t[u];
            }
        };
        batch(std::integral_constant<int, kDwBatch>{});
        batch(std::integral_constant<int, kDwBatch / 2>{});
        if (q < p.nparts) {
            constexpr int kN = kDwBatch / 2;
            float t[kN];
#pragma unroll
            for (int u = 0; u < kN; ++u) {
                const int r = q + u * kDwSlices < p.nparts ? q + u * kDwSlices : q;
                t[u] = load_part<kNt>(&col[(size_t)r * p.hidden]);
            }
#pragma unroll
            for (int u = 0; u < kN; ++u)
                s = q + u * kDwSlices < p.nparts ? s + t[u] : s;
        }
    }
    red[v][c] = s;
    __syncthreads();
#pragma unroll
    for (int n = kDwSlices / 2; n >= 1; n /= 2) {
        if (v < n)
            red[v][c] = red[v][c] + red[v + n][c];
        __syncthreads();
    }
    if (v == 0 && j < p.hidden)
        Scalar<T>::put(p.dw, j, red[0][c]);
}

// ---------------------------------------------------------------------------
// Kernel entry points, one name per operation and path.  Every kernel takes
// its arguments as scalars (the fields of its parameter struct; the
// backward's sizes ahead of its partial-row pointers) rather than the
// struct: built with kernel-argument preloading, gfx950 then starts every
// wave with them already in SGPRs, where a struct argument would be read
// from the kernel-argument segment first, one memory round trip before the
// first data load can issue.
// ---------------------------------------------------------------------------
template <typename T, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol, bool kWeightLds>
__global__ __launch_bounds__(kBlock) void rms_norm_vec(void *y, const void *x, void *res, const void *w, int64_t rows,
                                                       int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    vec_body<T, false, false, kTpr, kVpt, kBlock, kLoadCpol, kStoreCpol, kWeightLds>(p);
}

template <typename T, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol, bool kWeightLds>
__global__ __launch_bounds__(kBlock) void fused_add_rms_norm_vec(void *y, const void *x, void *res, const void *w,
                                                                 int64_t rows, int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    vec_body<T, true, true, kTpr, kVpt, kBlock, kLoadCpol, kStoreCpol, kWeightLds>(p);
}

template <typename T, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol, bool kWeightLds>
__global__ __launch_bounds__(kBlock) void rms_norm_residual_vec(void *y, const void *x, void *res, const void *w,
                                                                int64_t rows, int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    vec_body<T, true, false, kTpr, kVpt, kBlock, kLoadCpol, kStoreCpol, kWeightLds>(p);
}

template <typename T, int kTpr, int kEpa, int kBlock>
__global__ __launch_bounds__(kBlock) void rms_norm_generic(void *y, const void *x, void *res, const void *w,
                                                           int64_t rows, int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    generic_body<T, false, false, kTpr, kEpa, kBlock>(p);
}

template <typename T, int kTpr, int kEpa, int kBlock>
__global__ __launch_bounds__(kBlock) void fused_add_rms_norm_generic(void *y, const void *x, void *res, const void *w,
                                                                     int64_t rows, int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    generic_body<T, true, true, kTpr, kEpa, kBlock>(p);
}

template <typename T, int kTpr, int kEpa, int kBlock>
__global__ __launch_bounds__(kBlock) void rms_norm_residual_generic(void *y, const void *x, void *res, const void *w,
                                                                    int64_t rows, int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    generic_body<T, true, false, kTpr, kEpa, kBlock>(p);
}

template <typename T, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol>
__global__ __launch_bounds__(kBlock) void silu_and_mul_vec(void *out, const void *x, int64_t rows, int32_t d)
{
    const SwigluParams p{out, x, rows, d};
    swiglu_vec_body<T, kTpr, kVpt, kBlock, kLoadCpol, kStoreCpol>(p);
}

template <typename T>
__global__ __launch_bounds__(256) void silu_and_mul_generic(void *out, const void *x, int64_t rows, int32_t d)
{
    const SwigluParams p{out, x, rows, d};
    swiglu_generic_body<T>(p);
}

template <typename T, int kTpr, int kVpt, int kBlock>
__global__ __launch_bounds__(kBlock) void rms_norm_backward_vec(void *dx, const void *dy, const void *x, const void *w,
                                                                int64_t rows, int32_t hidden, float eps, float *part,
                                                                float *rho, int32_t part_nt)
{
    const BwdParams p{dx, dy, x, w, part, rho, rows, hidden, eps, part_nt};
    bwd_vec_body<T, kTpr, kVpt, kBlock>(p);
}

template <typename T, int kTpr, int kEpa, int kBlock>
__global__ __launch_bounds__(kBlock) void rms_norm_backward_generic(void *dx, const void *dy, const void *x,
                                                                    const void *w, int64_t rows, int32_t hidden,
                                                                    float eps, float *part, float *rho, int32_t part_nt)
{
    const BwdParams p{dx, dy, x, w, part, rho, rows, hidden, eps, part_nt};
    bwd_generic_body<T, kTpr, kEpa, kBlock>(p);
}

template <typename T>
__global__ __launch_bounds__(256) void rms_norm_backward_colsum(void *dx, const void *dy, const void *x, const void *w,
                                                                int64_t rows, int32_t hidden, float eps, float *part,
                                                                float *rho, int32_t part_nt)
{
    const BwdParams p{dx, dy, x, w, part, rho, rows, hidden, eps, part_nt};
    bwd_colsum_body<T>(p);
}

template <typename T, bool kNt>
__global__ __launch_bounds__(kDwBlock) void rms_norm_backward_dw(void *dw, const float *part, int32_t nparts,
                                                               int32_t hidden)
{
    const DwParams p{dw, part, nparts, hidden};
    bwd_dw_body<T, kNt>(p);
}

template <typename T, int kTpr, int kVpt, int kBlock, int kLoadCpol, int kStoreCpol>
__global__ __launch_bounds__(kBlock) void softmax_vec(void *y, const void *x, void *res, const void *w, int64_t rows,
                                                      int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    softmax_vec_body<T, kTpr, kVpt, kBlock, kLoadCpol, kStoreCpol>(p);
}

template <typename T, int kTpr, int kEpa, int kBlock>
__global__ __launch_bounds__(kBlock) void softmax_generic(void *y, const void *x, void *res, const void *w,
                                                          int64_t rows, int32_t hidden, float eps)
{
    const Params p{y, x, res, w, rows, hidden, eps};
    softmax_generic_body<T, kTpr, kEpa, kBlock>(p);
}

template <typename T, int kVpt>
__global__ __launch_bounds__(kSplitLanes) void softmax_split_stats(void *y, const void *x, float *stats, int64_t rows,
                                                                   int32_t hidden, int32_t chunks)
{
    const SplitParams p{y, x, stats, rows, hidden, chunks};
    softmax_split_stats_body<T, kVpt>(p);
}

template <typename T, int kVpt>
__global__ __launch_bounds__(kSplitLanes) void softmax_split_norm(void *y, const void *x, float *stats, int64_t rows,
                                                                  int32_t hidden, int32_t chunks)
{
    const SplitParams p{y, x, stats, rows, hidden, chunks};
    softmax_split_norm_body<T, kVpt>(p);
}

}  // namespace ks
