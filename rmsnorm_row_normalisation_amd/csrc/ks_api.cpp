// C ABI of ks_norm: argument validation, overlap checks, the launch policy
// and the calls into the per-dtype kernel units.  Validation and the policy
// make no HIP call, so they run (and are tested) on machines without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ks_internal.h"
#include "ks_norm.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxHidden = int64_t(1) << 24;   // float(hidden) stays exact
constexpr int64_t kMaxRows = INT32_MAX;             // one workgroup row index per grid slot at most

bool valid_dtype(int dtype)
{
    return dtype == KS_DTYPE_FLOAT32 || dtype == KS_DTYPE_FLOAT16 || dtype == KS_DTYPE_BFLOAT16;
}

int64_t elem_size(ks_dtype_t dtype) { return dtype == KS_DTYPE_FLOAT32 ? 4 : 2; }

bool is_pow2_team(int v) { return v >= ks::kMinTpr && v <= ks::kMaxTpr && (v & (v - 1)) == 0; }

ks_status_t check_sizes(ks_dtype_t dtype, int64_t rows, int64_t hidden, float eps)
{
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (rows < 0 || rows > kMaxRows || hidden <= 0 || hidden > kMaxHidden)
        return KS_ERROR_INVALID_VALUE;
    if (!(eps > 0.0f) || !isfinite(eps))
        return KS_ERROR_INVALID_VALUE;
    return KS_SUCCESS;
}

// Half-open byte ranges [a, a + n) and [b, b + m) share a byte.
bool overlaps(const void *a, int64_t n, const void *b, int64_t m)
{
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + (uintptr_t)m && pb < pa + (uintptr_t)n;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The launch policy.
//
// Row split (sets the summation order, so a function of op, dtype, hidden and
// alignment only): on the vector path (aligned buffers, row bytes a multiple
// of 16) the smallest power-of-two team of 8..1024 lanes that holds the row
// with at most 8 sixteen-byte pieces per lane (4 for 1024-lane teams); rows
// too wide for that take the generic path with 16-byte accesses; everything
// else takes the generic path with scalar accesses and a team sized to the
// row.
//
// Memory hints (speed only): stores are marked non-temporal (the data is not
// re-read by this kernel); loads too, except for rms_norm over batches larger
// than the last-level cache, where default loads measured faster; the fused
// kernel stages the weight in LDS when a workgroup holds several rows.
void choose_hints(ks_op_t op, int64_t rows, int64_t row_bytes, ks_plan_t *plan)
{
    if (plan->path != KS_PATH_VECTOR)
        return;
    const int64_t batch_bytes = rows * row_bytes;
    constexpr int64_t kLargeBatch = int64_t(64) << 20;
    plan->store_nt = 1;
    if (op == KS_OP_RMS_NORM) {
        plan->load_nt = batch_bytes >= kLargeBatch ? 0 : 1;
        plan->weight_lds = 0;
    } else {
        plan->load_nt = 1;
        plan->weight_lds = plan->rows_per_block >= 2 ? 1 : 0;
    }
}

ks_plan_t policy(ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, bool aligned)
{
    ks_plan_t plan;
    memset(&plan, 0, sizeof(plan));
    const int64_t esize = elem_size(dtype);
    const int64_t row_bytes = hidden * esize;
    const int vec_elems = (int)(16 / esize);
    if (aligned && row_bytes % 16 == 0) {
        const int64_t nvec = row_bytes / 16;
        for (int tpr = ks::kMinTpr; tpr <= ks::kMaxTpr; tpr *= 2) {
            const int maxv = tpr == ks::kMaxTpr ? ks::kMaxVptAt1024 : ks::kMaxVpt;
            if (nvec <= (int64_t)tpr * maxv) {
                plan.path = KS_PATH_VECTOR;
                plan.threads_per_row = tpr;
                plan.vectors_per_thread = (int32_t)((nvec + tpr - 1) / tpr);
                plan.elems_per_access = vec_elems;
                plan.block_threads = ks::block_threads_for(tpr);
                plan.rows_per_block = plan.block_threads / tpr;
                choose_hints(op, rows, row_bytes, &plan);
                return plan;
            }
        }
        plan.path = KS_PATH_GENERIC;
        plan.threads_per_row = 1024;
        plan.elems_per_access = vec_elems;
    } else {
        plan.path = KS_PATH_GENERIC;
        plan.threads_per_row = hidden <= 64 ? 8 : hidden <= 2048 ? 64 : hidden <= 16384 ? 256 : 1024;
        plan.elems_per_access = 1;
    }
    plan.vectors_per_thread = 0;
    plan.block_threads = plan.threads_per_row == 1024 ? 1024 : 256;
    plan.rows_per_block = plan.block_threads / plan.threads_per_row;
    return plan;
}

// Whether the hint combination is one of the compiled variants.
bool hints_compiled(const ks_plan_t &p)
{
    const int key = (p.load_nt ? 4 : 0) | (p.store_nt ? 2 : 0) | (p.weight_lds ? 1 : 0);
    if ((p.load_nt | p.store_nt | p.weight_lds) & ~1)
        return false;
    return key == 0 || key == 6 || key == 2 || key == 7;
}

// Whether an explicit plan names a compiled kernel that covers this row and
// suits the buffers' alignment.
bool plan_fits(const ks_plan_t &p, ks_dtype_t dtype, int64_t hidden, bool aligned)
{
    const int64_t esize = elem_size(dtype);
    const int64_t row_bytes = hidden * esize;
    const int vec_elems = (int)(16 / esize);
    const bool vec_ok = aligned && row_bytes % 16 == 0;
    if (p.path == KS_PATH_VECTOR) {
        if (!vec_ok || !is_pow2_team(p.threads_per_row) || !hints_compiled(p))
            return false;
        const int maxv = p.threads_per_row == ks::kMaxTpr ? ks::kMaxVptAt1024 : ks::kMaxVpt;
        if (p.vectors_per_thread < 1 || p.vectors_per_thread > maxv)
            return false;
        if ((int64_t)p.threads_per_row * p.vectors_per_thread * 16 < row_bytes)
            return false;
        return p.elems_per_access == vec_elems && p.block_threads == ks::block_threads_for(p.threads_per_row) &&
               p.rows_per_block == p.block_threads / p.threads_per_row;
    }
    if (p.path == KS_PATH_GENERIC) {
        const int t = p.threads_per_row;
        if (t != 8 && t != 64 && t != 256 && t != 1024)
            return false;
        if (p.vectors_per_thread != 0 || p.load_nt != 0 || p.store_nt != 0 || p.weight_lds != 0)
            return false;
        if (p.elems_per_access != 1 && !(p.elems_per_access == vec_elems && vec_ok))
            return false;
        const int block = t == 1024 ? 1024 : 256;
        return p.block_threads == block && p.rows_per_block == block / t;
    }
    return false;
}

ks_status_t launch(ks::Launch &l, ks_dtype_t dtype)
{
    hipError_t err;
    const bool vec = l.plan.path == KS_PATH_VECTOR;
    switch (dtype) {
    case KS_DTYPE_FLOAT32:
        err = !vec ? ks::launch_generic_f32(l) : l.fused ? ks::launch_vec_f32_fused(l) : ks::launch_vec_f32_rms(l);
        break;
    case KS_DTYPE_FLOAT16:
        err = !vec ? ks::launch_generic_f16(l) : l.fused ? ks::launch_vec_f16_fused(l) : ks::launch_vec_f16_rms(l);
        break;
    default:
        err = !vec ? ks::launch_generic_bf16(l) : l.fused ? ks::launch_vec_bf16_fused(l) : ks::launch_vec_bf16_rms(l);
        break;
    }
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return KS_ERROR_HIP;
    }
    return KS_SUCCESS;
}

ks_status_t select_plan(const ks_plan_t *requested, ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden,
                        bool aligned, ks_plan_t *out)
{
    if (requested == nullptr) {
        *out = policy(op, dtype, rows, hidden, aligned);
        return KS_SUCCESS;
    }
    if (!plan_fits(*requested, dtype, hidden, aligned))
        return KS_ERROR_INVALID_VALUE;
    *out = *requested;
    return KS_SUCCESS;
}

}  // namespace

extern "C" {

ks_status_t ks_rms_norm_ex(void *out, const void *x, const void *weight, int64_t rows, int64_t hidden, float eps,
                           ks_dtype_t dtype, const ks_plan_t *plan, hipStream_t stream)
{
    ks_status_t st = check_sizes(dtype, rows, hidden, eps);
    if (st != KS_SUCCESS)
        return st;
    if (rows > 0 && (out == nullptr || x == nullptr || weight == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(out) && aligned16(x) && aligned16(weight);
    ks::Launch l{out, x, nullptr, weight, rows, (int32_t)hidden, eps, false, {}, stream};
    st = select_plan(plan, KS_OP_RMS_NORM, dtype, rows, hidden, aligned, &l.plan);
    if (st != KS_SUCCESS || rows == 0)
        return st;
    const int64_t es = elem_size(dtype);
    const int64_t nbytes = rows * hidden * es;
    if (out != x && overlaps(out, nbytes, x, nbytes))
        return KS_ERROR_OVERLAP;
    if (overlaps(out, nbytes, weight, hidden * es))
        return KS_ERROR_OVERLAP;
    return launch(l, dtype);
}

ks_status_t ks_rms_norm(void *out, const void *x, const void *weight, int64_t rows, int64_t hidden, float eps,
                        ks_dtype_t dtype, hipStream_t stream)
{
    return ks_rms_norm_ex(out, x, weight, rows, hidden, eps, dtype, nullptr, stream);
}

ks_status_t ks_fused_add_rms_norm_ex(void *x, void *residual, const void *weight, int64_t rows, int64_t hidden,
                                     float eps, ks_dtype_t dtype, const ks_plan_t *plan, hipStream_t stream)
{
    ks_status_t st = check_sizes(dtype, rows, hidden, eps);
    if (st != KS_SUCCESS)
        return st;
    if (rows > 0 && (x == nullptr || residual == nullptr || weight == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(x) && aligned16(residual) && aligned16(weight);
    ks::Launch l{x, x, residual, weight, rows, (int32_t)hidden, eps, true, {}, stream};
    st = select_plan(plan, KS_OP_FUSED_ADD_RMS_NORM, dtype, rows, hidden, aligned, &l.plan);
    if (st != KS_SUCCESS || rows == 0)
        return st;
    const int64_t es = elem_size(dtype);
    const int64_t nbytes = rows * hidden * es;
    if (overlaps(x, nbytes, residual, nbytes) || overlaps(x, nbytes, weight, hidden * es) ||
        overlaps(residual, nbytes, weight, hidden * es))
        return KS_ERROR_OVERLAP;
    return launch(l, dtype);
}

ks_status_t ks_fused_add_rms_norm(void *x, void *residual, const void *weight, int64_t rows, int64_t hidden,
                                  float eps, ks_dtype_t dtype, hipStream_t stream)
{
    return ks_fused_add_rms_norm_ex(x, residual, weight, rows, hidden, eps, dtype, nullptr, stream);
}

ks_status_t ks_get_plan(ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, int aligned, ks_plan_t *plan)
{
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (plan == nullptr || rows < 0 || rows > kMaxRows || hidden <= 0 || hidden > kMaxHidden ||
        (op != KS_OP_RMS_NORM && op != KS_OP_FUSED_ADD_RMS_NORM))
        return KS_ERROR_INVALID_VALUE;
    *plan = policy(op, dtype, rows, hidden, aligned != 0);
    return KS_SUCCESS;
}

const char *ks_status_string(ks_status_t status)
{
    switch (status) {
    case KS_SUCCESS: return "KS_SUCCESS";
    case KS_ERROR_INVALID_VALUE: return "KS_ERROR_INVALID_VALUE: bad size, eps, pointer or plan";
    case KS_ERROR_UNSUPPORTED_DTYPE: return "KS_ERROR_UNSUPPORTED_DTYPE: dtype must be float32, float16 or bfloat16";
    case KS_ERROR_OVERLAP: return "KS_ERROR_OVERLAP: buffers overlap where the operation forbids it";
    case KS_ERROR_HIP: return "KS_ERROR_HIP: the HIP runtime reported an error (see ks_last_hip_error)";
    default: return "unknown ks_status_t";
    }
}

int ks_last_hip_error(void) { return g_last_hip_error; }

const char *ks_version(void) { return "ks_norm 0.1.0 gfx950"; }

}  // extern "C"
