// C ABI of ks_norm: argument validation, overlap checks, the launch policy
// and the calls into the per-dtype kernel units (RMSNorm forward and
// backward, fused residual-add RMSNorm in place and out of place, SwiGLU,
// softmax).  Validation and the policy
// make no HIP call, so they run (and are tested) on machines without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ks_internal.h"
#include "ks_norm.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local ks::TimingRequest g_timing;

// Clears the calling thread's timing request when an entry point returns, so
// that a request applies to exactly one call (whether or not it launched).
struct TimingScope {
    ~TimingScope() { g_timing = ks::TimingRequest{}; }
};

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

// Half-open byte ranges [a, a + n) and [b, b + m) share a byte (an empty
// range shares none).
bool overlaps(const void *a, int64_t n, const void *b, int64_t m)
{
    if (n <= 0 || m <= 0)
        return false;
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + (uintptr_t)m && pb < pa + (uintptr_t)n;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The launch policy: a function of op, dtype, rows, hidden and alignment.
// (Every vector plan sums a row in the same canonical order, so choosing the
// launch shape from the batch size never changes a result.  The one
// exception is the split softmax, which only calls with a workspace get.)
//
// Vector path (aligned buffers, row bytes a multiple of 16, rows up to 128 KiB):
//   * work units are the row's 16-byte pieces; a batch holds rows * nvec;
//   * pieces per lane aim at spreading the batch over 512 lanes per compute
//     unit (8 waves on each; 131072 lanes on 256 compute units), between 1
//     and 8 per lane, at most 4 for batches of 16384 pieces per compute unit
//     or more (4M on 256; more waves in flight stream better there);
//   * the team is the power of two of lanes that covers the row with that
//     many pieces, between 8 and 512 lanes (1024-lane workgroups measured
//     slower);
//   * loads and stores are marked non-temporal: the data is streamed once;
//   * the fused kernel stages the weight in LDS from 1024 pieces per compute
//     unit up (2^18 on 256), where several rows per compute unit share it;
//     below that the staging barrier costs more than the L2 re-reads it
//     saves.
// The two forms that add a residual (in place and out of place) read two
// streams per row: in large batches they take at most 2 pieces per lane and
// teams of up to 1024 lanes.  The out-of-place form never stages the weight
// in LDS (measured slower at every batch size).
// These rules were fitted to timings of every compiled shape and hint
// combination for hidden 1024..16384 and 1..32768 rows (bf16).
// Rows of 64..128 KiB take 1024-lane teams (5..8 pieces per lane); wider
// rows, or unaligned buffers, take the generic path.
//
// Softmax keeps every element of its piece in registers as an fp32
// exponential between the two reductions, so it takes at most 4 pieces per
// lane, and 2 from 4M pieces (fitted to timings for hidden 128..16384 and
// 1..8192 rows, bf16).
//
// SwiGLU (pieces are 16-byte pieces of the output row, each reading two input
// pieces) has no reduction and about three times the arithmetic per byte, so
// it wants more, shorter lanes: at most 2 pieces per lane, and a 1024-lane
// team where that covers the row with no more idle piece slots than a
// 512-lane team does.  Fitted to timings for output widths 1024..14336 and
// 1..8192 rows (bf16, fp16).
// The batch-size thresholds scale with the device's compute units (a whole
// MI355X has 256; a partitioned one exposes fewer): per compute unit, 512
// target lanes (131072 on 256), a large batch from 16384 pieces (4M) and LDS
// weight staging from 1024 pieces (2^18).
constexpr int64_t kTargetLanesPerCu = 512;
constexpr int64_t kLargeBatchPiecesPerCu = 16384;
constexpr int64_t kWeightLdsPiecesPerCu = 1024;
constexpr int kPolicyMaxTpr = 512;
constexpr int64_t kSwigluMaxVpt = 2;

int64_t pow2_ceil(int64_t v)
{
    int64_t p = 1;
    while (p < v)
        p *= 2;
    return p;
}

// RMSNorm backward (vector path).  Workgroups walk row groups (at most 256
// workgroups, one fp32 partial row of dw each); x and dy loads and dx
// stores non-temporal.  Fitted to graph-timed sweeps of every compiled plan
// (1024-thread workgroups with up to 3 (fp32) or 2 pieces per lane, 512-thread
// ones with up to 4) over hidden 512..16384, 64..32768 rows, bf16 and fp32
// with fp16 spot checks: 0.8% slower than the best plan per case on average
// (worst 9%), against 10% (worst 44%) for the fewest lanes on 1024 threads.
//   * below 2048 rows: 512-thread workgroups, the team the power of two
//     covering the row (up to 512 lanes) with one piece per lane, so the
//     batch spreads over as many workgroups as it can;
//   * 2048..32767 rows: 512-thread workgroups, rows of up to 512 pieces on
//     teams of up to 128 lanes (up to 4 pieces per lane), rows of 513..1024
//     pieces on 512 lanes with 2;
//   * from 32768 rows: 1024-thread workgroups with one piece per lane for
//     rows of up to 1024 pieces;
//   * rows over 1024 pieces: 512 lanes of 512-thread workgroups with up to 4
//     pieces per lane; fp32 rows over 2048 pieces (up to 3072): 1024 lanes
//     with 3.
constexpr int64_t kBwdMidRows = 2048;
constexpr int64_t kBwdHugeRows = 32768;
constexpr int64_t kBwdMidTeam = 128;

ks_plan_t backward_vector_plan(int64_t rows, int64_t nvec, int vec_elems)
{
    ks_plan_t plan;
    memset(&plan, 0, sizeof(plan));
    int64_t block = ks::kBwdBlockHalf;
    int64_t tpr = pow2_ceil(nvec);
    if ((nvec <= ks::kMaxTpr && rows >= kBwdHugeRows) || nvec > (int64_t)ks::kBwdBlockHalf * ks::kBwdMaxVptHalf)
        block = ks::kBwdBlock;
    else if (nvec <= ks::kBwdBlockHalf && rows >= kBwdMidRows && tpr > kBwdMidTeam)
        tpr = kBwdMidTeam;
    tpr = tpr < ks::kMinTpr ? ks::kMinTpr : tpr > block ? block : tpr;
    plan.path = KS_PATH_VECTOR;
    plan.threads_per_row = (int32_t)tpr;
    plan.vectors_per_thread = (int32_t)((nvec + tpr - 1) / tpr);
    plan.elems_per_access = vec_elems;
    plan.block_threads = (int32_t)block;
    plan.rows_per_block = (int32_t)(block / tpr);
    plan.load_nt = 1;
    plan.store_nt = 1;
    return plan;
}

// Split softmax (only where the caller gives a workspace): a split plan pays
// two launches and a second read of x, and wins where one workgroup per row
// leaves most compute units idle for long:
//   * rows wider than the vector path (over 8192 pieces, where the one-pass
//     plan is the three-pass generic one): any batch;
//   * rows of 4096..8192 pieces: batches of at most 4 rows (4096..5119
//     pieces), 16 (5120..6143) or 32 (6144..8192).
// Pieces per lane: 1 while a one-piece split has at most 1024 workgroups,
// 2 up to 4096, else 4 (longer chunks for large grids).
// Fitted to timings of the one-pass policy plan against every split plan for
// hidden 4096..131072 and 1..2048 rows (bf16, fp16, fp32) on 256 compute
// units; the row and workgroup counts scale with the compute units (rounded
// up, so a row count never drops to zero).
constexpr int64_t kSplitVectorPieces = 8192;

int64_t per_device(int64_t at_256_cus, int64_t cus) { return (at_256_cus * cus + 255) / 256; }

int64_t split_max_rows(int64_t nvec, int64_t cus)
{
    const int64_t at256 = nvec >= 6144 ? 32 : nvec >= 5120 ? 16 : nvec >= 4096 ? 4 : 0;
    return nvec > kSplitVectorPieces ? ks::kSplitMaxRows : per_device(at256, cus);
}

bool split_policy(ks_op_t op, int64_t rows, int64_t nvec, bool vec_ok, int64_t cus, ks_plan_t *plan)
{
    if (op != KS_OP_SOFTMAX || !vec_ok || rows > split_max_rows(nvec, cus))
        return false;
    const int64_t groups = rows * ks::split_chunks(nvec * 16, 1);
    plan->path = KS_PATH_SPLIT;
    plan->threads_per_row = ks::kSplitBlock;
    plan->vectors_per_thread = groups <= per_device(1024, cus) ? 1 : groups <= per_device(4096, cus) ? 2 : 4;
    plan->rows_per_block = 1;
    plan->block_threads = ks::kSplitBlock;
    plan->load_nt = 1;
    plan->store_nt = 1;
    return true;
}

// RMSNorm and its two residual forms on rows of 1024..2048 pieces (16..32
// KiB) in a batch that is not large: 16 pieces per lane on a one- or two-wave
// team (64 or 128 lanes), when that plan's grid comes to 1.75..2 workgroups of
// 4 (2) rows per compute unit.  There the 8-piece plan (two or four waves per
// row, joined through LDS and a barrier) measured slower per call: rms_norm by
// 10-24% (fp32 4096 and 16-bit 8192 wide at 1792..2048 rows, fp32 8192 and
// 16-bit 16384 wide at 920..1024 rows), the fused form by 4-12% (weight in
// LDS, as its rule above gives it) and the out-of-place form by 2-6% (weight
// not in LDS, as its rule gives it).  At other grids the 16-piece plans ranged
// from 19% slower to 7% faster, so they stay in this band.  rms_norm stages the
// weight in LDS for 16-bit dtypes (164 VGPRs against 218; 18-22% against
// 13-16% faster), not for fp32 (10-19% against 0-12%).
// rms_norm in batches of at least 32 rows per compute unit (8192 on 256):
// rows of exactly 1024 pieces (16 KiB) take 512 lanes x 2 pieces with the
// weight staged in LDS, 16-bit rows of exactly 2048 pieces (32 KiB) 128
// lanes x 16 pieces.  Against the large-batch plans (256 x 4, 512 x 4) they
// measured 1-2% faster at 8192 rows and 2.4-7% at 16384..32768 rows (hidden
// 8192 and 16384 in bf16 and fp16, 4096 in fp32; graph-timed, two passes
// each, bf16 on two boxes); at 4096 rows they were even or up to 1% slower, and
// fp32 rows of 2048 pieces were slower on 16 pieces per lane.
constexpr int64_t kHugeRmsRowsPerCu = 32;

bool huge_rms_plan(ks_op_t op, int64_t rows, int64_t nvec, int64_t esize, int64_t cus, int64_t *tpr, int64_t *vpt,
                   bool *weight_lds)
{
    if (op != KS_OP_RMS_NORM || rows < kHugeRmsRowsPerCu * cus)
        return false;
    if (nvec == 1024) {
        *tpr = 512;
        *vpt = 2;
        *weight_lds = true;
        return true;
    }
    if (nvec == 2048 && esize == 2) {
        *tpr = 128;
        *vpt = ks::kWideVpt;
        *weight_lds = false;
        return true;
    }
    return false;
}

bool wide_row_plan(ks_op_t op, int64_t rows, int64_t nvec, bool large, int64_t cus)
{
    if ((op != KS_OP_RMS_NORM && op != KS_OP_FUSED_ADD_RMS_NORM && op != KS_OP_RMS_NORM_RESIDUAL) || large ||
        nvec < 1024 || nvec > 2048)
        return false;
    const int64_t rows_per_group = nvec <= 1024 ? 4 : 2;
    const int64_t groups = (rows + rows_per_group - 1) / rows_per_group;
    return 4 * groups >= 7 * cus && groups <= 2 * cus;
}

// cus: the device's compute units (ks::kDefaultComputeUnits when unknown).
ks_plan_t policy(ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, bool aligned, bool split_ok,
                 int64_t cus)
{
    ks_plan_t plan;
    memset(&plan, 0, sizeof(plan));
    const int64_t esize = elem_size(dtype);
    const int64_t row_bytes = hidden * esize;
    const int vec_elems = (int)(16 / esize);
    const int64_t nvec = row_bytes / 16;
    const int bwd_vpt = ks::bwd_max_vpt((int)esize);
    if (split_ok && split_policy(op, rows, nvec, aligned && row_bytes % 16 == 0, cus, &plan)) {
        plan.elems_per_access = vec_elems;
        return plan;
    }
    if (op == KS_OP_RMS_NORM_BACKWARD && aligned && row_bytes % 16 == 0 &&
        (nvec <= (int64_t)ks::kBwdBlockHalf * ks::kBwdMaxVptHalf || nvec <= (int64_t)ks::kBwdBlock * bwd_vpt))
        return backward_vector_plan(rows, nvec, vec_elems);
    if (op != KS_OP_RMS_NORM_BACKWARD && aligned && row_bytes % 16 == 0 && nvec <= (int64_t)ks::kMaxTpr * ks::kMaxVpt) {
        const int64_t pieces = rows * nvec;
        const bool swiglu = op == KS_OP_SILU_AND_MUL;
        const bool adds_residual = op == KS_OP_FUSED_ADD_RMS_NORM || op == KS_OP_RMS_NORM_RESIDUAL;
        const bool large = pieces >= kLargeBatchPiecesPerCu * cus;
        const int64_t target_lanes = kTargetLanesPerCu * cus;
        const int64_t max_vpt = swiglu                  ? kSwigluMaxVpt
                                : op == KS_OP_SOFTMAX ? (large ? 2 : 4)
                                : adds_residual && large ? 2
                                : large                 ? 4
                                                        : ks::kMaxVpt;
        int64_t vpt = pow2_ceil((pieces + target_lanes - 1) / target_lanes);
        vpt = vpt < 1 ? 1 : vpt > max_vpt ? max_vpt : vpt;
        int64_t tpr = pow2_ceil((nvec + vpt - 1) / vpt);
        if (swiglu && tpr > kPolicyMaxTpr) {
            const int64_t slots512 = (nvec + kPolicyMaxTpr - 1) / kPolicyMaxTpr * kPolicyMaxTpr;
            const int64_t slots1024 = (nvec + ks::kMaxTpr - 1) / ks::kMaxTpr * ks::kMaxTpr;
            tpr = slots1024 <= slots512 ? ks::kMaxTpr : kPolicyMaxTpr;
        }
        const bool wide = nvec > (int64_t)kPolicyMaxTpr * ks::kMaxVpt;   // rows over 64 KiB
        const int64_t max_tpr = (swiglu || wide || (adds_residual && large)) ? ks::kMaxTpr : kPolicyMaxTpr;
        tpr = tpr < ks::kMinTpr ? ks::kMinTpr : tpr > max_tpr ? max_tpr : tpr;
        if (wide)
            tpr = ks::kMaxTpr;
        // the in-place fused form in a large batch: a row of a whole multiple
        // of 1024 pieces (within the piece cap) takes a 1024-lane team, e.g.
        // one piece per lane for 8192-wide bf16 rows (measured 1-3% faster
        // than 512 lanes x 2 at 16384..65536 rows of 8192; other widths keep
        // the rule above, which measured as fast or faster)
        if (op == KS_OP_FUSED_ADD_RMS_NORM && large && nvec % ks::kMaxTpr == 0 && nvec / ks::kMaxTpr <= max_vpt)
            tpr = ks::kMaxTpr;
        int64_t pieces_per_lane = (nvec + tpr - 1) / tpr;
        if (op == KS_OP_RMS_NORM_RESIDUAL && tpr == ks::kMaxTpr && pieces_per_lane == 7)
            pieces_per_lane = 8;   // the 7-piece build of this form spills registers
        bool weight_lds = op == KS_OP_FUSED_ADD_RMS_NORM && pieces >= kWeightLdsPiecesPerCu * cus;
        if (wide_row_plan(op, rows, nvec, large, cus)) {
            tpr = nvec <= 1024 ? 64 : 128;
            pieces_per_lane = ks::kWideVpt;
            if (op == KS_OP_RMS_NORM)
                weight_lds = esize == 2;
        }
        huge_rms_plan(op, rows, nvec, esize, cus, &tpr, &pieces_per_lane, &weight_lds);
        plan.path = KS_PATH_VECTOR;
        plan.threads_per_row = (int32_t)tpr;
        plan.vectors_per_thread = (int32_t)pieces_per_lane;
        plan.elems_per_access = vec_elems;
        plan.block_threads = ks::block_threads_for((int)tpr);
        plan.rows_per_block = plan.block_threads / (int32_t)tpr;
        plan.load_nt = 1;
        plan.store_nt = 1;
        plan.weight_lds = weight_lds ? 1 : 0;
        return plan;
    }
    plan.path = KS_PATH_GENERIC;
    if (op == KS_OP_SILU_AND_MUL) {            // elementwise grid-stride loop
        plan.threads_per_row = ks::kSwigluGenericBlock;
        plan.elems_per_access = 1;
    } else if (aligned && row_bytes % 16 == 0) {
        plan.threads_per_row = 1024;
        plan.elems_per_access = vec_elems;
    } else {
        plan.threads_per_row = hidden <= 64 ? 8 : hidden <= 2048 ? 64 : hidden <= 16384 ? 256 : 1024;
        plan.elems_per_access = 1;
    }
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
bool plan_fits(const ks_plan_t &p, ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, bool aligned,
               bool split_ok)
{
    if (op == KS_OP_SOFTMAX && p.weight_lds != 0)
        return false;
    if (p.path == KS_PATH_SPLIT) {
        const int64_t row_bytes = hidden * elem_size(dtype);
        const int v = p.vectors_per_thread;
        return split_ok && op == KS_OP_SOFTMAX && aligned && row_bytes % 16 == 0 && rows <= ks::kSplitMaxRows &&
               p.threads_per_row == ks::kSplitBlock && (v == 1 || v == 2 || v == 4) &&
               p.elems_per_access == (int)(16 / elem_size(dtype)) && p.rows_per_block == 1 &&
               p.block_threads == ks::kSplitBlock && p.load_nt == 1 && p.store_nt == 1;
    }
    if (op == KS_OP_SILU_AND_MUL) {
        if (p.weight_lds != 0)
            return false;
        if (p.path == KS_PATH_GENERIC)
            return p.threads_per_row == ks::kSwigluGenericBlock && p.vectors_per_thread == 0 &&
                   p.elems_per_access == 1 && p.rows_per_block == 1 && p.block_threads == ks::kSwigluGenericBlock &&
                   p.load_nt == 0 && p.store_nt == 0;
    }
    const int64_t esize = elem_size(dtype);
    const int64_t row_bytes = hidden * esize;
    const int vec_elems = (int)(16 / esize);
    const bool vec_ok = aligned && row_bytes % 16 == 0;
    if (op == KS_OP_RMS_NORM_BACKWARD && p.path == KS_PATH_VECTOR) {
        if (p.block_threads != ks::kBwdBlock && p.block_threads != ks::kBwdBlockHalf)
            return false;
        if (!vec_ok || !is_pow2_team(p.threads_per_row) || p.threads_per_row > p.block_threads ||
            p.vectors_per_thread < 1 || p.vectors_per_thread > ks::bwd_max_vpt((int)esize, p.block_threads))
            return false;
        if ((int64_t)p.threads_per_row * p.vectors_per_thread * 16 < row_bytes)
            return false;
        return p.elems_per_access == vec_elems && p.rows_per_block == p.block_threads / p.threads_per_row &&
               p.load_nt == 1 && p.store_nt == 1 && p.weight_lds == 0;
    }
    if (p.path == KS_PATH_VECTOR) {
        if (!vec_ok || !is_pow2_team(p.threads_per_row) || !hints_compiled(p))
            return false;
        if (p.vectors_per_thread < 1 ||
            (p.vectors_per_thread > ks::kMaxVpt &&
             !(p.vectors_per_thread == ks::kWideVpt && ks::wide_vpt_compiled(op, p.threads_per_row))))
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
    const ks_op_t op = l.op;
    switch (dtype) {
    case KS_DTYPE_FLOAT32:
        err = op == KS_OP_SOFTMAX                 ? ks::launch_softmax_f32(l)
              : !vec                              ? ks::launch_generic_f32(l)
              : op == KS_OP_FUSED_ADD_RMS_NORM    ? ks::launch_vec_f32_fused(l)
              : op == KS_OP_RMS_NORM_RESIDUAL     ? ks::launch_vec_f32_residual(l)
                                                  : ks::launch_vec_f32_rms(l);
        break;
    case KS_DTYPE_FLOAT16:
        err = op == KS_OP_SOFTMAX                 ? ks::launch_softmax_f16(l)
              : !vec                              ? ks::launch_generic_f16(l)
              : op == KS_OP_FUSED_ADD_RMS_NORM    ? ks::launch_vec_f16_fused(l)
              : op == KS_OP_RMS_NORM_RESIDUAL     ? ks::launch_vec_f16_residual(l)
                                                  : ks::launch_vec_f16_rms(l);
        break;
    default:
        err = op == KS_OP_SOFTMAX                 ? ks::launch_softmax_bf16(l)
              : !vec                              ? ks::launch_generic_bf16(l)
              : op == KS_OP_FUSED_ADD_RMS_NORM    ? ks::launch_vec_bf16_fused(l)
              : op == KS_OP_RMS_NORM_RESIDUAL     ? ks::launch_vec_bf16_residual(l)
                                                  : ks::launch_vec_bf16_rms(l);
        break;
    }
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return KS_ERROR_HIP;
    }
    return KS_SUCCESS;
}

// Check an explicit plan (no HIP call).  Without one the policy's plan is
// taken later, by policy_plan, once every argument check has passed: it
// needs the device's compute units, which is a HIP query.
ks_status_t check_plan(const ks_plan_t *requested, ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden,
                       bool aligned, bool split_ok = false)
{
    if (requested != nullptr && !plan_fits(*requested, op, dtype, rows, hidden, aligned, split_ok))
        return KS_ERROR_INVALID_VALUE;
    return KS_SUCCESS;
}

// The device's compute units, or the whole-MI355X default when no device is
// visible (a query of the plan on a machine without a GPU).
int64_t compute_units()
{
    const int cus = ks::device_compute_units();
    return cus > 0 ? cus : ks::kDefaultComputeUnits;
}

ks_plan_t plan_for(const ks_plan_t *requested, ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden,
                   bool aligned, bool split_ok = false)
{
    return requested != nullptr ? *requested : policy(op, dtype, rows, hidden, aligned, split_ok, compute_units());
}

// Workspace bytes of a softmax plan: a (maximum, sum) pair per chunk on the
// split path, none otherwise.
size_t softmax_workspace_bytes(const ks_plan_t &p, int64_t rows, int64_t row_bytes)
{
    if (p.path != KS_PATH_SPLIT || p.vectors_per_thread < 1)
        return 0;
    return (size_t)ks::split_workspace_floats(rows, row_bytes, p.vectors_per_thread) * sizeof(float);
}

// Softmax with or without a workspace (split_ok: the caller passed one, so
// the policy may pick a split plan and an explicit split plan is accepted).
ks_status_t softmax_call(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype, void *workspace,
                         size_t workspace_bytes, const ks_plan_t *plan, hipStream_t stream, bool split_ok)
{
    const TimingScope timing;
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (rows < 0 || rows > kMaxRows || hidden <= 0 || hidden > kMaxHidden)
        return KS_ERROR_INVALID_VALUE;
    if (rows > 0 && (out == nullptr || x == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(out) && aligned16(x);
    ks::Launch l{out, x, nullptr, nullptr, rows, (int32_t)hidden, 0.0f, KS_OP_SOFTMAX, {}, stream};
    ks_status_t st = check_plan(plan, KS_OP_SOFTMAX, dtype, rows, hidden, aligned, split_ok);
    if (st != KS_SUCCESS || rows == 0)       // an empty batch needs no workspace
        return st;
    l.plan = plan_for(plan, KS_OP_SOFTMAX, dtype, rows, hidden, aligned, split_ok);
    const int64_t nbytes = rows * hidden * elem_size(dtype);
    const size_t need = softmax_workspace_bytes(l.plan, rows, hidden * elem_size(dtype));
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 3u) != 0))
        return KS_ERROR_INVALID_VALUE;
    if (out != x && overlaps(out, nbytes, x, nbytes))
        return KS_ERROR_OVERLAP;
    if (overlaps(workspace, (int64_t)need, out, nbytes) || overlaps(workspace, (int64_t)need, x, nbytes))
        return KS_ERROR_OVERLAP;
    l.work = (float *)workspace;
    return launch(l, dtype);
}

}  // namespace

namespace ks {

// The checks ks_softmax_ws makes first (dtype, sizes, null pointers) and the
// bytes of workspace the plan it would pick needs for these buffers (0 for a
// one-pass plan or an empty batch).  The only HIP call is the device's
// compute-unit query behind the policy (once per device).
ks_status_t softmax_ws_need(const void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                            size_t *need)
{
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (rows < 0 || rows > kMaxRows || hidden <= 0 || hidden > kMaxHidden)
        return KS_ERROR_INVALID_VALUE;
    if (rows > 0 && (out == nullptr || x == nullptr))
        return KS_ERROR_INVALID_VALUE;
    if (rows == 0) {
        *need = 0;
        return KS_SUCCESS;
    }
    const ks_plan_t p = policy(KS_OP_SOFTMAX, dtype, rows, hidden, aligned16(out) && aligned16(x), true,
                               compute_units());
    *need = softmax_workspace_bytes(p, rows, hidden * elem_size(dtype));
    return KS_SUCCESS;
}

void record_hip_error(int err) { g_last_hip_error = err; }

TimingRequest &timing_request() { return g_timing; }

}  // namespace ks

extern "C" {

ks_status_t ks_rms_norm_ex(void *out, const void *x, const void *weight, int64_t rows, int64_t hidden, float eps,
                           ks_dtype_t dtype, const ks_plan_t *plan, hipStream_t stream)
{
    const TimingScope timing;
    ks_status_t st = check_sizes(dtype, rows, hidden, eps);
    if (st != KS_SUCCESS)
        return st;
    if (rows > 0 && (out == nullptr || x == nullptr || weight == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(out) && aligned16(x) && aligned16(weight);
    ks::Launch l{out, x, nullptr, weight, rows, (int32_t)hidden, eps, KS_OP_RMS_NORM, {}, stream};
    st = check_plan(plan, KS_OP_RMS_NORM, dtype, rows, hidden, aligned);
    if (st != KS_SUCCESS || rows == 0)
        return st;
    const int64_t es = elem_size(dtype);
    const int64_t nbytes = rows * hidden * es;
    if (out != x && overlaps(out, nbytes, x, nbytes))
        return KS_ERROR_OVERLAP;
    if (overlaps(out, nbytes, weight, hidden * es))
        return KS_ERROR_OVERLAP;
    l.plan = plan_for(plan, KS_OP_RMS_NORM, dtype, rows, hidden, aligned);
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
    const TimingScope timing;
    ks_status_t st = check_sizes(dtype, rows, hidden, eps);
    if (st != KS_SUCCESS)
        return st;
    if (rows > 0 && (x == nullptr || residual == nullptr || weight == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(x) && aligned16(residual) && aligned16(weight);
    ks::Launch l{x, x, residual, weight, rows, (int32_t)hidden, eps, KS_OP_FUSED_ADD_RMS_NORM, {}, stream};
    st = check_plan(plan, KS_OP_FUSED_ADD_RMS_NORM, dtype, rows, hidden, aligned);
    if (st != KS_SUCCESS || rows == 0)
        return st;
    const int64_t es = elem_size(dtype);
    const int64_t nbytes = rows * hidden * es;
    if (overlaps(x, nbytes, residual, nbytes) || overlaps(x, nbytes, weight, hidden * es) ||
        overlaps(residual, nbytes, weight, hidden * es))
        return KS_ERROR_OVERLAP;
    l.plan = plan_for(plan, KS_OP_FUSED_ADD_RMS_NORM, dtype, rows, hidden, aligned);
    return launch(l, dtype);
}

ks_status_t ks_fused_add_rms_norm(void *x, void *residual, const void *weight, int64_t rows, int64_t hidden,
                                  float eps, ks_dtype_t dtype, hipStream_t stream)
{
    return ks_fused_add_rms_norm_ex(x, residual, weight, rows, hidden, eps, dtype, nullptr, stream);
}

ks_status_t ks_rms_norm_residual_ex(void *out, const void *x, const void *residual, const void *weight,
                                   int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype,
                                   const ks_plan_t *plan, hipStream_t stream)
{
    const TimingScope timing;
    ks_status_t st = check_sizes(dtype, rows, hidden, eps);
    if (st != KS_SUCCESS)
        return st;
    if (rows > 0 && (out == nullptr || x == nullptr || residual == nullptr || weight == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(out) && aligned16(x) && aligned16(residual) && aligned16(weight);
    ks::Launch l{out, x, const_cast<void *>(residual), weight, rows, (int32_t)hidden, eps,
                 KS_OP_RMS_NORM_RESIDUAL, {}, stream};
    st = check_plan(plan, KS_OP_RMS_NORM_RESIDUAL, dtype, rows, hidden, aligned);
    if (st != KS_SUCCESS || rows == 0)
        return st;
    const int64_t es = elem_size(dtype);
    const int64_t nbytes = rows * hidden * es;
    // x and residual are only read (they may overlap each other); out may be
    // exactly either of them, and must not touch the weight
    if ((out != x && overlaps(out, nbytes, x, nbytes)) || (out != residual && overlaps(out, nbytes, residual, nbytes)) ||
        overlaps(out, nbytes, weight, hidden * es))
        return KS_ERROR_OVERLAP;
    l.plan = plan_for(plan, KS_OP_RMS_NORM_RESIDUAL, dtype, rows, hidden, aligned);
    return launch(l, dtype);
}

ks_status_t ks_rms_norm_residual(void *out, const void *x, const void *residual, const void *weight, int64_t rows,
                                 int64_t hidden, float eps, ks_dtype_t dtype, hipStream_t stream)
{
    return ks_rms_norm_residual_ex(out, x, residual, weight, rows, hidden, eps, dtype, nullptr, stream);
}

ks_status_t ks_rms_norm_backward_workspace_size(int64_t rows, int64_t hidden, size_t *bytes)
{
    if (bytes == nullptr || rows < 0 || rows > kMaxRows || hidden <= 0 || hidden > kMaxHidden)
        return KS_ERROR_INVALID_VALUE;
    *bytes = (size_t)ks::bwd_workspace_floats(rows, hidden) * sizeof(float);
    return KS_SUCCESS;
}

ks_status_t ks_rms_norm_backward_ex(void *dx, void *dweight, const void *dy, const void *x, const void *weight,
                                    int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype, void *workspace,
                                    size_t workspace_bytes, const ks_plan_t *plan, hipStream_t stream)
{
    const TimingScope timing;
    ks_status_t st = check_sizes(dtype, rows, hidden, eps);
    if (st != KS_SUCCESS)
        return st;
    if (rows > 0 && (dx == nullptr || dy == nullptr || x == nullptr || weight == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const size_t need = (size_t)ks::bwd_workspace_floats(rows, hidden) * sizeof(float);
    if (dweight != nullptr && need > 0 &&
        (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 3u) != 0))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(dx) && aligned16(dy) && aligned16(x) && aligned16(weight);
    ks::BwdLaunch l{dx, dweight, dy, x, weight, (float *)workspace, rows, (int32_t)hidden, eps, {}, stream};
    st = check_plan(plan, KS_OP_RMS_NORM_BACKWARD, dtype, rows, hidden, aligned);
    if (st != KS_SUCCESS || (rows == 0 && dweight == nullptr))
        return st;
    const int64_t es = elem_size(dtype);
    const int64_t nbytes = rows * hidden * es;
    const int64_t wbytes = hidden * es;
    const int64_t kbytes = dweight != nullptr ? (int64_t)need : 0;
    // outputs and workspace touch nothing else; the inputs may overlap each other
    if (overlaps(dx, nbytes, dy, nbytes) || overlaps(dx, nbytes, x, nbytes) || overlaps(dx, nbytes, weight, wbytes) ||
        overlaps(dx, nbytes, dweight, dweight ? wbytes : 0) || overlaps(dx, nbytes, workspace, kbytes))
        return KS_ERROR_OVERLAP;
    if (dweight != nullptr &&
        (overlaps(dweight, wbytes, dy, nbytes) || overlaps(dweight, wbytes, x, nbytes) ||
         overlaps(dweight, wbytes, weight, wbytes) || overlaps(dweight, wbytes, workspace, kbytes) ||
         overlaps(workspace, kbytes, dy, nbytes) || overlaps(workspace, kbytes, x, nbytes) ||
         overlaps(workspace, kbytes, weight, wbytes)))
        return KS_ERROR_OVERLAP;
    l.plan = plan_for(plan, KS_OP_RMS_NORM_BACKWARD, dtype, rows, hidden, aligned);
    hipError_t err;
    switch (dtype) {
    case KS_DTYPE_FLOAT32: err = ks::launch_bwd_f32(l); break;
    case KS_DTYPE_FLOAT16: err = ks::launch_bwd_f16(l); break;
    default: err = ks::launch_bwd_bf16(l); break;
    }
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return KS_ERROR_HIP;
    }
    return KS_SUCCESS;
}

ks_status_t ks_rms_norm_backward(void *dx, void *dweight, const void *dy, const void *x, const void *weight,
                                 int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream)
{
    return ks_rms_norm_backward_ex(dx, dweight, dy, x, weight, rows, hidden, eps, dtype, workspace, workspace_bytes,
                                   nullptr, stream);
}

ks_status_t ks_silu_and_mul_ex(void *out, const void *x, int64_t rows, int64_t d, ks_dtype_t dtype,
                               const ks_plan_t *plan, hipStream_t stream)
{
    const TimingScope timing;
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (rows < 0 || rows > kMaxRows || d <= 0 || d > kMaxHidden)
        return KS_ERROR_INVALID_VALUE;
    if (rows > 0 && (out == nullptr || x == nullptr))
        return KS_ERROR_INVALID_VALUE;
    const bool aligned = aligned16(out) && aligned16(x);
    ks::SwigluLaunch l{out, x, rows, (int32_t)d, {}, stream};
    ks_status_t st = check_plan(plan, KS_OP_SILU_AND_MUL, dtype, rows, d, aligned);
    if (st != KS_SUCCESS || rows == 0)
        return st;
    const int64_t es = elem_size(dtype);
    if (overlaps(out, rows * d * es, x, rows * 2 * d * es))
        return KS_ERROR_OVERLAP;
    l.plan = plan_for(plan, KS_OP_SILU_AND_MUL, dtype, rows, d, aligned);
    hipError_t err;
    switch (dtype) {
    case KS_DTYPE_FLOAT32: err = ks::launch_swiglu_f32(l); break;
    case KS_DTYPE_FLOAT16: err = ks::launch_swiglu_f16(l); break;
    default: err = ks::launch_swiglu_bf16(l); break;
    }
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return KS_ERROR_HIP;
    }
    return KS_SUCCESS;
}

ks_status_t ks_silu_and_mul(void *out, const void *x, int64_t rows, int64_t d, ks_dtype_t dtype, hipStream_t stream)
{
    return ks_silu_and_mul_ex(out, x, rows, d, dtype, nullptr, stream);
}

ks_status_t ks_softmax_ex(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                          const ks_plan_t *plan, hipStream_t stream)
{
    return softmax_call(out, x, rows, hidden, dtype, nullptr, 0, plan, stream, false);
}

ks_status_t ks_softmax(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype, hipStream_t stream)
{
    return softmax_call(out, x, rows, hidden, dtype, nullptr, 0, nullptr, stream, false);
}

ks_status_t ks_softmax_workspace_size(int64_t rows, int64_t hidden, ks_dtype_t dtype, const ks_plan_t *plan,
                                      size_t *bytes)
{
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (bytes == nullptr || rows < 0 || rows > kMaxRows || hidden <= 0 || hidden > kMaxHidden)
        return KS_ERROR_INVALID_VALUE;
    if (plan == nullptr && rows == 0) {
        *bytes = 0;
        return KS_SUCCESS;
    }
    const ks_plan_t p = plan != nullptr ? *plan : policy(KS_OP_SOFTMAX, dtype, rows, hidden, true, true, compute_units());
    *bytes = softmax_workspace_bytes(p, rows, hidden * elem_size(dtype));
    return KS_SUCCESS;
}

ks_status_t ks_softmax_ws_ex(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                             void *workspace, size_t workspace_bytes, const ks_plan_t *plan, hipStream_t stream)
{
    return softmax_call(out, x, rows, hidden, dtype, workspace, workspace_bytes, plan, stream, true);
}

ks_status_t ks_softmax_ws(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype, void *workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    return softmax_call(out, x, rows, hidden, dtype, workspace, workspace_bytes, nullptr, stream, true);
}

ks_status_t ks_get_plan_cus(ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, int flags, int compute_units,
                           ks_plan_t *plan)
{
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (plan == nullptr || rows < 0 || rows > kMaxRows || hidden <= 0 || hidden > kMaxHidden ||
        (flags & ~(KS_PLAN_ALIGNED | KS_PLAN_WORKSPACE)) != 0 || compute_units < 1 ||
        compute_units > ks::kMaxComputeUnits ||
        (op != KS_OP_RMS_NORM && op != KS_OP_FUSED_ADD_RMS_NORM && op != KS_OP_SILU_AND_MUL &&
         op != KS_OP_SOFTMAX && op != KS_OP_RMS_NORM_RESIDUAL && op != KS_OP_RMS_NORM_BACKWARD))
        return KS_ERROR_INVALID_VALUE;
    *plan = policy(op, dtype, rows, hidden, (flags & KS_PLAN_ALIGNED) != 0, (flags & KS_PLAN_WORKSPACE) != 0,
                   compute_units);
    return KS_SUCCESS;
}

ks_status_t ks_get_plan(ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, int flags, ks_plan_t *plan)
{
    if (!valid_dtype(dtype))
        return KS_ERROR_UNSUPPORTED_DTYPE;
    if (plan == nullptr)
        return KS_ERROR_INVALID_VALUE;
    return ks_get_plan_cus(op, dtype, rows, hidden, flags, (int)compute_units(), plan);
}

ks_status_t ks_time_next_call(hipEvent_t start, hipEvent_t stop)
{
    ks::timing_request() = ks::TimingRequest{start, stop};
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
    case KS_ERROR_SCRATCH_LIMIT:
        return "KS_ERROR_SCRATCH_LIMIT: the call needs more scratch than the library's static array holds "
               "(KS_NOALLOC_SCRATCH_BYTES); pass a workspace to ks_softmax_ws instead";
    default: return "unknown ks_status_t";
    }
}

int ks_last_hip_error(void) { return g_last_hip_error; }

#ifndef KS_BUILD_GIT
#define KS_BUILD_GIT "unknown"
#endif
const char *ks_version(void) { return "ks_norm 0.2.0 gfx950 (source " KS_BUILD_GIT ")"; }

}  // extern "C"
