/*
 * ks_norm: RMSNorm row normalisation (forward and backward), fused
 * residual-add RMSNorm, the SwiGLU activation and softmax for AMD Instinct
 * MI355X (gfx950).  C ABI.
 *
 * The operations are the ones defined in the kernscope README, section
 * "Numerical contract" (subsections "RMSNorm", "Fused residual-add RMSNorm",
 * "SwiGLU activation" and "Softmax"), with the input rules of its "Inputs"
 * section, and the out-of-place residual RMSNorm of the Triton Kernels README
 * ("Kernels").  The C-ABI
 * convention (a status code from every entry point, device pointers, an
 * explicit stream) follows the kernel-set README ("What it is", last line of
 * the operator table).
 *
 * Common conventions
 * ------------------
 * Layout     x, out and residual are dense row-major [rows, hidden] arrays
 *            (row stride = hidden elements); weight is a dense [hidden] array.
 *            All buffers hold the same dtype.  There are no stride arguments.
 * Memory     Every pointer is a device pointer owned by the caller.  The
 *            library never allocates, frees, copies or synchronises (scratch
 *            memory, where a call needs it, is a caller-owned workspace, or
 *            for ks_softmax_noalloc a static device array of the library's).
 *            weight is only read.  Any alignment is accepted; 16-byte aligned
 *            buffers with hidden * sizeof(element) a multiple of 16 take the
 *            vector path, others a narrower path with the same contract
 *            (its sums run in another order, so a result may differ from the
 *            vector path's in the last bit).
 * Streams    Work is enqueued on `stream` (0 = the default stream) and the
 *            call returns without waiting.  Calls that overlap in time on
 *            the same buffers race, as with any asynchronous kernel.
 * Arithmetic Per row: widen to fp32; sum of squares in fp32; mean = sum / H
 *            (IEEE division); scale = rsqrt(mean + eps) (eps rounded to fp32;
 *            rsqrt evaluated in double and rounded once to fp32);
 *            y = (v * scale) * fp32(weight);
 *            output rounded to the dtype with round-to-nearest-even.  The
 *            summation order depends only on hidden, dtype and alignment, so
 *            a row's result does not depend on how many rows are in the
 *            batch (the split plans of ks_softmax_ws aside).
 * Errors     Checked in this order, before any kernel launch:
 *              KS_ERROR_UNSUPPORTED_DTYPE  dtype is not one of ks_dtype_t;
 *              KS_ERROR_INVALID_VALUE      rows < 0 or rows > 2^31 - 1;
 *                                          hidden <= 0 or hidden > 2^24;
 *                                          eps not finite or eps <= 0; a
 *                                          NULL pointer while rows > 0; a
 *                                          bad plan; a missing or too small
 *                                          workspace;
 *              KS_ERROR_OVERLAP            forbidden aliasing (per call);
 *            rows == 0 returns KS_SUCCESS without touching HIP (the backward
 *            with a weight gradient still writes dw = 0).  The only HIP calls
 *            before the checks end are those of the device's compute-unit
 *            query (hipGetDevice, and hipDeviceGetAttribute once per device),
 *            which the launch policy reads; with no device visible the
 *            policy assumes a whole MI355X (256 compute units).
 *            KS_ERROR_HIP reports a failed launch (e.g. no device); the HIP
 *            error code is kept per thread in ks_last_hip_error().
 */
#ifndef KS_NORM_H
#define KS_NORM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KS_SUCCESS = 0,
    KS_ERROR_INVALID_VALUE = 1,
    KS_ERROR_UNSUPPORTED_DTYPE = 2,
    KS_ERROR_OVERLAP = 3,
    KS_ERROR_HIP = 4,
    KS_ERROR_SCRATCH_LIMIT = 5      /* ks_softmax_noalloc: the plan needs more scratch than the static array */
} ks_status_t;

typedef enum {
    KS_DTYPE_FLOAT32 = 0,
    KS_DTYPE_FLOAT16 = 1,
    KS_DTYPE_BFLOAT16 = 2
} ks_dtype_t;

typedef enum {
    KS_OP_RMS_NORM = 0,
    KS_OP_FUSED_ADD_RMS_NORM = 1,
    KS_OP_SILU_AND_MUL = 2,
    KS_OP_SOFTMAX = 3,
    KS_OP_RMS_NORM_RESIDUAL = 4,
    KS_OP_RMS_NORM_BACKWARD = 5
} ks_op_t;

/* How a launch maps rows onto threads.
 *   KS_PATH_VECTOR   each thread holds `vectors_per_thread` 16-byte pieces of
 *                    its row in registers; `threads_per_row` threads share a
 *                    row; the row is read once and written once.
 *   KS_PATH_GENERIC  `threads_per_row` threads stride over the row with
 *                    `elems_per_access`-element accesses, in two passes (sum,
 *                    then normalise and store; softmax: three, maximum, sum,
 *                    store); used for unaligned buffers,
 *                    row sizes that are not a multiple of 16 bytes, and rows
 *                    wider than the vector path holds.
 *   KS_PATH_SPLIT    softmax with a workspace only: a row is cut into chunks
 *                    of threads_per_row (256) * vectors_per_thread (1, 2 or
 *                    4) 16-byte pieces, one workgroup per chunk and row, in
 *                    two launches (each chunk's maximum and exponential sum,
 *                    then the combination and the store); for wide rows in
 *                    batches too small to fill the device one row per
 *                    workgroup.  Needs aligned buffers, row bytes a multiple
 *                    of 16 and at most 65535 rows. */
typedef enum {
    KS_PATH_VECTOR = 0,
    KS_PATH_GENERIC = 1,
    KS_PATH_SPLIT = 2
} ks_path_t;

typedef struct {
    int32_t path;               /* ks_path_t */
    int32_t threads_per_row;    /* 8, 16, 32, 64, 128, 256, 512 or 1024 */
    int32_t vectors_per_thread; /* vector path: 1..8, and 16 for RMSNorm and its residual forms
                                   on teams of 32..128 lanes; split path: 1, 2 or 4; generic path: 0 */
    int32_t elems_per_access;   /* generic path: 1 or 16 / element size; vector path: 16 / element size */
    int32_t rows_per_block;     /* rows handled by one workgroup */
    int32_t block_threads;      /* workgroup size */
    /* Vector path (split path: 1, 1, 0; generic path: 0).  Memory hints that change
     * speed, never results; compiled combinations (load_nt, store_nt,
     * weight_lds): (0,0,0), (1,1,0), (0,1,0), (1,1,1). */
    int32_t load_nt;            /* x / residual loads marked non-temporal */
    int32_t store_nt;           /* out / x / residual stores marked non-temporal */
    int32_t weight_lds;         /* weight staged once per workgroup in LDS */
} ks_plan_t;

/*
 * RMSNorm (kernscope README, "Numerical contract" > "RMSNorm"):
 *   out[r, :] = cast( fp32(x[r, :]) * rsqrt(mean(fp32(x[r, :])^2) + eps) * fp32(weight) )
 * out     [rows, hidden] output.  It may be exactly x (in place); any other
 *         overlap of out with x or weight is KS_ERROR_OVERLAP.
 * x       [rows, hidden] input, read only (unless out == x).
 * weight  [hidden], read only.
 */
ks_status_t ks_rms_norm(void *out, const void *x, const void *weight,
                        int64_t rows, int64_t hidden, float eps,
                        ks_dtype_t dtype, hipStream_t stream);

/*
 * Fused residual-add RMSNorm (kernscope README, "Numerical contract" >
 * "Fused residual-add RMSNorm"), in place, from the input snapshots:
 *   s        = fp32(x) + fp32(residual)
 *   residual = cast(s)
 *   x        = cast( s * rsqrt(mean(s^2) + eps) * fp32(weight) )
 * Normalisation uses the unrounded fp32 s.
 * x, residual  [rows, hidden], read and overwritten.
 * weight       [hidden], read only.
 * x, residual and weight must not overlap (KS_ERROR_OVERLAP), as the
 * README's "Inputs" section requires.
 */
ks_status_t ks_fused_add_rms_norm(void *x, void *residual, const void *weight,
                                  int64_t rows, int64_t hidden, float eps,
                                  ks_dtype_t dtype, hipStream_t stream);

/*
 * Out-of-place residual RMSNorm (Triton Kernels README, "Kernels": the
 * residual-fused RMSNorm, RMSNorm(x + residual) * w), with the kernscope
 * fused contract's arithmetic:
 *   s   = fp32(x) + fp32(residual)      (unrounded)
 *   out = cast( s * rsqrt(mean(s^2) + eps) * fp32(weight) )
 * Nothing but out is written: a row moves three times its size (read x and
 * residual, write out) instead of the in-place form's four.
 * out       [rows, hidden] output.  It may be exactly x or exactly residual;
 *           any other overlap with x, residual or weight is KS_ERROR_OVERLAP.
 * x, residual [rows, hidden], read only (they may overlap each other).
 * weight    [hidden], read only.
 * Errors, streams and plans as for ks_rms_norm (op KS_OP_RMS_NORM_RESIDUAL).
 */
ks_status_t ks_rms_norm_residual(void *out, const void *x, const void *residual, const void *weight,
                                 int64_t rows, int64_t hidden, float eps,
                                 ks_dtype_t dtype, hipStream_t stream);

ks_status_t ks_rms_norm_residual_ex(void *out, const void *x, const void *residual, const void *weight,
                                    int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype,
                                    const ks_plan_t *plan, hipStream_t stream);

/*
 * RMSNorm backward: the gradients of ks_rms_norm's contract.  No page states
 * a backward contract; the kernscope README's PyTorch reference of rms_norm
 * supports autograd, so these are the derivatives of
 *   y_j = x_j * rho * w_j,   rho = rsqrt(mean(x^2) + eps)
 * (the final cast passes gradients through), for an incoming gradient dy:
 *   dx_j = rho * (g_j - c * x_j),  g_j = dy_j * w_j,  c = rho^2 * sum_k(g_k * x_k) / H
 *   dw_j = sum over rows of dy_j * (x_j * rho)
 * in fp32 (rho is bit-identical to the forward's scale), rounded to the dtype.
 * dx         [rows, hidden] output.
 * dweight    [hidden] output, or NULL when the weight gradient is not wanted.
 *            With rows == 0 it is set to zero (one launch).
 * dy, x      [rows, hidden], read only.    weight  [hidden], read only.
 * workspace  fp32 scratch owned by the caller, at least
 *            ks_rms_norm_backward_workspace_size(rows, hidden) bytes, 4-byte
 *            aligned; needed only when dweight is not NULL (else may be NULL).
 *            Its contents on entry do not matter and are left undefined.
 * Overlaps: dx, dweight and workspace must not overlap each other or any
 * input (KS_ERROR_OVERLAP); the inputs may overlap each other.
 * dx does not depend on the plan or the batch; dw is summed in a fixed order
 * (deterministic for a given plan and batch size).  A workspace that is
 * missing or too small is KS_ERROR_INVALID_VALUE.  Errors, streams and plans
 * as above (op KS_OP_RMS_NORM_BACKWARD: vector plans use 1024-thread
 * workgroups with at most 3 pieces per lane for fp32 and 2 for 16-bit
 * dtypes, or 512-thread workgroups with at most 4, non-temporal hints on).
 */
ks_status_t ks_rms_norm_backward_workspace_size(int64_t rows, int64_t hidden, size_t *bytes);

ks_status_t ks_rms_norm_backward(void *dx, void *dweight, const void *dy, const void *x, const void *weight,
                                 int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

ks_status_t ks_rms_norm_backward_ex(void *dx, void *dweight, const void *dy, const void *x, const void *weight,
                                    int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype,
                                    void *workspace, size_t workspace_bytes, const ks_plan_t *plan,
                                    hipStream_t stream);

/*
 * The launch plan the calls of this header use for this op, dtype, batch and
 * row size on the current device.  All vector-path plans sum a row in one
 * canonical order, so the plan may change with `rows` (and with the device's
 * compute units) while every row's result stays the same; the path (vector
 * or generic) depends only on dtype, hidden and alignment.
 * `flags`: KS_PLAN_ALIGNED when all buffers are 16-byte aligned;
 * KS_PLAN_WORKSPACE for the plan of a call that passes a workspace
 * (ks_softmax_ws, whose plan may be a split plan; the other ops ignore it).
 * The policy's batch-size thresholds scale with the device's compute units:
 * ks_get_plan reads the current device's count (cached per device; 256, a
 * whole MI355X, when no device is visible); ks_get_plan_cus takes it as an
 * argument (1..4096) and makes no HIP call.  Returns KS_ERROR_INVALID_VALUE
 * for a NULL plan, a bad row count, hidden size or compute-unit count, an
 * unknown op or unknown flag bits.
 */
#define KS_PLAN_ALIGNED 1
#define KS_PLAN_WORKSPACE 2
ks_status_t ks_get_plan(ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, int flags,
                        ks_plan_t *plan);
ks_status_t ks_get_plan_cus(ks_op_t op, ks_dtype_t dtype, int64_t rows, int64_t hidden, int flags,
                            int compute_units, ks_plan_t *plan);

/*
 * Kernel timing without a profiler, per call.  The next call of this header
 * made on the calling thread records `start` when its first kernel begins and
 * `stop` when its last kernel ends (the HIP runtime's kernel-dispatch
 * events, hipExtLaunchKernel); the request then clears, whether or not that
 * call launched anything.  Either event may be NULL.  The events belong to
 * the caller (hipEventCreate, default flags), who reads the interval with
 * hipEventElapsedTime once the stream has reached them.  Kernel-dispatch
 * events are not graph nodes: make no timed call under stream capture.
 * No HIP call here; always KS_SUCCESS.
 */
ks_status_t ks_time_next_call(hipEvent_t start, hipEvent_t stop);

/*
 * The two operations with an explicit launch plan (for tuning and for
 * testing every compiled kernel).
 * plan  NULL = the plan ks_get_plan returns.  Otherwise it must name a
 *       compiled configuration that covers the row and whose path fits the
 *       buffers' alignment; else KS_ERROR_INVALID_VALUE.  Every plan computes
 *       the same contract; plans differ only in the fp32 summation order.
 */
ks_status_t ks_rms_norm_ex(void *out, const void *x, const void *weight,
                           int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype,
                           const ks_plan_t *plan, hipStream_t stream);

ks_status_t ks_fused_add_rms_norm_ex(void *x, void *residual, const void *weight,
                                     int64_t rows, int64_t hidden, float eps, ks_dtype_t dtype,
                                     const ks_plan_t *plan, hipStream_t stream);

/*
 * SwiGLU activation (kernscope README, "Numerical contract" > "SwiGLU
 * activation"; shapes as in its "Inputs" section):
 *   out[r, j] = cast( fp32(g) * sigmoid(fp32(g)) * fp32(u) ),
 *   g = x[r, j], u = x[r, d + j], 0 <= j < d,
 * with fp32 intermediates multiplied left to right; sigmoid(g) = 1 / (1 +
 * exp(-g)) with the device exp (within a few fp32 ulps of the exact value).
 * x    [rows, 2 d] input, gate half first; read only.
 * out  [rows, d] output; must not overlap x (KS_ERROR_OVERLAP).
 * d    output width, 1 <= d <= 2^24 (any parity).  rows may be 0.
 * Errors and stream rules as above.  The vector path needs 16-byte aligned
 * x and out and d * element size a multiple of 16; any other case runs a
 * narrower path with the same result.  Elementwise, so every plan gives the
 * same bits.
 */
ks_status_t ks_silu_and_mul(void *out, const void *x, int64_t rows, int64_t d, ks_dtype_t dtype,
                            hipStream_t stream);

/* SwiGLU with an explicit plan (op KS_OP_SILU_AND_MUL, hidden = d); plans
 * with weight_lds set are rejected, and the generic plan is the single
 * grid-stride one (threads_per_row = block_threads = 256, rows_per_block = 1). */
ks_status_t ks_silu_and_mul_ex(void *out, const void *x, int64_t rows, int64_t d, ks_dtype_t dtype,
                               const ks_plan_t *plan, hipStream_t stream);

/*
 * Softmax over the last dimension (kernscope README, "Numerical contract" >
 * "Softmax"; shapes as in its "Inputs" section):
 *   z = fp32(x[r, :]) - max(fp32(x[r, :])),
 *   out[r, :] = cast( exp(z) / sum(exp(z)) ),
 * with fp32 maximum, exponential, sum and quotient.  A row holding a NaN or
 * +inf, or only -inf, comes out all NaN; -inf entries of any other row come
 * out 0 (the page's rules, which are what the IEEE arithmetic above gives).
 * x       [rows, hidden] input, read only (unless out == x).
 * out     [rows, hidden] output.  It may be exactly x (in place); any other
 *         overlap is KS_ERROR_OVERLAP.
 * hidden  1 <= hidden <= 2^24; rows may be 0.  There is no eps.
 * Arithmetic: exp is the device library's expf for fp32 and the hardware
 * base-2 exponential for 16-bit dtypes (with a first-order correction of the
 * argument's rounding for fp16); the row sum follows the canonical fold of
 * the RMSNorm sum of squares (vector path: the same bits for every plan);
 * the quotient is exp * (1 / sum) with the reciprocal an IEEE division, plus
 * one remainder correction for fp32.  Within 1 ulp of the exactly evaluated
 * contract for 16-bit dtypes and well within rtol = atol = 1e-6 for fp32.
 * Errors and stream rules as above.
 */
ks_status_t ks_softmax(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                       hipStream_t stream);

/* Softmax with an explicit plan (op KS_OP_SOFTMAX); plans with weight_lds
 * set are rejected, and so are split plans, which need a workspace
 * (ks_softmax_ws_ex). */
ks_status_t ks_softmax_ex(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                          const ks_plan_t *plan, hipStream_t stream);

/* Bytes of workspace ks_softmax_ws_ex needs for `plan`, or, with plan null,
 * for the plan ks_softmax_ws picks for 16-byte aligned buffers (the most any
 * alignment needs): 8 * rows * chunks for a split plan, else 0.  Returns
 * KS_ERROR_INVALID_VALUE for bad sizes or a null `bytes`. */
ks_status_t ks_softmax_workspace_size(int64_t rows, int64_t hidden, ks_dtype_t dtype, const ks_plan_t *plan,
                                      size_t *bytes);

/*
 * Softmax with a caller-owned workspace: the same contract, arguments and
 * overlap rules as ks_softmax, and the policy may also pick a split plan
 * (KS_PATH_SPLIT) for wide rows in small batches, which spreads one row over
 * many workgroups.  A split plan keeps each chunk's maximum m_c and sum s_c
 * of exp(x - m_c) in the workspace and forms the row sum as the sum of
 * s_c * exp(m_c - M), M the row maximum: the same contract, within the same
 * bounds, but the row sum is rounded in another order than on the one-pass
 * plans, so its results may differ from ks_softmax's in the last bit.
 * workspace        device memory, 4-byte aligned, of at least
 *                  ks_softmax_workspace_size bytes (it may be null when that
 *                  is 0); owned by the caller, only written by the call, and
 *                  in use until the call's work on `stream` has finished.
 *                  It must not overlap x or out (KS_ERROR_OVERLAP).
 * workspace_bytes  its size; too small (or a null workspace when the plan
 *                  needs one) is KS_ERROR_INVALID_VALUE.
 */
ks_status_t ks_softmax_ws(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ks_softmax_ws with an explicit plan (any plan ks_softmax_ex accepts, or a
 * split plan: path KS_PATH_SPLIT, threads_per_row 256, vectors_per_thread 1,
 * 2 or 4, elems_per_access 16 / element size, rows_per_block 1,
 * block_threads 256, load_nt = store_nt = 1, weight_lds 0). */
ks_status_t ks_softmax_ws_ex(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                             void *workspace, size_t workspace_bytes, const ks_plan_t *plan, hipStream_t stream);

/*
 * Softmax for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid allocation.
 * The contract, arguments, plans and overlap rules are those of
 * ks_softmax_ws; the split plan's per-chunk statistics go to a device array
 * that the library itself holds (KS_NOALLOC_SCRATCH_BYTES on each GPU the
 * library runs on, kept until the process ends), so the caller passes no
 * workspace.  The call allocates, frees and copies nothing.
 *   - A plan that needs more than KS_NOALLOC_SCRATCH_BYTES of statistics
 *     (8 bytes per chunk and row; see ks_softmax_workspace_size) is rejected
 *     with KS_ERROR_SCRATCH_LIMIT before any HIP call.
 *   - The array needs no initial contents: a split call writes every
 *     statistic it reads, and a one-pass plan does not touch the array.
 *   - All calls on one GPU share that GPU's array and leave their statistics
 *     in it.  Calls whose work overlaps in time on one GPU (for example on
 *     two streams without an ordering between them) race on the array;
 *     order them on one stream, or give one of them ks_softmax_ws.
 *   - The first call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress, no allocation); a failure there is KS_ERROR_HIP.
 */
#define KS_NOALLOC_SCRATCH_BYTES (1u << 20)
ks_status_t ks_softmax_noalloc(void *out, const void *x, int64_t rows, int64_t hidden, ks_dtype_t dtype,
                               hipStream_t stream);

/* Static description of a status code. */
const char *ks_status_string(ks_status_t status);

/* hipError_t behind the calling thread's last KS_ERROR_HIP (0 if none). */
int ks_last_hip_error(void);

/* Library version string: name, version, target and the source revision it
 * was built from, e.g. "ks_norm 0.2.0 gfx950 (source 3e7a201c0ba1)". */
const char *ks_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KS_NORM_H */
