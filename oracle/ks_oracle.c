/*
 * CPU oracle for RMSNorm row normalisation (forward and backward), the
 * fused residual-add variant (in place, and out of place), the SwiGLU
 * activation and softmax over the last dimension.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library; the GPU library never
 * does, and the two share no code, headers or constants.
 *
 * What it follows (kernscope README, "Numerical contract"):
 *   - "RMSNorm": widen x to fp32, take rsqrt of (mean of the squares over the
 *     last axis plus eps), multiply by the widened weight, cast back to the
 *     input dtype; reduction and scaling carry fp32 intermediates.
 *   - "Fused residual-add RMSNorm": s = fp32(x_in) + fp32(residual_in);
 *     residual <- cast(s); x <- cast(RMSNorm of the unrounded fp32 s times the
 *     widened weight).  Outputs depend only on the input snapshots.
 *   - "Inputs": dtypes fp16 / bf16 / fp32, x of shape (..., H) flattened to
 *     (rows, H) contiguous, weight of shape (H,).
 *
 * Readings where the page is silent (each is listed with its reason in the
 * design notes):
 *   - The fp32 "mean of squares" is taken as the fp32 value nearest the exact
 *     mean: squares of widened values are exact in double, they are summed
 *     in index order in double and the sum is rounded once to fp32; the mean
 *     is one IEEE fp32 division by H.
 *   - eps is rounded to fp32 and added in fp32.
 *   - rsqrt is evaluated in double precision (IEEE sqrt, then IEEE divide)
 *     and rounded once to fp32: the correctly rounded fp32 value except when
 *     the exact result lies within about 2^-52 (relative) of an fp32
 *     rounding boundary.
 *   - The multiplications run left to right as written: (x * scale) * w.
 *   - "cast_to_input_dtype" is IEEE round-to-nearest, ties-to-even, with
 *     subnormals kept, overflow to infinity and NaN kept as a quiet NaN.
 *
 * Build: plain C11, single thread, -O2 -ffp-contract=off -fno-fast-math, so
 * every float operation below is one IEEE binary32/binary64 operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes of this file (the Python wrapper maps names onto them) */
enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* status codes of this file */
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_NO_MEMORY = 2 };

/* ------------------------------------------------------------------------ */
/* Binary formats, from their IEEE 754 / bfloat16 definitions.              */
/*   binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.              */
/*   bfloat16: the upper 16 bits of binary32: 1 sign, 8 exponent (bias      */
/*             127), 7 fraction bits.                                       */
/* ------------------------------------------------------------------------ */

typedef struct {
    int prec;          /* significand bits, the implicit leading bit included */
    int emin;          /* exponent of the smallest normal number */
    int exp_bits;      /* width of the exponent field */
    double max_finite; /* largest finite value */
} format_t;

static const format_t FMT_F16 = {11, -14, 5, 65504.0};
static const format_t FMT_BF16 = {8, -126, 8, 0x1.fep127};

/* Round a (a double, so exactly known) to the nearest value of format f,
   ties to even.  Returns +-inf when the rounded magnitude exceeds the largest
   finite value. */
static double round_to_format(double a, const format_t *f)
{
    if (isnan(a) || isinf(a) || a == 0.0)
        return a;
    int e;
    frexp(fabs(a), &e);          /* |a| = m * 2^e with m in [0.5, 1) */
    int lead = e - 1;            /* weight of the leading bit is 2^lead */
    if (lead < f->emin)
        lead = f->emin;          /* subnormal range: fixed quantum */
    int qexp = lead - (f->prec - 1); /* weight of the last significand bit */
    double n = ldexp(a, -qexp);  /* exact: power-of-two scaling */
    double r = nearbyint(n);     /* default mode: nearest, ties to even */
    double v = ldexp(r, qexp);
    if (fabs(v) > f->max_finite)
        return copysign(INFINITY, a);
    return v;
}

/* Bit pattern of v, which must already be a value of format f (or inf/NaN). */
static uint16_t encode_format(double v, const format_t *f)
{
    int bias = 1 - f->emin;
    int frac_bits = f->prec - 1;
    uint32_t exp_all_ones = (1u << f->exp_bits) - 1u;
    uint32_t sign = signbit(v) ? 1u : 0u;
    uint32_t sign_bit = sign << (f->exp_bits + frac_bits);
    if (isnan(v))  /* quiet NaN: exponent all ones, top fraction bit set */
        return (uint16_t)(sign_bit | (exp_all_ones << frac_bits) | (1u << (frac_bits - 1)));
    if (isinf(v))
        return (uint16_t)(sign_bit | (exp_all_ones << frac_bits));
    if (v == 0.0)
        return (uint16_t)sign_bit;
    double a = fabs(v);
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < f->emin) { /* subnormal: exponent field 0, fraction = a / 2^(emin - frac_bits) */
        uint32_t frac = (uint32_t)ldexp(a, -(f->emin - frac_bits));
        return (uint16_t)(sign_bit | frac);
    }
    uint32_t biased = (uint32_t)(lead + bias);
    uint32_t frac = (uint32_t)(ldexp(a, -(lead - frac_bits)) - ldexp(1.0, frac_bits));
    return (uint16_t)(sign_bit | (biased << frac_bits) | frac);
}

/* Value of a 16-bit pattern of format f. */
static double decode_format(uint16_t bits, const format_t *f)
{
    int frac_bits = f->prec - 1;
    int bias = 1 - f->emin;
    uint32_t exp_all_ones = (1u << f->exp_bits) - 1u;
    uint32_t sign = (bits >> (f->exp_bits + frac_bits)) & 1u;
    uint32_t ex = (bits >> frac_bits) & exp_all_ones;
    uint32_t frac = bits & ((1u << frac_bits) - 1u);
    double mag;
    if (ex == exp_all_ones)
        mag = frac ? NAN : INFINITY;
    else if (ex == 0)
        mag = ldexp((double)frac, f->emin - frac_bits);
    else
        mag = ldexp((double)((1u << frac_bits) | frac), (int)ex - bias - frac_bits);
    return sign ? -mag : mag;
}

static const format_t *format_of(int dtype)
{
    return dtype == ORACLE_F16 ? &FMT_F16 : &FMT_BF16;
}

/* widen element i of an array of the given dtype to fp32 (exact) */
static float load_elem(int dtype, const void *p, int64_t i)
{
    if (dtype == ORACLE_F32)
        return ((const float *)p)[i];
    return (float)decode_format(((const uint16_t *)p)[i], format_of(dtype));
}

/* round v to the dtype (ties to even) and store it as element i */
static void store_elem(int dtype, void *p, int64_t i, float v)
{
    if (dtype == ORACLE_F32) {
        ((float *)p)[i] = v;
        return;
    }
    const format_t *f = format_of(dtype);
    ((uint16_t *)p)[i] = encode_format(round_to_format((double)v, f), f);
}

static int check_args(int dtype, int64_t rows, int64_t hidden, float eps)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_BAD_ARG;
    if (rows < 0 || hidden <= 0 || !(eps > 0.0f) || isinf(eps))
        return ORACLE_BAD_ARG;
    return ORACLE_OK;
}

/* fp32 factor rsqrt(mean(v^2) + eps) of one row, from the exact sum of
   squares held in double (see the readings in the header comment). */
static float row_scale(double sum_sq, int64_t hidden, float eps)
{
    float ss = (float)sum_sq;           /* one rounding to fp32 */
    float mean = ss / (float)hidden;    /* IEEE fp32 division */
    float d = mean + eps;               /* fp32 add */
    return (float)(1.0 / sqrt((double)d));
}

/* ------------------------------------------------------------------------ */
/* Public functions.                                                         */
/* ------------------------------------------------------------------------ */

/* out[r, :] = cast(fp32(x[r, :]) * scale_r * fp32(w)); out may equal x. */
int oracle_rms_norm(int dtype, const void *x, const void *w, void *out,
                    int64_t rows, int64_t hidden, float eps)
{
    int st = check_args(dtype, rows, hidden, eps);
    if (st != ORACLE_OK)
        return st;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t base = r * hidden;
        double sum_sq = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            double v = (double)load_elem(dtype, x, base + j);
            sum_sq += v * v;  /* each square is exact in double */
        }
        float scale = row_scale(sum_sq, hidden, eps);
        for (int64_t j = 0; j < hidden; ++j) {
            float v = load_elem(dtype, x, base + j);
            float t = v * scale;
            float u = t * load_elem(dtype, w, j);
            store_elem(dtype, out, base + j, u);
        }
    }
    return ORACLE_OK;
}

/* In place: s = fp32(x) + fp32(residual); residual <- cast(s);
   x <- cast(fp32(s) * scale(s) * fp32(w)).  Every element of a row is read
   before any element of that row is written. */
int oracle_fused_add_rms_norm(int dtype, void *x, void *residual, const void *w,
                              int64_t rows, int64_t hidden, float eps)
{
    int st = check_args(dtype, rows, hidden, eps);
    if (st != ORACLE_OK)
        return st;
    float *s = (float *)malloc((size_t)hidden * sizeof(float));
    if (!s)
        return ORACLE_NO_MEMORY;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t base = r * hidden;
        double sum_sq = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            s[j] = load_elem(dtype, x, base + j) + load_elem(dtype, residual, base + j);
            double v = (double)s[j];
            sum_sq += v * v;
        }
        float scale = row_scale(sum_sq, hidden, eps);
        for (int64_t j = 0; j < hidden; ++j) {
            store_elem(dtype, residual, base + j, s[j]);
            float t = s[j] * scale;
            float u = t * load_elem(dtype, w, j);
            store_elem(dtype, x, base + j, u);
        }
    }
    free(s);
    return ORACLE_OK;
}

/* Out of place (Triton Kernels README, "Kernels": the residual-fused
   RMSNorm, RMSNorm(x + residual) * w, with FP32 accumulation as in its
   RMSNorm row): out <- cast(s * scale(s) * fp32(w)) with s = fp32(x) +
   fp32(residual); x and residual are only read.  Reading where the page is
   silent: s is the unrounded fp32 sum, as in the kernscope fused contract,
   and the normalisation is the kernscope one.  out may equal x or residual:
   a row's inputs are all read before its first output is written. */
int oracle_rms_norm_residual(int dtype, const void *x, const void *residual, const void *w,
                             void *out, int64_t rows, int64_t hidden, float eps)
{
    int st = check_args(dtype, rows, hidden, eps);
    if (st != ORACLE_OK)
        return st;
    float *s = (float *)malloc((size_t)hidden * sizeof(float));
    if (!s)
        return ORACLE_NO_MEMORY;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t base = r * hidden;
        double sum_sq = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            s[j] = load_elem(dtype, x, base + j) + load_elem(dtype, residual, base + j);
            sum_sq += (double)s[j] * (double)s[j];
        }
        float scale = row_scale(sum_sq, hidden, eps);
        for (int64_t j = 0; j < hidden; ++j) {
            float scaled = s[j] * scale;
            store_elem(dtype, out, base + j, scaled * load_elem(dtype, w, j));
        }
    }
    free(s);
    return ORACLE_OK;
}

/* round a double v once to the dtype (ties to even) and store it as element i */
static void store_elem_exact(int dtype, void *p, int64_t i, double v)
{
    if (dtype == ORACLE_F32) {
        ((float *)p)[i] = (float)v;
        return;
    }
    const format_t *f = format_of(dtype);
    ((uint16_t *)p)[i] = encode_format(round_to_format(v, f), f);
}

/* RMSNorm backward.  No page states a backward contract; the kernscope
   README says the PyTorch reference of rms_norm supports autograd, so the
   gradients are those of the forward contract
       y_j = x_j * rho * w_j,   rho = (sum_k x_k^2 / H + eps)^(-1/2),
   for an incoming gradient dy (the final cast passes gradients through):
       dx_j = rho * dy_j * w_j - (rho^3 / H) * x_j * sum_k dy_k * w_k * x_k
       dw_j = sum over rows of dy_j * x_j * rho.
   Readings: the gradients are evaluated exactly (in double, from the widened
   inputs and eps rounded to fp32) and rounded once to the dtype; dw may be
   NULL (not wanted); for rows == 0, dw is zero. */
int oracle_rms_norm_backward(int dtype, const void *dy, const void *x, const void *w, void *dx, void *dw,
                             int64_t rows, int64_t hidden, float eps)
{
    int st = check_args(dtype, rows, hidden, eps);
    if (st != ORACLE_OK)
        return st;
    double *dw_sum = (double *)calloc((size_t)hidden, sizeof(double));
    if (!dw_sum)
        return ORACLE_NO_MEMORY;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t base = r * hidden;
        double sum_sq = 0.0, dot = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            double xv = (double)load_elem(dtype, x, base + j);
            double gv = (double)load_elem(dtype, dy, base + j) * (double)load_elem(dtype, w, j);
            sum_sq += xv * xv;
            dot += gv * xv;
        }
        double rho = 1.0 / sqrt(sum_sq / (double)hidden + (double)eps);
        double coef = rho * rho * rho * dot / (double)hidden;
        for (int64_t j = 0; j < hidden; ++j) {
            double xv = (double)load_elem(dtype, x, base + j);
            double dyv = (double)load_elem(dtype, dy, base + j);
            double grad = rho * dyv * (double)load_elem(dtype, w, j) - coef * xv;
            store_elem_exact(dtype, dx, base + j, grad);
            dw_sum[j] += dyv * xv * rho;
        }
    }
    if (dw != NULL)
        for (int64_t j = 0; j < hidden; ++j)
            store_elem_exact(dtype, dw, j, dw_sum[j]);
    free(dw_sum);
    return ORACLE_OK;
}

/* Round n fp32 values to a 16-bit dtype (ties to even); used by cast tests. */
int oracle_round_f32_array(int dtype, const float *in, uint16_t *out, int64_t n)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_BAD_ARG;
    const format_t *f = format_of(dtype);
    for (int64_t i = 0; i < n; ++i)
        out[i] = encode_format(round_to_format((double)in[i], f), f);
    return ORACLE_OK;
}

/* Widen n 16-bit values to fp32; used by cast tests. */
int oracle_widen_array(int dtype, const uint16_t *in, float *out, int64_t n)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_BAD_ARG;
    const format_t *f = format_of(dtype);
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)decode_format(in[i], f);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* SwiGLU activation (kernscope README, "Numerical contract" > "SwiGLU        */
/* activation"; shapes from its "Inputs" section): x holds rows of 2D        */
/* values, gate = the first D, up = the last D;                              */
/*   out[r, j] = cast(fp32(gate) * sigmoid(fp32(gate)) * fp32(up))           */
/* with fp32 intermediates, multiplied left to right.                        */
/* Reading where the page is silent: sigmoid(g) is the fp32 value nearest   */
/* 1 / (1 + e^-g), evaluated in double with the C library's exp and rounded  */
/* once to fp32.                                                             */
/* ------------------------------------------------------------------------ */
static float sigmoid32(float g)
{
    return (float)(1.0 / (1.0 + exp(-(double)g)));
}

int oracle_silu_and_mul(int dtype, const void *x, void *out, int64_t rows, int64_t d)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_BAD_ARG;
    if (rows < 0 || d <= 0)
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < d; ++j) {
            float g = load_elem(dtype, x, r * 2 * d + j);
            float u = load_elem(dtype, x, r * 2 * d + d + j);
            float t = g * sigmoid32(g);
            store_elem(dtype, out, r * d + j, t * u);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Softmax over the last dimension (kernscope README, "Numerical contract" > */
/* "Softmax"; shapes from its "Inputs" section):                             */
/*   z   = fp32(x) - max(fp32(x)) over the row,                              */
/*   out = cast(exp(z) / sum(exp(z)) over the row)                           */
/* with the maximum, exponential, sum and division in fp32.  The page's      */
/* rules for non-finite rows (NaN or +inf anywhere, or a row of only -inf:   */
/* NaN everywhere; -inf entries of other rows: 0) are what IEEE arithmetic   */
/* gives once the maximum propagates NaN, so no case is special-cased here.  */
/* Readings where the page is silent:                                        */
/*   - the maximum of a row holding a NaN is NaN (as PyTorch's max is);      */
/*   - z is one IEEE fp32 subtraction of the widened element and the max;    */
/*   - the fp32 quotient is the fp32 value nearest exp(z) / sum(exp(z)) for  */
/*     those fp32 z: the exponentials are evaluated in double by the C       */
/*     library, summed in index order and divided in double, and the         */
/*     quotient is rounded once to fp32, then cast to the input dtype.       */
/* ------------------------------------------------------------------------ */
int oracle_softmax(int dtype, const void *x, void *out, int64_t rows, int64_t hidden)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_BAD_ARG;
    if (rows < 0 || hidden <= 0)
        return ORACLE_BAD_ARG;
    double *e = (double *)malloc((size_t)hidden * sizeof(double));
    if (e == NULL)
        return ORACLE_NO_MEMORY;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t base = r * hidden;
        float m = -INFINITY;
        int has_nan = 0;
        for (int64_t j = 0; j < hidden; ++j) {
            float v = load_elem(dtype, x, base + j);
            if (isnan(v))
                has_nan = 1;
            else if (v > m)
                m = v;
        }
        if (has_nan)
            m = NAN;
        double sum = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            float z = load_elem(dtype, x, base + j) - m;   /* fp32 subtraction */
            e[j] = exp((double)z);
            sum += e[j];
        }
        /* every element was read above, so out may alias x */
        for (int64_t j = 0; j < hidden; ++j)
            store_elem(dtype, out, base + j, (float)(e[j] / sum));
    }
    free(e);
    return ORACLE_OK;
}
