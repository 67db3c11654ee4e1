/* Runs every oracle function over small shapes, all dtypes and bit patterns
   drawn from a fixed generator (NaN, infinities and subnormals included),
   each buffer exactly as large as the call needs, so that AddressSanitizer
   and UndefinedBehaviorSanitizer see any access outside it.  Checks only
   the status codes; values are the pins' business. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_rms_norm(int, const void *, const void *, void *, int64_t, int64_t, float);
int oracle_fused_add_rms_norm(int, void *, void *, const void *, int64_t, int64_t, float);
int oracle_rms_norm_residual(int, const void *, const void *, const void *, void *, int64_t, int64_t, float);
int oracle_rms_norm_backward(int, const void *, const void *, const void *, void *, void *, int64_t, int64_t, float);
int oracle_round_f32_array(int, const float *, uint16_t *, int64_t);
int oracle_widen_array(int, const uint16_t *, float *, int64_t);
int oracle_silu_and_mul(int, const void *, void *, int64_t, int64_t);
int oracle_softmax(int, const void *, void *, int64_t, int64_t);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 16);
}

static void *filled(size_t bytes)
{
    unsigned char *p = (unsigned char *)malloc(bytes ? bytes : 1);
    for (size_t i = 0; i < bytes; ++i)
        p[i] = (unsigned char)next_u32();
    return p;
}

#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                  \
        }                                                              \
    } while (0)

int main(void)
{
    long calls = 0;
    for (int dtype = 0; dtype < 3; ++dtype) {
        const size_t es = dtype == 0 ? 4 : 2;
        for (int64_t rows = 0; rows <= 3; ++rows)
            for (int64_t h = 1; h <= 67; h += (h < 9 ? 1 : 7)) {
                const size_t n = (size_t)(rows * h);
                void *x = filled(n * es), *r = filled(n * es), *w = filled((size_t)h * es);
                void *out = filled(n * es), *dy = filled(n * es), *dw = filled((size_t)h * es);
                EXPECT(oracle_rms_norm(dtype, x, w, out, rows, h, 1e-6f) == 0);
                EXPECT(oracle_rms_norm_residual(dtype, x, r, w, out, rows, h, 1e-6f) == 0);
                EXPECT(oracle_rms_norm_backward(dtype, dy, x, w, out, dw, rows, h, 1e-6f) == 0);
                EXPECT(oracle_softmax(dtype, x, out, rows, h) == 0);
                EXPECT(oracle_fused_add_rms_norm(dtype, x, r, w, rows, h, 1e-6f) == 0);
                free(out);
                void *half = filled((n / 2 + 1) * es);
                if (h % 2 == 0)
                    EXPECT(oracle_silu_and_mul(dtype, x, half, rows, h / 2) == 0);
                free(half);
                free(x); free(r); free(w); free(dy); free(dw);
                calls += 6;
            }
    }
    /* bad arguments: a status, never an access */
    EXPECT(oracle_rms_norm(9, NULL, NULL, NULL, 1, 8, 1e-6f) != 0);
    EXPECT(oracle_rms_norm(0, NULL, NULL, NULL, -1, 8, 1e-6f) != 0);
    EXPECT(oracle_rms_norm(0, NULL, NULL, NULL, 1, 0, 1e-6f) != 0);
    EXPECT(oracle_rms_norm(0, NULL, NULL, NULL, 1, 8, 0.0f) != 0);
    EXPECT(oracle_softmax(0, NULL, NULL, 1, 0) != 0);
    EXPECT(oracle_silu_and_mul(0, NULL, NULL, 1, 0) != 0);
    for (int dtype = 1; dtype < 3; ++dtype) {
        float *f = (float *)filled(4096 * sizeof(float));
        uint16_t *b = (uint16_t *)filled(4096 * sizeof(uint16_t));
        float *g = (float *)filled(4096 * sizeof(float));
        EXPECT(oracle_round_f32_array(dtype, f, b, 4096) == 0);
        EXPECT(oracle_widen_array(dtype, b, g, 4096) == 0);
        free(f); free(b); free(g);
    }
    printf("oracle sweep: %ld calls\n", calls);
    return 0;
}
