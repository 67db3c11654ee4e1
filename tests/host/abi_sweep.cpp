// Drives every entry point of the C ABI over a grid of valid and invalid
// arguments and plans (no GPU: the launches are stand-ins).  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer by the CPU tests; any
// memory error or undefined behaviour aborts the run.  Checks on the way:
//   * every status is one of ks_status_t;
//   * a call that succeeds with rows > 0 reaches exactly one launch (the
//     backward: one launch call), a failing or empty call reaches none;
//   * the plan ks_get_plan returns is accepted by the matching _ex call, and
//     so is the plan ks_get_plan_cus returns for any compute-unit count (and
//     it reaches one launch of a compiled shape);
//   * a timing request (ks_time_next_call) is accepted before any call;
//   * a split softmax launch carries a workspace (checked by the stand-in).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ks_norm.h"

namespace ks {
extern long g_launches;
}

static long g_checks = 0;

#define CHECK(cond)                                                            \
    do {                                                                       \
        ++g_checks;                                                            \
        if (!(cond)) {                                                         \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

static const uintptr_t kBase = 0x100000000ull;          // fake device addresses, never dereferenced
static void *at(uintptr_t off) { return (void *)(kBase + off); }
static const uintptr_t kGiB = 1ull << 30;

static void expect_status(ks_status_t st, long before, int64_t rows)
{
    CHECK(st >= KS_SUCCESS && st <= KS_ERROR_SCRATCH_LIMIT);
    const long launched = ks::g_launches - before;
    if (st == KS_SUCCESS && rows > 0)
        CHECK(launched == 1);
    else if (st != KS_SUCCESS)
        CHECK(launched == 0);
}

int main()
{
    const int dtypes[] = {KS_DTYPE_FLOAT32, KS_DTYPE_FLOAT16, KS_DTYPE_BFLOAT16, 7, -1};
    const int64_t rows_set[] = {-1, 0, 1, 3, 4096, INT32_MAX, (int64_t)INT32_MAX + 1};
    const int64_t hidden_set[] = {-5, 0, 1, 5, 8, 1000, 1001, 4096, 32768, 32776, 65536, 65544, 1 << 24,
                                  (1 << 24) + 1};
    const float eps_set[] = {1e-6f, 0.0f, -1.0f, NAN, INFINITY};
    // buffer layouts: (out, x, residual, weight) offsets; some aligned, some not, some overlapping
    const uintptr_t layouts[][4] = {
        {0, 4 * kGiB, 8 * kGiB, 12 * kGiB}, {2, 4 * kGiB + 2, 8 * kGiB + 2, 12 * kGiB + 2},
        {0, 0, 8 * kGiB, 12 * kGiB},        {16, 0, 8 * kGiB, 12 * kGiB},
        {0, 4 * kGiB, 4 * kGiB, 12 * kGiB}, {0, 4 * kGiB, 8 * kGiB, 8 * kGiB + 64},
    };
    for (int dt : dtypes)
        for (int64_t rows : rows_set)
            for (int64_t hidden : hidden_set)
                for (float eps : eps_set)
                    for (const auto &L : layouts) {
                        void *o = at(L[0]), *x = at(L[1]), *r = at(L[2]), *w = at(L[3]);
                        const ks_dtype_t d = (ks_dtype_t)dt;
                        long before = ks::g_launches;
                        expect_status(ks_rms_norm(o, x, w, rows, hidden, eps, d, 0), before, rows);
                        before = ks::g_launches;
                        expect_status(ks_fused_add_rms_norm(x, r, w, rows, hidden, eps, d, 0), before, rows);
                        before = ks::g_launches;
                        expect_status(ks_rms_norm_residual(o, x, r, w, rows, hidden, eps, d, 0), before, rows);
                        before = ks::g_launches;
                        expect_status(ks_softmax(o, x, rows, hidden, d, 0), before, rows);
                        before = ks::g_launches;
                        expect_status(ks_silu_and_mul(o, x, rows, hidden, d, 0), before, rows);
                        size_t need = 0;
                        if (ks_softmax_workspace_size(rows, hidden, d, nullptr, &need) == KS_SUCCESS) {
                            before = ks::g_launches;
                            expect_status(ks_softmax_ws(o, x, rows, hidden, d, at(24 * kGiB), need, 0), before, rows);
                            before = ks::g_launches;
                            expect_status(ks_softmax_ws(o, x, rows, hidden, d, need ? nullptr : at(24 * kGiB), need, 0),
                                          before, rows);
                        }
                        if (ks_rms_norm_backward_workspace_size(rows, hidden, &need) == KS_SUCCESS) {
                            before = ks::g_launches;
                            // dx, dw, dy, x, weight, workspace: disjoint except where the layout overlaps
                            ks_status_t st = ks_rms_norm_backward(o, at(16 * kGiB), r, x, w, rows, hidden, eps, d,
                                                                  at(20 * kGiB), need, 0);
                            CHECK(st >= KS_SUCCESS && st <= KS_ERROR_HIP);
                            if (st != KS_SUCCESS)
                                CHECK(ks::g_launches == before);
                        }
                    }

    // every policy plan is accepted by its own _ex entry point (rows = 0: no launch)
    const int ops[] = {KS_OP_RMS_NORM, KS_OP_FUSED_ADD_RMS_NORM, KS_OP_SILU_AND_MUL, KS_OP_SOFTMAX,
                       KS_OP_RMS_NORM_RESIDUAL, KS_OP_RMS_NORM_BACKWARD};
    for (int op : ops)
        for (int dt = 0; dt < 3; ++dt)
            for (int64_t hidden = 1; hidden <= 70000; hidden = hidden < 64 ? hidden + 1 : hidden * 5 / 4 + 3)
                for (int64_t rows : {1ll, 7ll, 512ll, 8192ll, 1ll << 20})
                    for (int flags = 0; flags < 4; ++flags) {
                        const int aligned = flags & KS_PLAN_ALIGNED;
                        ks_plan_t p;
                        CHECK(ks_get_plan((ks_op_t)op, (ks_dtype_t)dt, rows, hidden, flags, &p) == KS_SUCCESS);
                        const uintptr_t a = aligned ? 0 : 2;
                        void *o = at(a), *x = at(4 * kGiB + a), *r = at(8 * kGiB + a), *w = at(12 * kGiB + a);
                        ks_status_t st = KS_ERROR_HIP;
                        switch (op) {
                        case KS_OP_RMS_NORM: st = ks_rms_norm_ex(o, x, w, 0, hidden, 1e-6f, (ks_dtype_t)dt, &p, 0); break;
                        case KS_OP_FUSED_ADD_RMS_NORM:
                            st = ks_fused_add_rms_norm_ex(x, r, w, 0, hidden, 1e-6f, (ks_dtype_t)dt, &p, 0);
                            break;
                        case KS_OP_SILU_AND_MUL: st = ks_silu_and_mul_ex(o, x, 0, hidden, (ks_dtype_t)dt, &p, 0); break;
                        case KS_OP_SOFTMAX:
                            st = (flags & KS_PLAN_WORKSPACE)
                                     ? ks_softmax_ws_ex(o, x, 0, hidden, (ks_dtype_t)dt, nullptr, 0, &p, 0)
                                     : ks_softmax_ex(o, x, 0, hidden, (ks_dtype_t)dt, &p, 0);
                            break;
                        case KS_OP_RMS_NORM_RESIDUAL:
                            st = ks_rms_norm_residual_ex(o, x, r, w, 0, hidden, 1e-6f, (ks_dtype_t)dt, &p, 0);
                            break;
                        default:
                            st = ks_rms_norm_backward_ex(o, nullptr, r, x, w, 0, hidden, 1e-6f, (ks_dtype_t)dt, nullptr,
                                                         0, &p, 0);
                            break;
                        }
                        CHECK(st == KS_SUCCESS);
                    }

    // explicit plans over a grid of field values: any status, never a crash; a
    // plan accepted for rows = 4 reaches exactly one launch
    const int paths[] = {0, 1, 2, -1};
    const int tprs[] = {0, 1, 7, 8, 16, 64, 256, 512, 1024, 2048};
    const int vpts[] = {-1, 0, 1, 3, 4, 5, 8, 9};
    const int epas[] = {0, 1, 2, 4, 8, 16};
    const int blocks[] = {0, 64, 256, 512, 1024};
    const int hints[] = {0, 1, 2, 3};
    for (int path : paths)
        for (int tpr : tprs)
            for (int vpt : vpts)
                for (int epa : epas)
                    for (int block : blocks)
                        for (int h : hints)
                          for (int rpt : {1, 2, 3, 4}) {
                            ks_plan_t p{path, tpr, vpt, epa, tpr > 0 ? block / tpr * rpt : 0, block, h & 1, h >> 1,
                                        h == 2};
                            for (int64_t hidden : {5ll, 1000ll, 4096ll, 40000ll}) {
                                long before = ks::g_launches;
                                expect_status(ks_rms_norm_ex(at(0), at(4 * kGiB), at(12 * kGiB), 4, hidden, 1e-6f,
                                                             KS_DTYPE_BFLOAT16, &p, 0), before, 4);
                                before = ks::g_launches;
                                expect_status(ks_fused_add_rms_norm_ex(at(4 * kGiB), at(8 * kGiB), at(12 * kGiB), 4,
                                                                       hidden, 1e-6f, KS_DTYPE_FLOAT16, &p, 0),
                                              before, 4);
                                before = ks::g_launches;
                                expect_status(ks_rms_norm_residual_ex(at(0), at(4 * kGiB), at(8 * kGiB), at(12 * kGiB),
                                                                      4, hidden, 1e-6f, KS_DTYPE_FLOAT32, &p, 0),
                                              before, 4);
                                before = ks::g_launches;
                                expect_status(ks_softmax_ex(at(0), at(4 * kGiB), 4, hidden, KS_DTYPE_FLOAT32, &p, 0),
                                              before, 4);
                                before = ks::g_launches;
                                expect_status(ks_silu_and_mul_ex(at(0), at(4 * kGiB), 4, hidden, KS_DTYPE_FLOAT16, &p,
                                                                 0), before, 4);
                                size_t need = 0;
                                CHECK(ks_softmax_workspace_size(4, hidden, KS_DTYPE_FLOAT16, &p, &need) == KS_SUCCESS);
                                before = ks::g_launches;
                                expect_status(ks_softmax_ws_ex(at(0), at(4 * kGiB), 4, hidden, KS_DTYPE_FLOAT16,
                                                               at(8 * kGiB), need, &p, 0), before, 4);
                            }
                        }
    // the policy on devices of other compute-unit counts: every plan is a
    // compiled shape its own _ex call accepts, and it launches once
    for (int cus : {1, 2, 7, 32, 38, 80, 128, 256, 304, 1024, 4096})
        for (int op : ops)
            for (int dt = 0; dt < 3; ++dt)
                for (int64_t hidden : {1ll, 8ll, 100ll, 1024ll, 1536ll, 4096ll, 8192ll, 16384ll, 32768ll, 65536ll})
                    for (int64_t rows : {1ll, 4ll, 512ll, 2048ll, 32768ll})
                        for (int flags = 0; flags < 4; ++flags) {
                            ks_plan_t p;
                            CHECK(ks_get_plan_cus((ks_op_t)op, (ks_dtype_t)dt, rows, hidden, flags, cus, &p) ==
                                  KS_SUCCESS);
                            // buffers 64 GiB apart: the largest case here (32768 rows of 65536 fp32) is 8 GiB
                            const uintptr_t a = (flags & KS_PLAN_ALIGNED) ? 0 : 2;
                            void *o = at(a), *x = at(64 * kGiB + a), *r = at(128 * kGiB + a), *w = at(192 * kGiB + a);
                            const ks_dtype_t d = (ks_dtype_t)dt;
                            const long before = ks::g_launches;
                            ks_status_t st = KS_ERROR_HIP;
                            size_t need = 0;
                            switch (op) {
                            case KS_OP_RMS_NORM: st = ks_rms_norm_ex(o, x, w, rows, hidden, 1e-6f, d, &p, 0); break;
                            case KS_OP_FUSED_ADD_RMS_NORM:
                                st = ks_fused_add_rms_norm_ex(x, r, w, rows, hidden, 1e-6f, d, &p, 0);
                                break;
                            case KS_OP_SILU_AND_MUL: st = ks_silu_and_mul_ex(o, x, rows, hidden, d, &p, 0); break;
                            case KS_OP_SOFTMAX:
                                CHECK(ks_softmax_workspace_size(rows, hidden, d, &p, &need) == KS_SUCCESS);
                                st = (flags & KS_PLAN_WORKSPACE)
                                         ? ks_softmax_ws_ex(o, x, rows, hidden, d, at(256 * kGiB), need, &p, 0)
                                         : ks_softmax_ex(o, x, rows, hidden, d, &p, 0);
                                break;
                            case KS_OP_RMS_NORM_RESIDUAL:
                                st = ks_rms_norm_residual_ex(o, x, r, w, rows, hidden, 1e-6f, d, &p, 0);
                                break;
                            default:
                                st = ks_rms_norm_backward_ex(o, nullptr, r, x, w, rows, hidden, 1e-6f, d, nullptr, 0,
                                                             &p, 0);
                                break;
                            }
                            CHECK(st == KS_SUCCESS);
                            CHECK(ks::g_launches - before == 1);
                        }
    for (int cus : {-1, 0, 4097}) {
        ks_plan_t p;
        CHECK(ks_get_plan_cus(KS_OP_RMS_NORM, KS_DTYPE_BFLOAT16, 4, 4096, 1, cus, &p) == KS_ERROR_INVALID_VALUE);
    }
    // a timing request is accepted and spent by the next call, launched or rejected
    CHECK(ks_time_next_call(nullptr, nullptr) == KS_SUCCESS);
    CHECK(ks_rms_norm(at(0), at(4 * kGiB), at(12 * kGiB), 4, 0, 1e-6f, KS_DTYPE_BFLOAT16, 0) == KS_ERROR_INVALID_VALUE);
    {
        const long before = ks::g_launches;
        CHECK(ks_rms_norm(at(0), at(4 * kGiB), at(12 * kGiB), 4, 4096, 1e-6f, KS_DTYPE_BFLOAT16, 0) == KS_SUCCESS);
        CHECK(ks::g_launches - before == 1);
    }
    for (int op = -2; op < 8; ++op) {
        ks_plan_t p;
        const ks_status_t st = ks_get_plan((ks_op_t)op, KS_DTYPE_BFLOAT16, 4, 4096, 1, &p);
        CHECK((op >= 0 && op <= 5) ? st == KS_SUCCESS : st == KS_ERROR_INVALID_VALUE);
    }
    CHECK(ks_get_plan(KS_OP_RMS_NORM, KS_DTYPE_BFLOAT16, 4, 4096, 1, nullptr) == KS_ERROR_INVALID_VALUE);
    for (int flags = -1; flags < 9; ++flags) {
        ks_plan_t p;
        const ks_status_t st = ks_get_plan(KS_OP_SOFTMAX, KS_DTYPE_BFLOAT16, 4, 65536, flags, &p);
        CHECK((flags >= 0 && flags < 4) ? st == KS_SUCCESS : st == KS_ERROR_INVALID_VALUE);
    }
    for (int s = -1; s < 7; ++s)
        CHECK(ks_status_string((ks_status_t)s) != nullptr);
    printf("abi sweep: %ld checks, %ld launches\n", g_checks, ks::g_launches);
    return 0;
}
