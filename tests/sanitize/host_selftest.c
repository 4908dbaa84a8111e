/*
 * Host-side self-test of the GEMV library (test infrastructure), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host code only by
 * tests/sanitize/build.py and run by tests/test_sanitize_cpu.py: it needs no
 * GPU.  It drives the planner (gemv_describe_launch_for) over seeded row
 * counts and lengths on several device descriptions, the status strings, and
 * every entry point's argument checks that return before touching a device,
 * so that an out-of-bounds access, an overflow or an undefined shift in the
 * host code stops the run.  Exits 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gemv.h"
#include "gemv_quant.h"
#include "gemv_softmax.h"

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t state = 2026;
static uint64_t next(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return state >> 17;
}

int main(void)
{
    static const int devices[][2] = {{256, 160 * 1024}, {304, 64 * 1024}, {80, 64 * 1024}, {1, 1024}};
    static const int elems[6] = {4, 8, 16, 32, 8, 8};
    long plans = 0;
    for (int d = 0; d < 4; ++d) {
        for (int it = 0; it < 20000; ++it) {
            const int kind = (int)(next() % 6);
            const int M = (int)(next() % ((it % 3) == 0 ? (1u << 30) : 70000u)) + (it % 5 == 0 ? 0 : 1);
            int N = (int)(next() % ((it % 4) == 0 ? (1u << 30) : 140000u));
            if (kind == 3)
                N -= N % 128;
            const int aligned = (int)(next() % 2);
            gemv_launch_info info;
            memset(&info, 0xAB, sizeof info);
            const int rc = gemv_describe_launch_for(kind, M, N, aligned, devices[d][0], devices[d][1], &info);
            CHECK(rc == GEMV_OK);
            if (rc != GEMV_OK)
                continue;
            ++plans;
            /* M == 0 launches nothing: grid 0 */
            if (!(info.grid >= (M > 0) && info.block >= 64 && info.block <= 1024 && info.block % 64 == 0))
                fprintf(stderr, "kind %d M %d N %d aligned %d device %d/%d: variant %d grid %d block %d\n", kind, M, N,
                        aligned, devices[d][0], devices[d][1], info.variant, info.grid, info.block);
            CHECK(info.variant >= 1 && info.variant <= 7);
            CHECK(info.grid >= (M > 0) && info.block >= 64 && info.block <= 1024 && info.block % 64 == 0);
            CHECK((int64_t)info.grid * info.block <= ((int64_t)1 << 30));
            CHECK(info.units_in_flight >= 1 && info.units_in_flight <= 8);
            CHECK(info.lds_bytes >= 0 && info.lds_bytes <= devices[d][1]);
            if (N == 0 || N % elems[kind] != 0 || !aligned)
                CHECK(info.variant == 3);
        }
    }
    CHECK(plans > 70000);
    /* explicit plans (gemv_check_plan_for): random plans, shapes and devices
     * give a status and, when accepted, a launch within the limits */
    long accepted = 0;
    for (int it = 0; it < 200000; ++it) {
        const int d = (int)(next() % 4);
        const int kind = (int)(next() % 7) - (it % 50 == 0);   /* -1 and 6: invalid kinds */
        const int M = (int)(next() % ((it % 3) == 0 ? (1u << 30) : 70000u));
        int N = (int)(next() % ((it % 4) == 0 ? (1u << 30) : 140000u));
        if (kind == 3 && it % 2)
            N -= N % 128;
        if (kind >= 0 && kind < 6 && it % 3)
            N -= N % elems[kind];
        /* fields drawn mostly from the accepted values, sometimes not */
        static const int variants[] = {1, 2, 4, 5, 6, 2, 1, 0, 3, 7};
        static const int waves[] = {4, 8, 2, 16, 4, 8, 12, 3, 0};
        static const int depths[] = {4, 2, 8, 1, 3, 5, 4, 0, 6};
        static const int rows[] = {1, 2, 4, 8, 0, -1};
        static const int orders[] = {-1, 2, 1, 0, -1, 3, -2};
        static const int caps[] = {0, 2, 3, 4, 0, 1, 6, -1};
        const gemv_plan p = {variants[next() % 10], waves[next() % 9], depths[next() % 9], rows[next() % 6],
                             orders[next() % 7], caps[next() % 8]};
        gemv_launch_info info;
        memset(&info, 0xAB, sizeof info);
        const int rc = gemv_check_plan_for(kind, M, N, devices[d][0], devices[d][1], &p, &info);
        CHECK(rc == GEMV_OK || rc == GEMV_E_UNSUPPORTED || rc == GEMV_E_INVAL);
        if (rc != GEMV_OK)
            continue;
        ++accepted;
        CHECK(info.variant == p.variant && info.units_in_flight == p.units_in_flight);
        CHECK(info.grid >= 1 && (int64_t)info.grid * info.block <= ((int64_t)1 << 30));
        CHECK(info.lds_bytes >= 0 && info.lds_bytes <= devices[d][1]);
    }
    CHECK(accepted > 100);
    {
        const gemv_plan ok = {2, 4, 4, 1, -1, 0};
        gemv_launch_info info;
        CHECK(gemv_check_plan_for(1, 4096, 4096, 256, 163840, NULL, &info) == GEMV_E_INVAL);
        CHECK(gemv_check_plan_for(1, 4096, 4096, 256, 163840, &ok, NULL) == GEMV_E_INVAL);
        CHECK(gemv_check_plan_for(1, 4096, 4096, 256, 163840, &ok, &info) == GEMV_OK);
        CHECK(gemv_launch_plan(1, NULL, NULL, NULL, NULL, 4096, 4096, &ok, 0) == GEMV_E_INVAL);
    }
    /* argument checks that return before any device call */
    gemv_launch_info info;
    CHECK(gemv_describe_launch_for(0, -1, 4, 1, 256, 163840, &info) == GEMV_E_INVAL);
    CHECK(gemv_describe_launch_for(3, 4, 100, 1, 256, 163840, &info) == GEMV_E_UNSUPPORTED);
    CHECK(gemv_describe_launch_for(9, 4, 4, 1, 256, 163840, &info) == GEMV_E_INVAL);
    CHECK(gemv_describe_launch_for(0, 4, 4, 1, 0, 163840, &info) == GEMV_E_INVAL);
    CHECK(gemv_describe_launch_for(0, 4, 4, 1, 256, 163840, NULL) == GEMV_E_INVAL);
    CHECK(gemv_f32(NULL, NULL, NULL, -1, 4, 0) == GEMV_E_INVAL);
    CHECK(gemv_f16(NULL, NULL, NULL, 4, -1, 0) == GEMV_E_INVAL);
    CHECK(gemv_f16(NULL, NULL, NULL, 0, 4, 0) == GEMV_OK);
    CHECK(gemv_f16x32(NULL, NULL, NULL, 4, 4, 0) == GEMV_E_INVAL);
    CHECK(gemv_f16_acc16(NULL, NULL, NULL, 4, 4, 0) == GEMV_E_INVAL);
    CHECK(gemv_q8(NULL, NULL, NULL, NULL, 4, 4, 0) == GEMV_E_INVAL);
    CHECK(gemv_q4(NULL, NULL, NULL, NULL, 4, 100, 0) == GEMV_E_UNSUPPORTED);
    CHECK(gemv_q4(NULL, NULL, NULL, NULL, 4, 128, 0) == GEMV_E_INVAL);
    CHECK(gemv_quantize_q8(NULL, NULL, NULL, NULL, -1, 4, 0) == GEMV_E_INVAL);
    CHECK(gemv_quantize_q4(NULL, NULL, NULL, NULL, 4, 100, 0) != GEMV_OK);
    CHECK(gemv_softmax_f16(NULL, NULL, -1, 4, 0) == GEMV_E_INVAL);
    CHECK(gemv_softmax_f16(NULL, NULL, 0, 4, 0) == GEMV_OK);
    CHECK(gemv_probe_read(NULL, 15, NULL, 0, 0) == GEMV_E_INVAL);
    CHECK(gemv_probe_copy(NULL, NULL, 0, 0) == GEMV_OK);
    for (int s = -2; s < 8; ++s)
        CHECK(gemv_status_string(s) != NULL && strlen(gemv_status_string(s)) > 0);
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("host self-test: %ld plans and every argument check passed\n", plans);
    return failures ? 1 : 0;
}
