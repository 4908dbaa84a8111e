/*
 * Self-test of the C oracle (test infrastructure), built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/sanitize/build.py and run by
 * tests/test_sanitize_cpu.py.  Every oracle entry point runs on small cases
 * whose results are known in closed form, including empty and ragged shapes,
 * so that an out-of-bounds access or undefined arithmetic in the oracle
 * stops the run.  Exits 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemv_f32(const float* A, const float* x, double* y, int64_t M, int64_t N);
int oracle_gemv_f16(const uint16_t* A, const uint16_t* x, double* y, int64_t M, int64_t N);
int oracle_gemv_f16x32(const uint16_t* A, const float* x, double* y, int64_t M, int64_t N);
int oracle_gemv_q8(const int8_t* A, const uint16_t* s, const uint16_t* x, double* y, int64_t M, int64_t N);
int oracle_gemv_q4(const uint8_t* A, const uint16_t* s, const uint16_t* x, double* y, int64_t M, int64_t N);
int oracle_quantize_q8(const float* W, int8_t* q, uint16_t* s, double* e, int64_t M, int64_t N);
int oracle_quantize_q4(const float* W, uint8_t* q, uint16_t* s, double* e, int64_t M, int64_t N);
int oracle_softmax_f16(const uint16_t* x, double* y, int64_t M, int64_t N);
uint16_t oracle_double_to_half(double v);
double oracle_half_to_double(uint16_t h);

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t state = 12345;
static int small_int(void) /* -3..3, from a 64-bit LCG */
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (int)((state >> 33) % 7) - 3;
}

int main(void)
{
    /* every binary16 pattern survives the round trip through double */
    for (uint32_t h = 0; h < 65536; ++h) {
        const double v = oracle_half_to_double((uint16_t)h);
        if (v == v)
            CHECK(oracle_double_to_half(v) == (uint16_t)h || (v == 0.0 && ((h & 0x7FFF) == 0)));
    }
    /* identity and row sums, ragged shapes, FP32 / FP16 / FP16 with FP32 x */
    for (int64_t M = 1; M <= 9; M += 4) {
        for (int64_t N = 1; N <= 67; N += 11) {
            float* A = calloc((size_t)(M * N), sizeof(float));
            uint16_t* Ah = calloc((size_t)(M * N), sizeof(uint16_t));
            float* x = malloc((size_t)N * sizeof(float));
            uint16_t* xh = malloc((size_t)N * sizeof(uint16_t));
            double* y = malloc((size_t)M * sizeof(double));
            double rowsum_ref = 0;
            for (int64_t j = 0; j < N; ++j) {
                x[j] = (float)small_int();
                xh[j] = oracle_double_to_half(x[j]);
                rowsum_ref += x[j];
            }
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j) {
                    A[i * N + j] = 1.0f;
                    Ah[i * N + j] = oracle_double_to_half(1.0);
                }
            CHECK(oracle_gemv_f32(A, x, y, M, N) == 0);
            for (int64_t i = 0; i < M; ++i)
                CHECK(y[i] == rowsum_ref);
            CHECK(oracle_gemv_f16(Ah, xh, y, M, N) == 0);
            for (int64_t i = 0; i < M; ++i)
                CHECK(y[i] == rowsum_ref);
            CHECK(oracle_gemv_f16x32(Ah, x, y, M, N) == 0);
            for (int64_t i = 0; i < M; ++i)
                CHECK(y[i] == rowsum_ref);
            free(A), free(Ah), free(x), free(xh), free(y);
        }
    }
    /* INT8 and INT4: one-hot x picks a column, q * s exactly */
    {
        const int64_t M = 5, N = 256;
        int8_t* q8 = malloc((size_t)(M * N));
        uint8_t* q4 = malloc((size_t)(M * N / 2));
        uint16_t s8[5], s4[5 * 2], x[256];
        double y[5];
        for (int64_t k = 0; k < M * N; ++k)
            q8[k] = (int8_t)(k % 255 - 127);
        for (int64_t k = 0; k < M * N / 2; ++k)
            q4[k] = (uint8_t)(k * 37 + 11);
        for (int i = 0; i < 5; ++i)
            s8[i] = oracle_double_to_half(0.5);
        for (int i = 0; i < 10; ++i)
            s4[i] = oracle_double_to_half(i % 2 ? 0.25 : 2.0);
        for (int64_t c = 0; c < N; c += 37) {
            for (int64_t j = 0; j < N; ++j)
                x[j] = oracle_double_to_half(j == c ? 1.0 : 0.0);
            CHECK(oracle_gemv_q8(q8, s8, x, y, M, N) == 0);
            for (int64_t i = 0; i < M; ++i)
                CHECK(y[i] == 0.5 * q8[i * N + c]);
            CHECK(oracle_gemv_q4(q4, s4, x, y, M, N) == 0);
            for (int64_t i = 0; i < M; ++i) {
                const uint8_t b = q4[i * N / 2 + c / 2];
                const int nib = c % 2 ? b >> 4 : b & 15;
                const int qv = nib >= 8 ? nib - 16 : nib;
                CHECK(y[i] == qv * (c / 128 ? 0.25 : 2.0));
            }
        }
        free(q8), free(q4);
    }
    /* quantiser: codes within range, dequantised weight within half a step */
    {
        const int64_t M = 3, N = 384;
        float* W = malloc((size_t)(M * N) * sizeof(float));
        int8_t* q8 = malloc((size_t)(M * N));
        uint8_t* q4 = calloc((size_t)(M * N / 2), 1);
        uint16_t s8[3], s4[3 * 3];
        double e[3];
        for (int64_t k = 0; k < M * N; ++k)
            W[k] = (float)(small_int() * 0.3 + 0.01 * (double)(k % 7));
        CHECK(oracle_quantize_q8(W, q8, s8, e, M, N) == 0);
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                const double s = oracle_half_to_double(s8[i]);
                CHECK(q8[i * N + j] >= -127 && q8[i * N + j] <= 127);
                CHECK(fabs(q8[i * N + j] * s - W[i * N + j]) <= 0.5 * s * (1 + 1e-3) + 1e-7);
            }
        CHECK(oracle_quantize_q4(W, q4, s4, e, M, N) == 0);
        for (int64_t i = 0; i < M; ++i)
            CHECK(e[i] >= 0);
        free(W), free(q8), free(q4);
    }
    /* softmax: rows sum to one, empty shapes accepted */
    {
        const int64_t M = 4, N = 33;
        uint16_t x[4 * 33];
        double y[4 * 33];
        for (int k = 0; k < M * N; ++k)
            x[k] = oracle_double_to_half(small_int());
        CHECK(oracle_softmax_f16(x, y, M, N) == 0);
        for (int64_t i = 0; i < M; ++i) {
            double t = 0;
            for (int64_t j = 0; j < N; ++j)
                t += y[i * N + j];
            CHECK(fabs(t - 1.0) < 1e-12);
        }
        CHECK(oracle_softmax_f16(x, y, 0, N) == 0);
    }
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("oracle self-test: all checks passed\n");
    return failures ? 1 : 0;
}
