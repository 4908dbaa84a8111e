/*
 * C-only smoke test of the library's C ABI (test infrastructure): plain C,
 * the HIP runtime's C API for device memory, the library through
 * include/gemv.h, and the CPU oracle library as the reference.  Runs each
 * GEMV format, the quantiser and the softmax once on a small seeded case
 * and checks the results (FP16 weights with an FP32 x included); exits 0 on success, 1 on a mismatch, 2 on a setup
 * error.  Built by __graft_entry__.build(); run by tests/test_gpu_c_smoke.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gemv.h"
#include "gemv_quant.h"
#include "gemv_softmax.h"

/* oracle entry points (oracle/gemv_oracle.c, quant_oracle.c, softmax_oracle.c) */
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

#define M 300
#define N 2048

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni(void) /* splitmix64 -> [-1, 1) */
{
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static void* dev_copy(const void* h, size_t n)
{
    void* d = NULL;
    if (hipMalloc(&d, n) != hipSuccess || hipMemcpy(d, h, n, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "device allocation failed\n");
        exit(2);
    }
    return d;
}

static double floored_rel(const float* y, const double* r, int n)
{
    double mx = 0, e = 0;
    for (int i = 0; i < n; ++i)
        mx = fmax(mx, fabs(r[i]));
    for (int i = 0; i < n; ++i) {
        const double den = fmax(fabs(r[i]), 0.01 * mx);
        e = fmax(e, fabs(y[i] - r[i]) / den);
    }
    return e;
}

static int check(const char* what, int rc, double err, double gate)
{
    printf("c-smoke %-12s status %d  error %.3e  gate %.0e\n", what, rc, err, gate);
    return rc == GEMV_OK && err <= gate;
}

int main(void)
{
    int ok = 1;
    static float A32[M * N], x32[N], W[M * N];
    static uint16_t A16[M * N], x16[N], s8[M], s4[M * (N / 128)], sx[M * N], sy[M * N];
    static int8_t A8[M * N];
    static uint8_t A4[M * N / 2];
    static double ref[M * N];
    static float y[M];
    for (int i = 0; i < M * N; ++i) {
        A32[i] = (float)uni();
        A16[i] = oracle_double_to_half(uni() / 45.0);
        A8[i] = (int8_t)(int)floor(uni() * 127.5);
        W[i] = (float)uni();
        sx[i] = oracle_double_to_half(3.0 * uni());
    }
    for (int i = 0; i < M * N / 2; ++i)
        A4[i] = (uint8_t)(int)floor((uni() + 1.0) * 128.0);
    for (int j = 0; j < N; ++j) {
        x32[j] = (float)uni();
        x16[j] = oracle_double_to_half(uni());
    }
    for (int i = 0; i < M; ++i)
        s8[i] = oracle_double_to_half((1.0 + 0.5 * uni()) / 127.0);
    for (int i = 0; i < M * (N / 128); ++i)
        s4[i] = oracle_double_to_half((1.0 + 0.5 * uni()) / 7.0);

    float* dy = NULL;
    if (hipMalloc((void**)&dy, sizeof y) != hipSuccess)
        return 2;
    void* dA32 = dev_copy(A32, sizeof A32);
    void* dx32 = dev_copy(x32, sizeof x32);
    void* dA16 = dev_copy(A16, sizeof A16);
    void* dx16 = dev_copy(x16, sizeof x16);
    void* dA8 = dev_copy(A8, sizeof A8);
    void* ds8 = dev_copy(s8, sizeof s8);
    void* dA4 = dev_copy(A4, sizeof A4);
    void* ds4 = dev_copy(s4, sizeof s4);
    int rc;

    rc = gemv_f32((const float*)dA32, (const float*)dx32, dy, M, N, 0);
    hipMemcpy(y, dy, sizeof y, hipMemcpyDeviceToHost);
    oracle_gemv_f32(A32, x32, ref, M, N);
    ok &= check("gemv_f32", rc, floored_rel(y, ref, M), 1e-4);

    rc = gemv_f16((const uint16_t*)dA16, (const uint16_t*)dx16, dy, M, N, 0);
    hipMemcpy(y, dy, sizeof y, hipMemcpyDeviceToHost);
    oracle_gemv_f16(A16, x16, ref, M, N);
    ok &= check("gemv_f16", rc, floored_rel(y, ref, M), 2e-3);

    rc = gemv_f16x32((const uint16_t*)dA16, (const float*)dx32, dy, M, N, 0);
    hipMemcpy(y, dy, sizeof y, hipMemcpyDeviceToHost);
    oracle_gemv_f16x32(A16, x32, ref, M, N);
    ok &= check("gemv_f16x32", rc, floored_rel(y, ref, M), 1e-4);

    rc = gemv_q8((const int8_t*)dA8, (const uint16_t*)ds8, (const uint16_t*)dx16, dy, M, N, 0);
    hipMemcpy(y, dy, sizeof y, hipMemcpyDeviceToHost);
    oracle_gemv_q8(A8, s8, x16, ref, M, N);
    ok &= check("gemv_q8", rc, floored_rel(y, ref, M), 1e-4);

    rc = gemv_q4((const uint8_t*)dA4, (const uint16_t*)ds4, (const uint16_t*)dx16, dy, M, N, 0);
    hipMemcpy(y, dy, sizeof y, hipMemcpyDeviceToHost);
    oracle_gemv_q4(A4, s4, x16, ref, M, N);
    ok &= check("gemv_q4", rc, floored_rel(y, ref, M), 1e-4);

    /* quantiser: codes and scales bit for bit */
    {
        static int8_t q[M * N], oq[M * N];
        static uint16_t s[M], os[M];
        void* dW = dev_copy(W, sizeof W);
        void *dq = NULL, *ds = NULL;
        hipMalloc(&dq, sizeof q);
        hipMalloc(&ds, sizeof s);
        rc = gemv_quantize_q8((const float*)dW, (int8_t*)dq, (uint16_t*)ds, NULL, M, N, 0);
        hipMemcpy(q, dq, sizeof q, hipMemcpyDeviceToHost);
        hipMemcpy(s, ds, sizeof s, hipMemcpyDeviceToHost);
        oracle_quantize_q8(W, oq, os, NULL, M, N);
        const int same = memcmp(q, oq, sizeof q) == 0 && memcmp(s, os, sizeof s) == 0;
        ok &= check("quantize_q8", rc, same ? 0.0 : 1.0, 0.0);
        hipFree(dW);
        hipFree(dq);
        hipFree(ds);
    }

    /* INT4 quantiser: codes and group scales bit for bit */
    {
        static uint8_t q[M * N / 2], oq[M * N / 2];
        static uint16_t s[M * (N / 128)], os[M * (N / 128)];
        void* dW = dev_copy(W, sizeof W);
        void *dq = NULL, *ds = NULL;
        hipMalloc(&dq, sizeof q);
        hipMalloc(&ds, sizeof s);
        rc = gemv_quantize_q4((const float*)dW, (uint8_t*)dq, (uint16_t*)ds, NULL, M, N, 0);
        hipMemcpy(q, dq, sizeof q, hipMemcpyDeviceToHost);
        hipMemcpy(s, ds, sizeof s, hipMemcpyDeviceToHost);
        memset(oq, 0, sizeof oq);
        oracle_quantize_q4(W, oq, os, NULL, M, N);
        const int same = memcmp(q, oq, sizeof q) == 0 && memcmp(s, os, sizeof s) == 0;
        ok &= check("quantize_q4", rc, same ? 0.0 : 1.0, 0.0);
        hipFree(dW);
        hipFree(dq);
        hipFree(ds);
    }

    /* softmax: error relative to max(|ref|, 1e-4) */
    {
        void* dx = dev_copy(sx, sizeof sx);
        void* dyh = NULL;
        hipMalloc(&dyh, sizeof sy);
        rc = gemv_softmax_f16((const uint16_t*)dx, (uint16_t*)dyh, M, N, 0);
        hipMemcpy(sy, dyh, sizeof sy, hipMemcpyDeviceToHost);
        oracle_softmax_f16(sx, ref, M, N);
        double e = 0;
        for (int i = 0; i < M * N; ++i)
            e = fmax(e, fabs(oracle_half_to_double(sy[i]) - ref[i]) / fmax(fabs(ref[i]), 1e-4));
        ok &= check("softmax_f16", rc, e, 2e-3);
        hipFree(dx);
        hipFree(dyh);
    }

    /* status codes need no device work */
    ok &= gemv_f16(NULL, NULL, dy, -1, N, 0) == GEMV_E_INVAL;
    ok &= gemv_q4((const uint8_t*)dA4, (const uint16_t*)ds4, (const uint16_t*)dx16, dy, M, 200, 0) == GEMV_E_UNSUPPORTED;
    printf("c-smoke status strings: %s / %s\n", gemv_status_string(GEMV_OK), gemv_status_string(GEMV_E_UNSUPPORTED));

    hipFree(dy);
    hipFree(dA32); hipFree(dx32); hipFree(dA16); hipFree(dx16);
    hipFree(dA8); hipFree(ds8); hipFree(dA4); hipFree(ds4);
    printf("c-smoke %s\n", ok ? "PASSED" : "FAILED");
    return ok ? 0 : 1;
}
