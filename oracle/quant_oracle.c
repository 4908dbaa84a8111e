/*
 * CPU oracle for the weight quantiser that produces the INT8 and INT4
 * operands of the GEMV path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What the pages fix ("membound", section "The kernel decode actually runs:
 * dequant GEMV"): INT8 weights are symmetric with one scale per row; INT4
 * weights are symmetric with one scale per group of 128 columns; the scales
 * are binary16; a weight's reference value is exactly q*s; the quantisation
 * error is reported on its own as an RMSE (2.3e-3 for INT8 and 4.1e-2 for
 * INT4 on weights uniform on [-1, 1]).
 *
 * What the pages leave open, and the reading taken here:
 *   - the scale is the absolute maximum over the row (INT8) or group (INT4)
 *     divided by the largest code, 127 or 7 (symmetric absmax scaling; the
 *     page's RMSE figures are what this rule gives on U[-1, 1]);
 *   - the scale is rounded to binary16 (round to nearest, ties to even)
 *     before the codes are chosen, so that q*s with the stored s is the
 *     weight the GEMV reads; a scale beyond binary16's range is clamped to
 *     65504, one that rounds to zero gives all-zero codes;
 *   - a code is w / s rounded to the nearest integer, ties to even, and
 *     clipped to [-127, 127] or [-7, 7] (clipping only bites when the
 *     binary16 scale lies below the exact one, i.e. in binary16's
 *     subnormal range);
 *   - these decisions (the division by the largest code, the rounding of the
 *     scale, the division w / s) are taken in IEEE binary32, the precision
 *     the GPU takes them in, so that both sides choose the same integers;
 *   - RMSE = sqrt(sum of (q*s - w)^2 over all weights / (M*N)), with the sum
 *     per row returned here in double.
 * INT4 storage: two's-complement nibbles, two per byte, the low nibble
 * holding the even column; scales [M][N/128] row-major.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off (binary32 operations stay
 * binary32 on x86-64: FLT_EVAL_METHOD is 0 with SSE arithmetic).
 */
#include <math.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* binary16 bit pattern -> double (IEEE 754 definition: bias 15, 10 fraction
 * bits, subnormals f * 2^-24). */
static double q_half_to_double(uint16_t h)
{
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (h & 0x8000) ? -v : v;
}

/* Round a non-negative double to the nearest integer, ties to even. */
static double round_half_even(double m)
{
    const double f = floor(m);
    const double d = m - f;           /* exact for m < 2^52 */
    if (d > 0.5)
        return f + 1.0;
    if (d < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* double -> binary16 bit pattern, round to nearest, ties to even, from the
 * format's definition.  Finite values of magnitude >= 65520 (the midpoint
 * between 65504 and 2^16) overflow to infinity. */
static uint16_t double_to_half(double v)
{
    if (isnan(v))
        return 0x7E00;
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (a >= 65520.0)
        return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: multiples of 2^-24; 1024 * 2^-24 is the smallest
         * normal, whose bit pattern 0x0400 is the carry of the fraction */
        const double r = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)r;
    }
    int E;
    frexp(a, &E);                     /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                    /* a in [2^e, 2^(e+1)) */
    double r = round_half_even(ldexp(a, 10 - e));   /* in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)r - 1024));
}

uint16_t oracle_double_to_half(double v) { return double_to_half(v); }

/* Scale of one row or group: binary32 absmax / qmax, rounded to binary16,
 * clamped to the largest finite binary16. */
static uint16_t scale_of(float amax, float qmax)
{
    const float s = amax / qmax;      /* one binary32 division */
    uint16_t h = double_to_half((double)s);
    if (h == 0x7C00)
        h = 0x7BFF;
    return h;
}

/* Code of one weight against the binary16 scale sf (as binary32). */
static int code_of(float w, float sf, float qmax)
{
    if (sf == 0.0f)
        return 0;
    const float t = w / sf;           /* one binary32 division */
    if (isnan(t))
        return 0;                     /* a NaN weight has no code under the rule; 0 keeps this defined */
    double r = (t < 0.0f) ? -round_half_even(-(double)t) : round_half_even((double)t);
    if (r > qmax)
        r = qmax;
    if (r < -qmax)
        r = -qmax;
    return (int)r;
}

/* INT8: q int8[M*N], scale binary16[M], row_sse double[M] (may be NULL). */
int oracle_quantize_q8(const float* W, int8_t* q, uint16_t* scale, double* row_sse, int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const float* w = W + i * N;
        float amax = 0.0f;
        for (int64_t j = 0; j < N; ++j)
            if (fabsf(w[j]) > amax)
                amax = fabsf(w[j]);
        const uint16_t h = scale_of(amax, 127.0f);
        const double s = q_half_to_double(h);
        scale[i] = h;
        double sse = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const int c = code_of(w[j], (float)s, 127.0f);
            q[i * N + j] = (int8_t)c;
            const double d = (double)c * s - (double)w[j];
            sse += d * d;
        }
        if (row_sse)
            row_sse[i] = sse;
    }
    return 0;
}

/* INT4: q uint8[M*N/2] (low nibble = even column), scale binary16[M*N/128],
 * row_sse double[M] (may be NULL).  N must be a multiple of 128. */
int oracle_quantize_q4(const float* W, uint8_t* q, uint16_t* scale, double* row_sse, int64_t M, int64_t N)
{
    if (M < 0 || N < 0 || N % 128 != 0)
        return -1;
    const int64_t G = N / 128;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double sse = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            const float* w = W + i * N + g * 128;
            float amax = 0.0f;
            for (int j = 0; j < 128; ++j)
                if (fabsf(w[j]) > amax)
                    amax = fabsf(w[j]);
            const uint16_t h = scale_of(amax, 7.0f);
            const double s = q_half_to_double(h);
            scale[i * G + g] = h;
            for (int j = 0; j < 128; ++j) {
                const int c = code_of(w[j], (float)s, 7.0f);
                const int64_t col = g * 128 + j;
                uint8_t* byte = &q[i * (N / 2) + col / 2];
                const uint8_t nib = (uint8_t)(c & 0xF);        /* two's complement */
                if (col % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xF0) | nib);
                else
                    *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
                const double d = (double)c * s - (double)w[j];
                sse += d * d;
            }
        }
        if (row_sse)
            row_sse[i] = sse;
    }
    return 0;
}
