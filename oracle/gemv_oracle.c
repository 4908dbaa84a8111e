/*
 * CPU oracle for row-major GEMV, y[M] = A[M,N] . x[N].
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes, and where that is defined:
 *   - The product itself is the plain definition y_i = sum_j A_ij x_j
 *     ("Making GEMV Fast", section "Algorithm"; the llama.cpp FP16 GEMV
 *     walkthrough, opening equation y_i = sum_j W_ij x_j).
 *   - A is dense row-major: element (i, j) sits at linear offset i*N + j
 *     ("Making GEMV Fast", section "Row-major indexing refresher").
 *   - INT8 weights carry one symmetric scale per row; INT4 weights carry one
 *     symmetric scale per group of 128 columns; the reference value of a
 *     weight is exactly q*s ("membound", section "The kernel decode actually
 *     runs: dequant GEMV").  Scales are IEEE binary16.  INT4 storage: two
 *     signed (two's complement) nibbles per byte, the low nibble holding the
 *     even column.
 *   - The reference is computed in double on every run, before anything is
 *     timed ("membound", section "Correctness").
 *
 * Arithmetic: every operand is decoded to double, every product w_ij * x_j is
 * exact in double (at most 48 significant bits), and the N additions run in
 * column order j = 0..N-1, starting from 0.0.  The only rounding is in those
 * additions.  No blocking, no fusion, no reordering within a row.  Rows are
 * independent, so they are spread over OpenMP threads; that does not change
 * any row's result.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16 -> double, written from the format's definition:
 * 1 sign bit, 5 exponent bits with bias 15, 10 fraction bits.
 *   exponent 0     : subnormal, value = fraction * 2^-24 (i.e. f/1024 * 2^-14)
 *   exponent 1..30 : normal,    value = (1024 + fraction) * 2^(e - 25)
 *   exponent 31    : infinity (fraction 0) or NaN (fraction != 0)          */
static double half_bits_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

double oracle_half_to_double(uint16_t h) { return half_bits_to_double(h); }

/* Decode a whole array (used by the decoder's own pin over all 65536 codes). */
void oracle_half_to_double_array(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t k = 0; k < n; ++k)
        out[k] = half_bits_to_double(h[k]);
}

/* Signed value of column j's nibble in one INT4 row: byte j/2, low nibble for
 * even j, high nibble for odd j, two's complement (8..15 mean -8..-1). */
static int int4_value(const uint8_t* row, int64_t j)
{
    const uint8_t b = row[j / 2];
    const int nib = (j % 2 == 0) ? (b & 0x0F) : (b >> 4);
    return nib >= 8 ? nib - 16 : nib;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following parallel regions (benchmark leg: all host
 * threads, then one).  Does not change any result. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* FP32 A and x. */
int oracle_gemv_f32(const float* A, const float* x, double* y, int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const float* row = A + i * N;
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j)
            acc += (double)row[j] * (double)x[j];
        y[i] = acc;
    }
    return 0;
}

/* FP16 A and x (binary16 bit patterns). */
int oracle_gemv_f16(const uint16_t* A, const uint16_t* x, double* y, int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const uint16_t* row = A + i * N;
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j)
            acc += half_bits_to_double(row[j]) * half_bits_to_double(x[j]);
        y[i] = acc;
    }
    return 0;
}

/* FP16 A (binary16 bit patterns) with an FP32 x: the hidden state kept in
 * FP32 (llama.cpp FP16 GEMV walkthrough, implementation note on the
 * original kernel).  Each product (11 x 24 significant bits) is exact in
 * double. */
int oracle_gemv_f16x32(const uint16_t* A, const float* x, double* y, int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const uint16_t* row = A + i * N;
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j)
            acc += half_bits_to_double(row[j]) * (double)x[j];
        y[i] = acc;
    }
    return 0;
}

/* INT8 A with one binary16 scale per row; w_ij = q_ij * s_i. */
int oracle_gemv_q8(const int8_t* A, const uint16_t* scale, const uint16_t* x, double* y,
                   int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const int8_t* row = A + i * N;
        const double s = half_bits_to_double(scale[i]);
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double w = (double)row[j] * s;
            acc += w * half_bits_to_double(x[j]);
        }
        y[i] = acc;
    }
    return 0;
}

/* INT4 A, packed [M][N/2], with one binary16 scale per row and 128-column
 * group, stored [M][N/128]; w_ij = q_ij * s_{i, j/128}.  N must be a
 * multiple of 128 (the group width). */
int oracle_gemv_q4(const uint8_t* A, const uint16_t* scale, const uint16_t* x, double* y,
                   int64_t M, int64_t N)
{
    if (M < 0 || N < 0 || N % 128 != 0)
        return -1;
    const int64_t groups = N / 128;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const uint8_t* row = A + i * (N / 2);
        const uint16_t* srow = scale + i * groups;
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double w = (double)int4_value(row, j) * half_bits_to_double(srow[j / 128]);
            acc += w * half_bits_to_double(x[j]);
        }
        y[i] = acc;
    }
    return 0;
}
