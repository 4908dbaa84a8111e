/*
 * CPU oracle for the row-wise softmax of an FP16 matrix, the second
 * memory-bound decode kernel of the "membound" page (section "Bonus kernel:
 * online softmax").
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * The page's kernel computes the row maximum and the normaliser in one sweep
 * with the online update and normalises in a second pass; up to rounding
 * that reaches exactly the plain definition, which is what this oracle
 * computes, in double, for every row i of x[M][N] (binary16 inputs):
 *
 *     m_i = max_j x_ij,   d_i = sum_j exp(x_ij - m_i),   y_ij = exp(x_ij - m_i) / d_i.
 *
 * IEEE special values follow from the formula: -inf entries give 0; a row of
 * only -inf, or with +inf or NaN, gives NaN.  The result is returned in
 * double (not rounded to binary16); the comparison with the GPU's binary16
 * output scores relative to max(|reference|, 1e-4), as the page does.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off, libm exp.
 */
#include <math.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* binary16 bit pattern -> double (IEEE 754: bias 15, 10 fraction bits,
 * subnormals f * 2^-24, exponent 31 infinity or NaN). */
static double s_half_to_double(uint16_t h)
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

int oracle_softmax_f16(const uint16_t* x, double* y, int64_t M, int64_t N)
{
    if (M < 0 || N < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        const uint16_t* row = x + i * N;
        double* out = y + i * N;
        double m = -INFINITY;
        int nan = 0;
        for (int64_t j = 0; j < N; ++j) {
            const double v = s_half_to_double(row[j]);
            if (isnan(v))
                nan = 1;
            else if (v > m)
                m = v;
        }
        double d = 0.0;
        for (int64_t j = 0; j < N; ++j)
            d += exp(s_half_to_double(row[j]) - m);
        for (int64_t j = 0; j < N; ++j)
            out[j] = nan ? NAN : exp(s_half_to_double(row[j]) - m) / d;
    }
    return 0;
}
