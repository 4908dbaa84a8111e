/*
 * gemv_softmax.h -- C ABI of the row-wise softmax of a binary16 matrix, the
 * second memory-bound decode kernel ("membound", section "Bonus kernel:
 * online softmax"), in the same library as the GEMV (include/gemv.h).
 *
 *     y_ij = exp(x_ij - m_i) / sum_k exp(x_ik - m_i),   m_i = max_k x_ik
 *
 * x and y are binary16 [M][N] row-major (uint16_t bit patterns).  The row
 * maximum and normaliser are found in one sweep with the online update
 * m' = max(m, x), d = d e^(m - m') + e^(x - m') (Milakov and Gimelshein,
 * as on that page); all arithmetic is FP32 and outputs are rounded to
 * nearest even binary16.  Floor traffic is one read and one write of each
 * element: rows of up to 131072 columns are held in registers between the
 * sweep and the normalisation, longer rows are read twice.
 *
 * Special values follow the formula: -inf entries give 0; a row of only
 * -inf, or holding +inf or NaN, gives NaN throughout.  Outputs below
 * binary16's normal range (about 6.1e-5) are subnormal and carry absolute,
 * not relative, precision.
 *
 * Conventions: device pointers, caller-owned buffers, asynchronous on
 * `stream`, gemv_status codes, nothing allocated, deterministic.  y must not
 * overlap x.  M == 0 or N == 0 is a no-op.  The bandwidth path needs
 * 16-byte-aligned x and y and N % 8 == 0; other inputs take an element-wise
 * path.
 */
#ifndef MBGR_GEMV_SOFTMAX_H
#define MBGR_GEMV_SOFTMAX_H

#include <stdint.h>

#include "gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* GEMV_E_INVAL for negative sizes or a missing x or y when M*N > 0. */
int gemv_softmax_f16(const uint16_t* x, uint16_t* y, int M, int N, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MBGR_GEMV_SOFTMAX_H */
