/*
 * gemv_quant.h -- C ABI of the weight quantiser that produces the INT8 and
 * INT4 operands of gemv_q8 / gemv_q4 (include/gemv.h) from FP32 weights, and
 * reports the quantisation error.
 *
 * Formats ("membound", section "The kernel decode actually runs: dequant
 * GEMV"): INT8 symmetric with one binary16 scale per row; INT4 symmetric
 * with one binary16 scale per group of 128 columns, two's-complement
 * nibbles, two per byte, the even column in the low nibble.  That page
 * reports the quantisation error separately from the GEMV's parity check,
 * as an RMSE on U[-1, 1] weights.
 *
 * Rule (the page names the formats, not the rule; absmax scaling reproduces
 * its RMSE figures):
 *   scale = absmax / qmax, qmax = 127 (INT8) or 7 (INT4), one IEEE binary32
 *           division, then rounded to the nearest binary16 (ties to even);
 *           a scale beyond 65504 is clamped to 65504;
 *   code  = w / scale, one binary32 division, rounded to the nearest integer
 *           (ties to even) and clipped to [-qmax, qmax]; a zero scale gives
 *           zero codes.
 * So q * scale, with the stored scale, is the weight gemv_q8 / gemv_q4 read,
 * and |q * scale - w| <= scale / 2 wherever no clipping occurs.
 *
 * Conventions: device pointers, caller-owned buffers, asynchronous on
 * `stream`, status codes from gemv.h (gemv_status), nothing allocated.
 * An infinite weight gives its row (INT8) or group (INT4) the largest
 * binary16 scale, 65504, and clipped codes; a NaN weight has no code under
 * the rule and gets code 0 (its row's row_sse is NaN).
 * row_sse, if not NULL, receives per row sum_j (q_ij * scale - w_ij)^2 in
 * FP32; RMSE = sqrt(sum_i row_sse[i] / (M * N)).  Results are deterministic.
 * The bandwidth path needs a 16-byte-aligned W (and, for INT8, N % 4 == 0
 * and a 4-byte-aligned q); other inputs take an element-wise path.
 */
#ifndef MBGR_GEMV_QUANT_H
#define MBGR_GEMV_QUANT_H

#include <stdint.h>

#include "gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* INT8: W float[M*N] row-major -> q int8[M*N], scale binary16[M],
 * row_sse float[M] (optional).  N == 0 writes scale = 0 and row_sse = 0.
 * GEMV_E_INVAL for negative sizes or a missing W, q or scale. */
int gemv_quantize_q8(const float* W, int8_t* q, uint16_t* scale, float* row_sse, int M, int N,
                     hipStream_t stream);

/* INT4: W float[M*N] row-major -> q uint8[M*(N/2)], scale binary16[M*(N/128)]
 * row-major, row_sse float[M] (optional).  N must be a multiple of 128
 * (GEMV_E_UNSUPPORTED otherwise). */
int gemv_quantize_q4(const float* W, uint8_t* q, uint16_t* scale, float* row_sse, int M, int N,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MBGR_GEMV_QUANT_H */
