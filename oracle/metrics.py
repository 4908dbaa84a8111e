"""Parity metric between a GPU result and the oracle (test infrastructure).

The pages compare GPU output with a CPU reference through a relative error,
so that summation-order differences are absorbed ("cuda-gemv-optimization",
section "Correctness verification"), report the maximum relative error next
to every benchmark row ("membound", section "Results"), and floor the
denominator so that outputs near zero do not raise false alarms ("membound",
section "Bonus kernel: online softmax", which scores relative to
max(ref, 1e-4)).

Reading taken here: the floor scales with the row-result magnitude, at 1% of
the largest |reference| output, because GEMV outputs are sums of random-sign
terms and some land arbitrarily close to zero:

    err = max_i |y_i - r_i| / max(|r_i|, 0.01 * max_k |r_k|)

Gates: 1e-4 for the FP32 and dequantised INT8/INT4 paths, 2e-3 for FP16
inputs with FP32 accumulation, and 1e-4 for FP16 weights with FP32
activations (each product rounds once, like the FP32 path).  The lossy
FP16-accumulation path is gated instead by a componentwise bound derived from
its arithmetic (``acc16_bound``).  The unfloored elementwise maximum, the
normwise error and the componentwise error relative to sum_j |w_ij x_j| are
reported as diagnostics and never gated.
"""
from __future__ import annotations

import numpy as np

GATES = {"f32": 1e-4, "q8": 1e-4, "q4": 1e-4, "f16": 2e-3, "f16x32": 1e-4}
FLOOR_FRACTION = 0.01

U16 = 2.0 ** -11
U32 = 2.0 ** -24


def _gamma(k: int, u: float) -> float:
    return k * u / (1.0 - k * u) if k * u < 1.0 else float("inf")


def acc16_bound(abs_sum: np.ndarray, N: int) -> np.ndarray:
    """Componentwise error bound of the FP16-accumulation path.

    The llama.cpp walkthrough's implementation note says the original kernel
    may accumulate in FP16; the pages give no precision for that mode, so the
    bound is derived from the arithmetic.  Each lane keeps running sums in
    binary16, at most k = max(ceil(N/64), 4) terms per sum (one column per
    lane and pass in the element-wise kernel; four pairs per 16-byte chunk
    in the streaming kernel, whose 64 lanes cover 512 columns per pass, so
    that its 4 ceil(N/512) terms never exceed k), one rounding per term
    (relative u16 = 2^-11 for normal results; absolute at most 2^-25 in the
    subnormal range).  The sums are widened exactly and combined in FP32 in
    at most 8 levels.  The standard recursive-summation bound (Higham,
    "Accuracy and Stability of Numerical Algorithms", section 4.2) gives

        |y_i - r_i| <= ((1 + g16(k)) (1 + g32(8)) - 1) * sum_j |A_ij x_j|
                       + N * 2^-24,

    g(k) = k u / (1 - k u), with the subnormal terms (at most 2^-25 per
    column, before later roundings) bounded generously by 2^-24 per column.
    """
    k = max(-(-int(N) // 64), 4)
    a = np.asarray(abs_sum, dtype=np.float64)
    g16, g32 = _gamma(k, U16), _gamma(8, U32)
    return (g16 + g32 + g16 * g32) * a + N * 2.0 ** -24


def acc16_ratio(y: np.ndarray, ref: np.ndarray, abs_sum: np.ndarray, N: int) -> float:
    """max_i |y_i - r_i| / bound_i; at most 1 when the bound holds."""
    y = np.asarray(y, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    if y.size == 0:
        return 0.0
    if not np.all(np.isfinite(y)):
        return float("inf")
    return float(np.max(np.abs(y - r) / acc16_bound(abs_sum, N).ravel()))


def parity_error(y: np.ndarray, ref: np.ndarray) -> float:
    """Floored max relative error; NaN/Inf in either input give +inf."""
    y = np.asarray(y, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    if y.shape != r.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {r.shape}")
    if y.size == 0:
        return 0.0
    if not (np.all(np.isfinite(y)) and np.all(np.isfinite(r))):
        same = (np.isnan(y) & np.isnan(r)) | (y == r)
        if not np.all(same):
            return float("inf")
        finite = np.isfinite(r)
        y, r = y[finite], r[finite]
        if y.size == 0:
            return 0.0
    scale = np.max(np.abs(r))
    denom = np.maximum(np.abs(r), FLOOR_FRACTION * scale)
    err = np.abs(y - r)
    if scale == 0.0:
        return 0.0 if np.all(err == 0.0) else float("inf")
    return float(np.max(err / denom))


def parity_report(y: np.ndarray, ref: np.ndarray, abs_sum: np.ndarray | None = None) -> dict:
    """Gated metric plus ungated diagnostics."""
    y64 = np.asarray(y, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    out = {"floored_rel": parity_error(y64, r)}
    if r.size:
        err = np.abs(y64 - r)
        with np.errstate(divide="ignore", invalid="ignore"):
            out["elementwise_rel"] = float(np.max(np.where(r != 0, err / np.abs(r), np.where(err == 0, 0.0, np.inf))))
        m = float(np.max(np.abs(r)))
        out["normwise_rel"] = float(np.max(err) / m) if m > 0 else float(np.max(err))
        if abs_sum is not None:
            a = np.asarray(abs_sum, dtype=np.float64).ravel()
            with np.errstate(divide="ignore", invalid="ignore"):
                out["componentwise"] = float(np.max(np.where(a > 0, err / a, 0.0)))
    return out


# ---------------------------------------------------------------- softmax
SOFTMAX_FLOOR = 1e-4
SOFTMAX_GATE = 2e-3


def softmax_error(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - r| / max(|r|, 1e-4): the "membound" page scores its FP16
    softmax relative to max(ref, 1e-4) so that binary16-subnormal outputs
    (below about 6e-5, where relative precision collapses) raise no false
    alarms (section "Bonus kernel: online softmax").  Gate 2e-3, as for the
    other binary16 results: binary16 output rounding alone is up to 2^-11
    (4.9e-4) relative, or 2^-25 absolute (3e-4 against the floor) for
    subnormal outputs.  NaN must meet NaN."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if y.shape != r.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {r.shape}")
    if y.size == 0:
        return 0.0
    nan_r, nan_y = np.isnan(r), np.isnan(y)
    if np.any(nan_r != nan_y):
        return float("inf")
    ok = ~nan_r
    if not np.any(ok):
        return 0.0
    return float(np.max(np.abs(y[ok] - r[ok]) / np.maximum(np.abs(r[ok]), SOFTMAX_FLOOR)))
