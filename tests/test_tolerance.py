"""Pins for the parity metric and its gates (CPU only).

The gate must accept every correctly rounded FP32-accumulating order a GPU
may use and reject an FP16 accumulator (the pages' FP16 path accumulates in
FP32: llama.cpp FP16 GEMV walkthrough, and "membound", section "The stages,
and what Nsight says about each", stage 3).  Both are emulated here in numpy
on the workloads' own value distributions.
"""
import numpy as np
import pytest

from oracle.metrics import GATES, parity_error, parity_report


def _wave_order_f32(W, x, elems_per_lane):
    """Emulate one 64-lane wave per row: lane l accumulates (in float32) the
    chunks l, l+64, ... of elems_per_lane consecutive columns, then a
    butterfly combines the 64 partials."""
    M, N = W.shape
    chunk = 64 * elems_per_lane
    assert N % chunk == 0
    Wc = W.reshape(M, N // chunk, 64, elems_per_lane).astype(np.float32)
    xc = x.reshape(N // chunk, 64, elems_per_lane).astype(np.float32)
    acc = np.zeros((M, 64), np.float32)
    for p in range(N // chunk):
        for e in range(elems_per_lane):
            acc = (acc + Wc[:, p, :, e] * xc[p, :, e]).astype(np.float32)
    width = 64
    while width > 1:
        width //= 2
        acc = (acc[:, :width] + acc[:, width:2 * width]).astype(np.float32)
    return acc[:, 0]


def _running_sum_f16(W, x):
    acc = np.zeros(W.shape[0], np.float16)
    for j in range(W.shape[1]):
        acc = (acc + (W[:, j].astype(np.float32) * np.float32(x[j])).astype(np.float16)).astype(np.float16)
    return acc


def test_metric_basics():
    r = np.array([100.0, -50.0, 0.0, 1e-9])
    assert parity_error(r, r) == 0.0
    # errors near zero are measured against 1% of the largest |r|
    y = r + np.array([0.0, 0.0, 0.5, 0.0])
    assert parity_error(y, r) == pytest.approx(0.5)
    y = r + np.array([1e-3, 0.0, 0.0, 0.0])
    assert parity_error(y, r) == pytest.approx(1e-5)
    assert parity_error(np.array([np.nan]), np.array([1.0])) == float("inf")
    assert parity_error(np.array([np.nan, 1.0]), np.array([np.nan, 1.0])) == 0.0
    assert parity_error(np.zeros(0), np.zeros(0)) == 0.0
    rep = parity_report(y, r, abs_sum=np.abs(r) + 1)
    assert set(rep) >= {"floored_rel", "elementwise_rel", "normwise_rel", "componentwise"}


def test_gate_accepts_correct_fp32_order_f32_workload():
    rng = np.random.default_rng(0)
    M, N = 256, 8192
    A = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    x = rng.uniform(-1, 1, N).astype(np.float32)
    ref = A.astype(np.float64) @ x.astype(np.float64)
    err = parity_error(_wave_order_f32(A, x, 4), ref)
    assert err < GATES["f32"] / 3, err


def test_gate_accepts_fp32_accumulation_and_rejects_fp16_accumulation():
    rng = np.random.default_rng(0)
    M, N = 128, 4096
    A = (rng.standard_normal((M, N)) / np.sqrt(N)).astype(np.float16)
    x = rng.standard_normal(N).astype(np.float16)
    ref = A.astype(np.float64) @ x.astype(np.float64)
    good = _wave_order_f32(A.astype(np.float32), x.astype(np.float32), 8)
    assert parity_error(good, ref) < GATES["f16"] / 20
    bad = _running_sum_f16(A, x)
    assert parity_error(bad, ref) > GATES["f16"]


def test_gate_rejects_a_dropped_term():
    rng = np.random.default_rng(1)
    M, N = 64, 4096
    A = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    x = rng.uniform(-1, 1, N).astype(np.float32)
    ref = A.astype(np.float64) @ x.astype(np.float64)
    y = ref - A[:, 17].astype(np.float64) * x[17]
    assert parity_error(y, ref) > GATES["f32"]
