"""Pins for the quantiser oracle (CPU only), each against something other
than the oracle itself: numpy's binary16 rounding, the RMSE the "membound"
page prints (golden fixture), the closed-form RMSE of absmax scaling on
uniform weights, exactly representable weights, ties, the half-step error
bound, and the clipping and degenerate cases."""
import json
import math
import os

import numpy as np
import pytest

from qpack import unpack_int4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sig(v, digits):
    return float(f"{v:.{digits - 1}e}")


# ---------------------------------------------------------------- binary16 rounding
def test_double_to_half_matches_numpy(oracle_mod):
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.uniform(-1, 1, 2000) * 2.0 ** rng.integers(-30, 17, 2000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
         2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -11), 2047.5, 2048.0 + 1.0],
    ])
    for v in vals:
        with np.errstate(over="ignore"):
            want = int(np.array(v, dtype=np.float64).astype(np.float16).view(np.uint16))
        assert oracle_mod.double_to_half(v) == want, (v, hex(want))


# ---------------------------------------------------------------- the page's RMSE
def test_rmse_matches_the_page(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "membound_quant_rmse.json")))
    rng = np.random.default_rng(0)
    W = rng.uniform(-1, 1, (4096, 4096)).astype(np.float32)
    _, _, e8 = oracle_mod.quantize_q8(W)
    _, _, e4 = oracle_mod.quantize_q4(W)
    d = g["printed_significant_digits"]
    assert _sig(oracle_mod.quant_rmse(e8, *W.shape), d) == g["q8_rmse_printed"]
    assert _sig(oracle_mod.quant_rmse(e4, *W.shape), d) == g["q4_rmse_printed"]


def test_rmse_closed_form_uniform(oracle_mod):
    # absmax scaling on U[-1, 1]: the code error is uniform on [-s/2, s/2]
    # (variance s^2/12) except at the absmax element itself (error 0), with
    # s = max|w| / qmax and E[max^2] = n / (n + 2) for the max of n U(0, 1).
    rng = np.random.default_rng(1)
    M, N = 512, 8192
    W = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    for quant, qmax, n in ((oracle_mod.quantize_q8, 127, N), (oracle_mod.quantize_q4, 7, 128)):
        _, _, e = quant(W)
        want = math.sqrt((n - 1) / n * (n / (n + 2)) / qmax ** 2 / 12)
        got = oracle_mod.quant_rmse(e, M, N)
        assert abs(got - want) / want < 3e-3, (qmax, got, want)


# ---------------------------------------------------------------- exact cases
def test_representable_weights_are_exact(oracle_mod):
    rng = np.random.default_rng(2)
    M, N = 6, 512
    k8 = rng.integers(-127, 128, (M, N))
    k8[:, 5] = 127                                  # absmax 127 * 2^-7 -> scale 2^-7
    q, s, e = oracle_mod.quantize_q8((k8 * 2.0 ** -7).astype(np.float32))
    assert np.array_equal(q, k8) and np.all(s == 0x2000) and np.all(e == 0)   # 0x2000 = 2^-7
    k4 = rng.integers(-7, 8, (M, N))
    k4[:, ::128] = -7                               # every group holds -7: scale 2^-3
    q4, s4, e4 = oracle_mod.quantize_q4((k4 * 2.0 ** -3).astype(np.float32))
    assert np.array_equal(unpack_int4(q4), k4) and np.all(s4 == 0x3000) and np.all(e4 == 0)


def test_ties_round_to_even(oracle_mod):
    W = np.zeros((1, 16), np.float32)
    W[0, :8] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]    # scale exactly 1.0
    q, s, _ = oracle_mod.quantize_q8(W)
    assert s[0] == 0x3C00
    assert list(q[0, :8]) == [127, 2, 4, -2, -4, 0, 2, 0]
    W4 = np.zeros((1, 128), np.float32)
    W4[0, :6] = [7.0, 2.5, 3.5, -2.5, -0.5, 6.5]                # scale exactly 1.0
    q4, s4, _ = oracle_mod.quantize_q4(W4)
    assert s4[0, 0] == 0x3C00
    assert list(unpack_int4(q4)[0, :6]) == [7, 2, 4, -2, 0, 6]


def test_error_within_half_step_and_absmax_maps_to_qmax(oracle_mod):
    # also pins the INT4 nibble order and group index: a swapped nibble or a
    # wrong group scale breaks the half-step bound
    rng = np.random.default_rng(3)
    M, N = 40, 1024
    W = (rng.standard_normal((M, N)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32)
    q, s, _ = oracle_mod.quantize_q8(W)
    sd = s.view(np.float16).astype(np.float64)
    err = np.abs(q.astype(np.float64) * sd[:, None] - W)
    assert np.all(err <= 0.5 * sd[:, None] * (1 + 1e-6))
    assert np.all(np.abs(q[np.arange(M), np.argmax(np.abs(W), axis=1)]) == 127)
    q4, s4, _ = oracle_mod.quantize_q4(W)
    sd4 = np.repeat(s4.view(np.float16).astype(np.float64), 128, axis=1)
    deq = unpack_int4(q4) * sd4
    assert np.all(np.abs(deq - W) <= 0.5 * sd4 * (1 + 1e-6))
    Wg = np.abs(W).reshape(M, N // 128, 128)
    idx = np.argmax(Wg, axis=2)
    codes = unpack_int4(q4).reshape(M, N // 128, 128)
    assert np.all(np.abs(np.take_along_axis(codes, idx[..., None], axis=2)) == 7)


def test_row_sse_is_the_squared_error(oracle_mod):
    rng = np.random.default_rng(4)
    W = rng.uniform(-1, 1, (8, 640)).astype(np.float32)
    q, s, e = oracle_mod.quantize_q8(W)
    d = q.astype(np.float64) * s.view(np.float16).astype(np.float64)[:, None] - W
    assert np.allclose(e, np.sum(d * d, axis=1), rtol=1e-12)


# ---------------------------------------------------------------- degenerate cases
def test_zero_rows_and_groups(oracle_mod):
    W = np.zeros((3, 256), np.float32)
    W[1, 200] = 0.75
    q, s, e = oracle_mod.quantize_q8(W)
    assert s[0] == 0 and np.all(q[0] == 0) and e[0] == 0
    q4, s4, e4 = oracle_mod.quantize_q4(W)
    assert np.all(s4[0] == 0) and s4[1, 0] == 0 and s4[1, 1] != 0
    assert np.all(unpack_int4(q4)[1, :128] == 0) and unpack_int4(q4)[1, 200] == 7


def test_scale_saturates_and_codes_clip(oracle_mod):
    # a scale beyond binary16's range is clamped to 65504; codes then clip
    W = np.array([[1.0e7, -1.0e7, 65504.0 * 127, 1.0]], np.float32)
    q, s, _ = oracle_mod.quantize_q8(W)
    assert s[0] == 0x7BFF
    assert list(q[0]) == [127, -127, 127, 0]
    # a scale in binary16's subnormal range is coarse; codes clip at +-7
    W4 = np.zeros((1, 128), np.float32)
    W4[0, 0], W4[0, 1] = 3.0e-7, -3.0e-7        # 3e-7 / 7 rounds to 2^-24
    q4, s4, _ = oracle_mod.quantize_q4(W4)
    assert s4[0, 0] == 0x0001
    assert list(unpack_int4(q4)[0, :2]) == [5, -5]
    # a scale that rounds to zero gives all-zero codes
    W5 = np.zeros((1, 128), np.float32)
    W5[0, 0] = 1.0e-8
    q5, s5, e5 = oracle_mod.quantize_q4(W5)
    assert s5[0, 0] == 0 and np.all(q5 == 0) and e5[0] == pytest.approx(1.0e-16, rel=1e-6)


def test_q4_rejects_partial_groups(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.quantize_q4(np.zeros((2, 100), np.float32))
