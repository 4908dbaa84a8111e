"""Pins for the softmax oracle (CPU only), each against something other than
the oracle itself: scipy's softmax, closed forms, the online recurrence the
"membound" page uses (section "Bonus kernel: online softmax"), shift
invariance, masking, and the error metric's floor."""
import math

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

from qpack import f16


def test_against_scipy(oracle_mod):
    rng = np.random.default_rng(0)
    x = f16(rng.standard_normal((64, 3000)) * 3)
    y = oracle_mod.softmax_f16(x)
    ref = scipy_softmax(x.astype(np.float64), axis=1)
    assert np.max(np.abs(y - ref) / ref) < 1e-13


def test_constant_row_is_uniform(oracle_mod):
    for N in (1, 7, 4096):
        y = oracle_mod.softmax_f16(np.full((3, N), 1.5, np.float16))
        assert np.all(y == 1.0 / N)


def test_two_columns_are_the_logistic(oracle_mod):
    rng = np.random.default_rng(1)
    x = f16(rng.uniform(-8, 8, (200, 2)))
    y = oracle_mod.softmax_f16(x)
    a, b = x[:, 0].astype(np.float64), x[:, 1].astype(np.float64)
    want = np.array([1.0 / (1.0 + math.exp(bb - aa)) for aa, bb in zip(a, b)])
    assert np.allclose(y[:, 0], want, rtol=1e-14, atol=0)
    assert np.allclose(y[:, 0] + y[:, 1], 1.0, rtol=1e-15, atol=0)


def _online(row):
    """The page's single-sweep update: m' = max(m, x), d = d e^(m - m') + e^(x - m')."""
    m, d = -math.inf, 0.0
    for v in row:
        m2 = max(m, v)
        d = (d * math.exp(m - m2) if m != -math.inf else 0.0) + math.exp(v - m2)
        m = m2
    return [math.exp(v - m) / d for v in row]


@pytest.mark.parametrize("N", [1, 2, 5, 64, 300])
def test_matches_the_online_recurrence(oracle_mod, N):
    rng = np.random.default_rng(N)
    x = f16(rng.standard_normal((4, N)) * 4)
    y = oracle_mod.softmax_f16(x)
    for i in range(4):
        want = _online([float(v) for v in x[i]])
        assert np.allclose(y[i], want, rtol=1e-13, atol=0)


def test_shift_invariance_exact(oracle_mod):
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 9, (10, 500)).astype(np.float16)
    y0 = oracle_mod.softmax_f16(x)
    y1 = oracle_mod.softmax_f16((x.astype(np.float64) + 1024).astype(np.float16))   # exact in binary16
    assert np.array_equal(y0, y1)


def test_rows_sum_to_one(oracle_mod):
    rng = np.random.default_rng(3)
    x = f16(rng.standard_normal((32, 8192)))
    y = oracle_mod.softmax_f16(x)
    assert np.all(np.abs(y.sum(axis=1) - 1.0) < 8192 * 2.0 ** -52)


def test_masked_entries(oracle_mod):
    rng = np.random.default_rng(4)
    x = f16(rng.standard_normal((5, 64)))
    xm = x.copy()
    xm[:, 10:20] = -np.inf
    y = oracle_mod.softmax_f16(xm)
    assert np.all(y[:, 10:20] == 0)
    keep = np.r_[0:10, 20:64]
    assert np.allclose(y[:, keep], oracle_mod.softmax_f16(x[:, keep]), rtol=1e-15, atol=0)


def test_special_rows_give_nan(oracle_mod):
    x = np.zeros((3, 8), np.float16)
    x[0, :] = -np.inf
    x[1, 3] = np.inf
    x[2, 5] = np.nan
    y = oracle_mod.softmax_f16(x)
    assert np.all(np.isnan(y))


def test_empty(oracle_mod):
    assert oracle_mod.softmax_f16(np.zeros((0, 5), np.float16)).shape == (0, 5)
    assert oracle_mod.softmax_f16(np.zeros((3, 0), np.float16)).shape == (3, 0)


def test_metric_floor_and_gate():
    from oracle.metrics import SOFTMAX_GATE, softmax_error

    r = np.array([0.5, 1e-6, 0.0])
    # an error of 1e-7 at a 1e-6 output is measured against the 1e-4 floor
    assert softmax_error(r + [0, 1e-7, 0], r) == pytest.approx(1e-3)
    # rounding the exact result to binary16 passes the gate everywhere
    rng = np.random.default_rng(5)
    ref = scipy_softmax(rng.standard_normal((16, 4096)) * 3, axis=1)
    assert softmax_error(ref.astype(np.float16).astype(np.float64), ref) < SOFTMAX_GATE / 3
    # while dropping one term of the normaliser does not
    bad = ref.copy()
    bad[0] = ref[0] / (1 - ref[0].max())
    assert softmax_error(bad, ref) > SOFTMAX_GATE
    assert softmax_error(np.array([np.nan]), np.array([np.nan])) == 0.0
    assert softmax_error(np.array([np.nan]), np.array([1.0])) == float("inf")


def test_large_logits_do_not_overflow(oracle_mod):
    # exp(60000) overflows double; the result depends only on differences
    x = np.array([[60000.0, 59968.0, 59936.0, -60000.0]], np.float16)
    y = oracle_mod.softmax_f16(x)
    want = scipy_softmax(np.array([0.0, -32.0, -64.0, -120000.0]))
    assert np.allclose(y[0], want, rtol=1e-14, atol=0)
