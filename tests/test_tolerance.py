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


# ---------------------------------------------------------------- FP16 accumulation bound
def _fma16(a, x, s):
    """One binary16 FMA: a*x + s formed exactly (in float64 at these
    magnitudes), then rounded once to binary16."""
    return (a.astype(np.float64) * x.astype(np.float64) + s.astype(np.float64)).astype(np.float16)


def _butterfly_f32(acc):
    acc = acc.astype(np.float32)
    width = acc.shape[1]
    while width > 1:
        width //= 2
        acc = (acc[:, :width] + acc[:, width:2 * width]).astype(np.float32)
    return acc[:, 0]


def _acc16_stream_order(A, x):
    """Emulate the streaming kernel: lane l owns the 8-column chunks l, l+64,
    ... of a row and keeps two binary16 running sums (even and odd columns);
    the pair is widened and added in FP32, then a 64-lane FP32 butterfly."""
    M, N = A.shape
    assert N % 8 == 0
    pad = -N % 512                # lanes past the row end add exact zeros
    A = np.concatenate([A, np.zeros((M, pad), np.float16)], axis=1)
    x = np.concatenate([x, np.zeros(pad, np.float16)])
    P = (N + pad) // 512
    Ar = A.reshape(M, P, 64, 4, 2)
    xr = x.reshape(P, 64, 4, 2)
    acc = np.zeros((M, 64, 2), np.float16)
    for p in range(P):
        for w in range(4):
            acc = _fma16(Ar[:, p, :, w, :], xr[p, :, w, :], acc)
    lane = acc[:, :, 0].astype(np.float32) + acc[:, :, 1].astype(np.float32)
    return _butterfly_f32(lane)


def _acc16_elementwise_order(A, x):
    """Emulate the element-wise kernel: one binary16 sum per lane over the
    columns l, l+64, ... (ceil(N/64) terms)."""
    M, N = A.shape
    pad = -N % 64
    Ap = np.concatenate([A, np.zeros((M, pad), np.float16)], axis=1).reshape(M, -1, 64)
    xp = np.concatenate([x, np.zeros(pad, np.float16)]).reshape(-1, 64)
    acc = np.zeros((M, 64), np.float16)
    for p in range(Ap.shape[1]):
        acc = _fma16(Ap[:, p, :], xp[p], acc)
    return _butterfly_f32(acc)


def _abs_sum(A, x):
    return np.abs(A.astype(np.float64)) @ np.abs(x.astype(np.float64))


@pytest.mark.parametrize("dist", ["workload", "positive"])
@pytest.mark.parametrize("N", [8, 64, 200, 520, 8192])
def test_acc16_bound_holds_for_both_kernel_orders(dist, N):
    from oracle.metrics import acc16_ratio

    rng = np.random.default_rng(31 + N)
    M = 128 if N > 512 else 4096
    if dist == "workload":      # the FP16 decode workload's distribution
        A = (rng.standard_normal((M, N)) / np.sqrt(N)).astype(np.float16)
        x = rng.standard_normal(N).astype(np.float16)
    else:                       # all terms positive: the roundings cannot cancel
        A = rng.uniform(0, 1, (M, N)).astype(np.float16)
        x = rng.uniform(0, 1, N).astype(np.float16)
    ref = A.astype(np.float64) @ x.astype(np.float64)
    for order in (_acc16_stream_order, _acc16_elementwise_order):
        r = acc16_ratio(order(A, x), ref, _abs_sum(A, x), N)
        assert r <= 1.0, (order.__name__, dist, r)
    if dist == "positive" and N == 8192:
        # the bound is not vacuous: a same-direction pile-up uses about 1 % of it
        assert acc16_ratio(_acc16_elementwise_order(A, x), ref, _abs_sum(A, x), N) > 0.004


def test_acc16_bound_rejects_one_running_sum_per_row():
    # one binary16 sum over the whole row (k = N, not ceil(N/64)) stagnates
    # once the sum's spacing exceeds the terms, far outside the bound
    from oracle.metrics import acc16_ratio

    rng = np.random.default_rng(32)
    M, N = 16, 8192
    A = rng.uniform(0, 1, (M, N)).astype(np.float16)
    x = rng.uniform(0, 1, N).astype(np.float16)
    acc = np.zeros(M, np.float16)
    for j in range(N):
        acc = _fma16(A[:, j], x[j:j + 1], acc)
    ref = A.astype(np.float64) @ x.astype(np.float64)
    assert acc16_ratio(acc, ref, _abs_sum(A, x), N) > 1.0


def test_acc16_bound_closed_form():
    from oracle.metrics import acc16_bound

    # N = 8192: k = 128 binary16 terms per sum, g16 = 1/15, g32(8) = 8u/(1-8u)
    g16 = 128 * 2.0 ** -11 / (1 - 128 * 2.0 ** -11)
    g32 = 8 * 2.0 ** -24 / (1 - 8 * 2.0 ** -24)
    assert g16 == pytest.approx(1 / 15)
    want = (1 + g16) * (1 + g32) - 1 + 8192 * 2.0 ** -24
    assert acc16_bound(np.array([1.0]), 8192)[0] == pytest.approx(want, rel=1e-12)
    # the bound is finite only while k * u16 < 1
    assert np.isinf(acc16_bound(np.array([1.0]), 64 * 2048)[0])


def test_componentwise_fp32_bound_accepts_orders_and_catches_a_dropped_term():
    # the brute-force GPU test's gate: g(2N+8) * sum |w x|
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from gpu_util import within_fp32_bound

    rng = np.random.default_rng(9)
    for N in (1, 7, 126, 300):
        A = rng.uniform(-1, 1, (17, N)).astype(np.float32)
        x = rng.uniform(-1, 1, N).astype(np.float32)
        ops = {"A": A, "x": x}
        ref = A.astype(np.float64) @ x.astype(np.float64)
        # a sequential FP32 sum and a 64-lane wave order both pass
        seq = np.array([np.float32(0)] * 17)
        for j in range(N):
            seq = (seq + (A[:, j] * x[j]).astype(np.float32)).astype(np.float32)
        assert within_fp32_bound("f32", ops, seq, ref) <= 1.0
        if N > 1:
            bad = ref - A[:, N // 2].astype(np.float64) * x[N // 2]
            assert within_fp32_bound("f32", ops, bad, ref) > 1.0


def _dot2_f32(a0, b0, a1, b1, c):
    """v_dot2_f32_f16 with two roundings (the pair sum, then the addend): the
    products of binary16 operands are exact in FP32, and the instruction is
    not correctly rounded, so the pessimistic order is emulated."""
    s = (a0.astype(np.float64) * b0 + a1.astype(np.float64) * b1).astype(np.float32)
    return (s.astype(np.float64) + c).astype(np.float32)


def _q8_kernel_order(q, s, x, offset):
    """Emulate the INT8 streaming kernel: lane l owns the 16-column chunks l,
    l+64, ... of a row; each chunk enters a float32 running sum through eight
    v_dot2_f32_f16 steps, then a 64-lane butterfly and the row scale.
    offset=False: exact binary16 codes (the kernel's decode).  offset=True:
    the biased decode (q + 128) 2^-24 with 128 sum(x) removed once per row,
    a decode that cancels catastrophically for non-zero-mean x."""
    M, N = q.shape
    assert N % 1024 == 0
    xh = x.astype(np.float32)
    qc = q.reshape(M, N // 1024, 64, 16).astype(np.float32)
    xc = xh.reshape(N // 1024, 64, 16)
    if offset:
        qc = (qc + 128) * np.float32(2.0 ** -24)
    acc = np.zeros((M, 64), np.float32)
    for p in range(N // 1024):
        for k in range(8):
            acc = _dot2_f32(qc[:, p, :, 2 * k], xc[p, :, 2 * k], qc[:, p, :, 2 * k + 1], xc[p, :, 2 * k + 1], acc)
    t = _butterfly_f32(acc)
    sf = s.astype(np.float32)
    if offset:
        xsum = np.float32(np.sum(xh.astype(np.float64)))
        t = (t.astype(np.float64) * 2.0 ** 24 - 128.0 * xsum).astype(np.float32)
    return (t * sf).astype(np.float32)


@pytest.mark.parametrize("codes", ["uniform", "outlier"])
def test_q8_exact_decode_error_does_not_depend_on_the_mean_of_x(codes):
    # the INT8 reference weight is exactly q*s with FP32 accumulation
    # ("membound", dequant GEMV section): with exact codes the error stays at
    # FP32 level for zero-mean, non-negative and shifted x alike; the biased
    # decode passes zero-mean x and fails the gate on the others
    import oracle
    from memory_bound_gemv_row_amd import inputs

    M, N = 256, 8192
    if codes == "uniform":
        ops = inputs.make_q8(M, N, seed=3)
        q, s = ops["A"], ops["scale"]
    else:
        oracle.build(force=False)
        q, sb, _ = oracle.quantize_q8(inputs.make_gauss_weights(M, N, seed=3, outlier=25.0))
        s = sb.view(np.float16)
    errs = {}
    for dist in inputs.X_DISTS:
        x = inputs.make_x_f16(N, dist, seed=4)
        ref = oracle.gemv_q8(q, s, x)
        exact = parity_error(_q8_kernel_order(q, s, x, offset=False), ref)
        biased = parity_error(_q8_kernel_order(q, s, x, offset=True), ref)
        errs[dist] = (exact, biased)
        assert exact < GATES["q8"] / 5, (codes, dist, exact)
    spread = max(e for e, _ in errs.values()) / min(e for e, _ in errs.values())
    assert spread < 4, errs
    assert errs["abs_normal"][1] > GATES["q8"], errs
    assert errs["shifted"][1] > GATES["q8"], errs


# ---------------------------------------------------------------- row-slab order
def _slab_butterfly(v):
    """The row-slab reduction of one row's 64 lane sums: FP32 adds of lane
    pairs at xor distances 32 and 16 (the two lane-permute swaps), 8 (a
    rotation by 8 within 16 lanes), then 1, 2 and 4 within each group of 8."""
    v = v.astype(np.float32)
    idx = np.arange(64)
    for d in (32, 16, 8, 1, 2, 4):
        v = (v + v[:, idx ^ d]).astype(np.float32)
    return v[:, 0]


def _slab_order(kind, W, s, x, S, drop_wave=None):
    """Emulate gemv_slab: wave w of S owns passes w, w + S, ...; lane l of
    that wave sums its chunk of each pass in FP32 (INT8/INT4 products exact,
    each v_dot2_f32_f16 step with two roundings; FP16 weights with FP32 x one
    rounding per v_fma_mix_f32 step); the wave's 64 lane sums meet in the
    slab butterfly, the S wave sums are added in wave order, and INT8 takes
    its row scale last.  W holds exact weight values (codes for INT8/INT4).
    drop_wave leaves one wave's sum out (a planted mistake)."""
    M, N = W.shape
    E = {"q8": 16, "q4": 32, "f16x32": 8}[kind]
    P = N // (64 * E)
    assert N == P * 64 * E and P % S == 0
    Wc = W.reshape(M, P, 64, E).astype(np.float64)
    xc = x.astype(np.float64).reshape(P, 64, E)
    waves = []
    for w in range(S):
        acc = np.zeros((M, 64), np.float32)
        for p in range(w, P, S):
            if kind == "f16x32":
                for k in range(E):
                    acc = (acc.astype(np.float64) + Wc[:, p, :, k] * xc[p, :, k]).astype(np.float32)
            elif kind == "q8":
                for k in range(0, E, 2):
                    acc = _dot2_f32(Wc[:, p, :, k], xc[p, :, k], Wc[:, p, :, k + 1], xc[p, :, k + 1], acc)
            else:
                part = np.zeros((M, 64), np.float32)
                for word in range(4):
                    for j in range(4):   # pairs (x_j, x_{j+4}) of the word's 8 columns
                        c0, c1 = 8 * word + j, 8 * word + j + 4
                        part = _dot2_f32(Wc[:, p, :, c0], xc[p, :, c0], Wc[:, p, :, c1], xc[p, :, c1], part)
                # a lane's 32 columns lie in one 128-column group: (p * 64 + l) // 4
                sg = s.astype(np.float64)[:, (p * 64 + np.arange(64)) // 4]
                acc = (acc.astype(np.float64) + sg * part.astype(np.float64)).astype(np.float32)
        if w != drop_wave:
            waves.append(_slab_butterfly(acc))
    t = waves[0]
    for v in waves[1:]:
        t = (t + v).astype(np.float32)
    if kind == "q8":
        t = (t.astype(np.float64) * s.astype(np.float64)).astype(np.float32)
    return t


@pytest.mark.parametrize("kind,N,S", [("q8", 24576, 12), ("q4", 14336, 7), ("f16x32", 8192, 16)])
def test_slab_order_within_the_gate(kind, N, S):
    # The row-slab kernel's order (passes split over the waves, the batched
    # butterfly, wave sums added in LDS) on the workloads' value
    # distributions and, for INT8/INT4, non-zero-mean activations: its
    # floored error stays far inside the gate, as the streaming kernel's
    # does; leaving one wave's sum out fails it
    import oracle
    from memory_bound_gemv_row_amd import inputs
    from qpack import unpack_int4

    oracle.build(force=False)
    M = 48
    ops = inputs.make(kind, M, N, seed=7)
    for dist in (inputs.X_DISTS if kind != "f16x32" else ("normal",)):
        x = ops["x"] if kind == "f16x32" else inputs.make_x_f16(N, dist, seed=8)
        if kind == "q8":
            W, s = ops["A"], ops["scale"]
            ref = oracle.gemv_q8(ops["A"], s, x)
        elif kind == "q4":
            W, s = unpack_int4(ops["A"]), ops["scale"]
            ref = oracle.gemv_q4(ops["A"], s, x)
        else:
            W, s = ops["A"], None
            ref = oracle.gemv_f16x32(ops["A"], x)
        err = parity_error(_slab_order(kind, W, s, x, S), ref)
        assert err < GATES[kind] / 5, (kind, dist, err)
        assert parity_error(_slab_order(kind, W, s, x, S, drop_wave=S // 2), ref) > GATES[kind], (kind, dist)
