"""GPU parity of split rows: few long rows, a workgroup of S waves per row
whose wave sums meet in LDS (the survey's cross-wave reduction step, for a
row that spans waves; "cuda-gemv-optimization", the shared-memory kernel,
and the llama.cpp walkthrough's block-per-row kernel combine one row's
partial sums the same way).

Every format the split kernel serves, every waves-per-row value (2, 4, 8,
16), both in-flight depths, rows whose units do not divide among the waves,
ragged last passes (lanes past the row end), a single row, against the CPU
oracle at each path's gate and against the FP32 summation bound.
"""
import numpy as np
import pytest
import torch

from memory_bound_gemv_row_amd import binding, inputs

from gpu_util import run_gpu, run_oracle, say, within_fp32_bound, within_gate

pytestmark = pytest.mark.gpu

_ELEMS = {"f32": 4, "f16": 8, "f16x32": 8, "q8": 16, "q4": 32}


def _n(kind, units, ragged):
    """A row length of `units` 1-KiB wave loads; `ragged` leaves the last
    pass partly filled (INT4 keeps whole 128-column groups)."""
    n = units * 64 * _ELEMS[kind]
    if ragged:
        n -= 128 if kind == "q4" else 3 * _ELEMS[kind]
    return n


# (M, units per row, ragged): waves per row S from 2 to 16 on 256 CUs, two
# units per wave (2 in flight) and more (4 in flight, padded)
_CASES = [(1, 40, True), (3, 33, False), (17, 20, True), (300, 9, True), (300, 4, False), (700, 16, True),
          (700, 5, False), (1100, 30, True), (17, 12, False), (200, 10, True), (100, 4, True)]


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "q8", "q4"])
def test_split_rows_match_the_oracle(gpu, oracle_mod, kind):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    seen = set()
    for M, units, ragged in _CASES:
        if kind == "q4" and units > 16:
            continue        # INT4 splits only rows of at most 16 units
        N = _n(kind, units, ragged)
        info = binding.describe_launch(kind, M, N)
        if info["variant"] == 6:
            seen.add((info["block"] // 64, info["units_in_flight"]))
        ops = inputs.make(kind, M, N, seed=M * 31 + N)
        label = f"{kind} split M={M} N={N} {info}"
        say(f"[split] {label}")
        y = run_gpu(kind, ops)
        ref = run_oracle(oracle_mod, kind, ops)
        rep = within_gate(oracle_mod, kind, ops, y, ref)
        assert rep["ok"], (label, rep)
        assert within_fp32_bound(kind, ops, y, ref) <= 1.0, label
    if cus == 256:
        # the cases reach every waves-per-row value and both depths (INT4,
        # split only for rows of at most 16 units and fewer rows than CUs,
        # up to 4 waves per row; INT8 splits with 2 in flight; FP16 with
        # FP32 x splits only fewer rows than CUs, 4 in flight: from one row
        # per CU its rows take row slabs, and its 2-deep split runs as an
        # explicit plan in test_gpu_plans)
        want = {2, 4} if kind == "q4" else {2, 4, 8, 16}
        depths = {2} if kind == "q8" else ({4} if kind == "f16x32" else {2, 4})
        assert {s for s, _ in seen} == want and {d for _, d in seen} == depths, seen


@pytest.mark.parametrize("kind", ["f16", "q8", "q4"])
def test_split_rows_integer_inputs_bit_exact(gpu, oracle_mod, kind):
    # integer-valued operands make every FP32 summation order exact, so the
    # S-way split must reproduce the oracle bit for bit
    rng = np.random.default_rng(5)
    M, N = 37, _n(kind, 12, True)
    if kind == "f16":
        ops = {"A": rng.integers(-3, 4, (M, N)).astype(np.float16), "x": rng.integers(-3, 4, N).astype(np.float16)}
    elif kind == "q8":
        ops = {"A": rng.integers(-128, 128, (M, N), dtype=np.int8), "scale": np.full(M, 2.0 ** -7, np.float16),
               "x": rng.integers(-3, 4, N).astype(np.float16)}
    else:
        ops = {"A": rng.integers(0, 256, (M, N // 2), dtype=np.uint8),
               "scale": (2.0 ** (np.arange(N // 128) % 8 - 4)).astype(np.float16)[None, :].repeat(M, 0),
               "x": rng.integers(-3, 4, N).astype(np.float16)}
    info = binding.describe_launch(kind, M, N)
    assert info["variant"] == 6, info
    say(f"[split exact] {kind} M={M} N={N} {info}")
    y = run_gpu(kind, ops)
    ref = run_oracle(oracle_mod, kind, ops)
    assert np.array_equal(y.astype(np.float64), ref), (kind, np.max(np.abs(y - ref)))


# Plans the FP32/FP16 cost model picks over the measured rules on MI355X:
# (kind, M, N, (variant, block, units in flight, rows per wave)) -- split
# rows at thousands of rows, two rows per wave with 2 in flight, and 4-wave
# workgroups with 8 in flight for a few long rows
_MODEL_CASES = [("f16", 4351, 9856, (6, 128, 2, 1)), ("f16", 2552, 9088, (6, 128, 2, 1)),
                ("f16", 278, 16896, (6, 256, 4, 1)), ("f32", 902, 5248, (6, 128, 4, 1)),
                ("f16", 16384, 2560, (2, 256, 2, 2)), ("f32", 11646, 1664, (2, 256, 2, 2))]


@pytest.mark.parametrize("case", _MODEL_CASES, ids=lambda c: f"{c[0]}_{c[1]}x{c[2]}")
def test_cost_model_plans_match_the_oracle(gpu, oracle_mod, case):
    kind, M, N, want = case
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    info = binding.describe_launch(kind, M, N)
    if cus == 256:
        got = (info["variant"], info["block"], info["units_in_flight"], info["rows_per_wave"])
        assert got == want, (kind, M, N, info)
    ops = inputs.make(kind, M, N, seed=M + 7 * N)
    label = f"{kind} model plan M={M} N={N} {info}"
    say(f"[model] {label}")
    y = run_gpu(kind, ops)
    ref = run_oracle(oracle_mod, kind, ops)
    rep = within_gate(oracle_mod, kind, ops, y, ref)
    assert rep["ok"], (label, rep)
    assert within_fp32_bound(kind, ops, y, ref) <= 1.0, label
