"""Fault injection into the parity gate (CPU only): a GPU result with one
corrupted element must fail the gate that bench.py aborts on, for every
format (for the lossy FP16-accumulation path, by more than its derived
bound), while the uncorrupted result passes ("membound", section
"Correctness": every kernel is checked before it is timed, and the run
aborts on failure)."""
import numpy as np
import pytest

import bench
from memory_bound_gemv_row_amd import inputs


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
def test_corrupted_element_fails_the_gate(oracle_mod, kind):
    M, N = 64, 1024
    ops = inputs.make(kind, M, N, seed=3)
    fn = {"f32": oracle_mod.gemv_f32, "f16": oracle_mod.gemv_f16, "f16x32": oracle_mod.gemv_f16x32,
          "f16_acc16": oracle_mod.gemv_f16}
    if kind in fn:
        ref = fn[kind](ops["A"], ops["x"])
    else:
        ref = (oracle_mod.gemv_q8 if kind == "q8" else oracle_mod.gemv_q4)(ops["A"], ops["scale"], ops["x"])
    good = ref.astype(np.float32)                   # what a correct kernel returns
    _, rep = bench.cpu_baseline(kind, ops, good, seconds=0.01)
    assert rep["ok"], rep
    bad = good.copy()
    if kind == "f16_acc16":
        # the lossy path's gate is its derived bound: exceed it twice over
        from oracle.metrics import acc16_bound

        abs_sum = np.abs(ops["A"].astype(np.float64)) @ np.abs(ops["x"].astype(np.float64))
        bad[17] += 2 * acc16_bound(abs_sum, N)[17]
    else:
        bad[17] += 0.05 * np.max(np.abs(ref))       # one element off by 5 % of the scale
    _, rep = bench.cpu_baseline(kind, ops, bad, seconds=0.01)
    assert not rep["ok"], rep
