"""The bench's byte model and rate arithmetic against numbers the pages print.

The "membound" page publishes times together with the GB/s, MBU and
speed-up columns derived from them; recomputing those columns from the
printed times with our byte model must land on the printed values (within
the rounding of the printed times).  This pins the byte model, including
that x is counted and that the quantised formats' binary16 scales are
counted as streamed bytes.
"""
import json
import os

import pytest

from memory_bound_gemv_row_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HALF_ULP_MS = 0.00005     # the pages print times to 4 decimals


def _range(nbytes, ms):
    return (nbytes / ((ms + HALF_ULP_MS) * 1e-3) / 1e9, nbytes / ((ms - HALF_ULP_MS) * 1e-3) / 1e9)


def test_fp16_table_gbps_and_mbu():
    t = json.load(open(os.path.join(GOLDEN, "membound_fp16_table.json")))
    den = t["mbu_denominator_gbps"]
    for r in t["rows"]:
        lo, hi = _range(acc.alg_bytes("f16", r["M"], r["N"]), r["ms"])
        assert lo - 0.05 <= r["gbps"] <= hi + 0.05, r
        assert lo / den * 100 - 0.05 <= r["mbu"] <= hi / den * 100 + 0.05, r
    # the page's headline: the best achieved rate is the denominator
    assert max(r["gbps"] for r in t["rows"]) == den


def test_dequant_table_counts_scales():
    t = json.load(open(os.path.join(GOLDEN, "membound_dequant_table.json")))
    implied = []
    for r in t["rows"]:
        for key, kind in (("fp16", "f16"), ("q8", "q8"), ("q4", "q4")):
            lo, hi = _range(acc.alg_bytes(kind, r["M"], r["N"]), r[key + "_ms"])
            mbu = r[key + "_mbu"] / 100
            implied.append(((lo / (mbu + 0.0005)), hi / (mbu - 0.0005)))
    # one run, one ceiling: every row must be consistent with a single denominator
    lo = max(a for a, _ in implied)
    hi = min(b for _, b in implied)
    assert lo <= hi and 419.0 < lo and hi < 421.5
    # dropping the INT4 scales from the byte count breaks that consistency
    r = t["rows"][1]
    no_scale = (r["M"] * r["N"]) // 2 + 2 * r["N"] + 4 * r["M"]
    assert no_scale / (r["q4_ms"] * 1e-3) / 1e9 / (r["q4_mbu"] / 100) < 410


def test_dequant_speedups_are_time_ratios():
    t = json.load(open(os.path.join(GOLDEN, "membound_dequant_table.json")))
    for r in t["rows"]:
        for key in ("q8", "q4"):
            lo = acc.ratio(r["fp16_ms"] - HALF_ULP_MS, r[key + "_ms"] + HALF_ULP_MS)
            hi = acc.ratio(r["fp16_ms"] + HALF_ULP_MS, r[key + "_ms"] - HALF_ULP_MS)
            assert lo - 0.005 <= r[key + "_x"] <= hi + 0.005, (r, key)


def test_int4_cap():
    t = json.load(open(os.path.join(GOLDEN, "membound_dequant_table.json")))
    per_elem = acc.weight_bytes("q4", 128, 128) / (128 * 128)
    assert per_elem == 0.515625 and round(per_elem, 3) == t["int4_bytes_per_elem_printed"]
    for M, N in ((8192, 8192), (4096, 14336), (14336, 4096)):
        cap = acc.alg_bytes("f16", M, N) / acc.alg_bytes("q4", M, N)
        assert round(cap, 2) == t["int4_cap_printed"]


def test_arithmetic_intensity_limit():
    # "Making GEMV Fast", section "Arithmetic intensity": AI -> 1/2 FLOP per byte for large M, N
    assert abs(acc.arithmetic_intensity("f32", 1 << 16, 1 << 16) - 0.5) < 1e-4
    assert acc.arithmetic_intensity("f32", 1, 1) == 1 / 12


@pytest.mark.parametrize("kind,M,N,copies", [("f16", 8192, 8192, 8), ("q4", 4096, 14336, 36), ("f32", 1024, 1024, 256)])
def test_ring_covers_a_gibibyte(kind, M, N, copies):
    assert acc.ring_copies(kind, M, N) == copies
    assert acc.ring_copies(kind, M, N) * acc.weight_bytes(kind, M, N) >= 1 << 30
