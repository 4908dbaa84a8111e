"""Launch geometry rules, checked on the host through
gemv_describe_launch_for (the library's planner for a device of given CU
count and LDS per workgroup; no GPU needed)."""
import itertools

import pytest

from memory_bound_gemv_row_amd import binding
from memory_bound_gemv_row_amd.binding import GemvError

MI355X = dict(cus=256, lds_max=160 * 1024)
ELEMS_PER_CHUNK = {"f32": 4, "f16": 8, "f16_acc16": 8, "f16x32": 8, "q8": 16, "q4": 32}
X_GRANULES = {"f32": 1, "f16": 1, "f16_acc16": 1, "f16x32": 2, "q8": 2, "q4": 4}   # 16-byte granules of x per chunk
KINDS = list(ELEMS_PER_CHUNK)


def plan(kind, M, N, cus=256, lds_max=160 * 1024, aligned=True):
    return binding.describe_launch_for(kind, M, N, cus, lds_max, aligned)


def staged_bytes(kind, N):
    nchunks = N // ELEMS_PER_CHUNK[kind]
    return (nchunks + 63) // 64 * 64 * X_GRANULES[kind] * 16


def _four_rows(kind, M, N, cus):
    # FP rows of 24 units and more at 11-16 rows per CU: four rows per wave,
    # one 4-wave workgroup per CU at most (some CUs idle below 16 rows per
    # CU: measured faster than filling them)
    P = -(-(N // ELEMS_PER_CHUNK[kind]) // 64) if N else 0
    return kind in ("f32", "f16", "f16_acc16") and P >= 24 and P % 16 and 11 * cus < M <= 16 * cus


def _fewer_stagings(kind, M, p, cus):
    # FP16 with FP32 x, 8-14 rows per CU: two rows per wave staged, fewer
    # workgroups than CUs (fewer stagings of x measured faster)
    return kind == "f16x32" and p["variant"] == 1 and p["rows_per_wave"] >= 2 and M <= 14 * cus


_MS = [1, 7, 64, 255, 1000, 1024, 1025, 2048, 4096, 8192, 14336, 40000, 300000, (1 << 24) + 3]
_NS = [0, 3, 8, 16, 128, 256, 512, 1000, 1024, 1536, 2048, 4096, 8192, 14336, 16384, 20480, 32768, 34816, 49152,
       65536, 81920, 98304]
_DEVICES = [MI355X, dict(cus=304, lds_max=64 * 1024), dict(cus=80, lds_max=64 * 1024)]


@pytest.mark.parametrize("dev", _DEVICES, ids=lambda d: f"{d['cus']}cu_{d['lds_max'] // 1024}k")
@pytest.mark.parametrize("kind", KINDS)
def test_every_plan_is_consistent(kind, dev):
    for M, N in itertools.product(_MS, _NS):
        if kind == "q4" and N % 128:
            continue
        p = plan(kind, M, N, **dev)
        where = (kind, M, N, dev, p)
        assert p["variant"] in (1, 2, 3, 4, 5, 6, 7), where
        assert 1 <= p["grid"] and p["block"] % 64 == 0 and 64 <= p["block"] <= 1024, where
        assert p["block"] in (256, 512, 768) or p["variant"] in (6, 7), where
        assert p["grid"] * p["block"] <= 1 << 30, where            # 32-bit work-item count
        aligned_path = N > 0 and N % ELEMS_PER_CHUNK[kind] == 0
        if not aligned_path:
            assert p["variant"] == 3, where
        if p["variant"] == 4:                                       # packed short rows
            assert kind in ("q8", "q4") and N // ELEMS_PER_CHUNK[kind] <= 32, where
        elif p["variant"] in (1, 2, 3, 5):
            # every row has a wave: grid x waves x rows per wave covers M
            assert p["grid"] * (p["block"] // 64) * p["rows_per_wave"] >= M, where
        if p["variant"] == 1:
            assert kind in ("q8", "q4", "f16x32"), where           # FP32/FP16 read x with each unit
            # split staging (order 2) keeps one spare 16-byte granule per lane after x
            spare = 64 * 16 if p["stage_order"] == 2 else 0
            assert p["lds_bytes"] == staged_bytes(kind, N) + spare <= dev["lds_max"], where
            assert p["stage_order"] in (0, 1, 2), where
        else:
            assert p["lds_bytes"] == 0 and p["stage_order"] == -1, where
        if (p["variant"] in (1, 2) and M >= 8 * dev["cus"] and not _fewer_stagings(kind, M, p, dev["cus"])
                and not _four_rows(kind, M, N, dev["cus"])):
            assert p["grid"] >= dev["cus"], where                 # every CU gets a workgroup
        if p["variant"] == 5:
            assert 1 <= -(-(N // ELEMS_PER_CHUNK[kind]) // 64) <= 3, where   # rows of one to three units
        if p["variant"] == 6:
            # split rows: one workgroup of S waves per row (the grid holds
            # every row: the kernel does not walk), S a power of two from 2
            # to 16 with at least two units per wave, 2 or 4 in flight
            S = p["block"] // 64
            P = -(-(N // ELEMS_PER_CHUNK[kind]) // 64)
            assert kind != "f16_acc16" and aligned_path, where
            assert S in (2, 4, 8, 16) and 2 * S <= P and p["grid"] == M and p["rows_per_wave"] == 1, where
            assert M * p["block"] <= 1 << 30 and p["units_in_flight"] in (2, 4), where
            if kind == "q8":
                # INT8: up to 6 rows per CU, 2 in flight
                assert M <= 6 * dev["cus"] and p["units_in_flight"] == 2, where
            elif kind == "f16x32":
                # FP16 with FP32 x: up to 7 rows per CU, two waves per row
                # from one row per CU, 4 in flight below 3 rows per CU, else
                # 2
                assert M <= 7 * dev["cus"] and (S == 2 or M < dev["cus"]), where
                assert p["units_in_flight"] == (4 if M < 3 * dev["cus"] else 2), where
            elif kind not in ("f32", "f16"):
                # the rule alone: only where one wave per row leaves the CUs
                # short of waves (fewer than 8 per CU), 2 in flight for two
                # units per wave
                assert M <= 16 * dev["cus"], where
                assert p["units_in_flight"] == (2 if -(-P // S) == 2 else 4), where
        if p["variant"] == 7:
            _check_slab(kind, M, N, dev, p, where)
        assert 1 <= p["units_in_flight"] <= 8, where


def _check_slab(kind, M, N, dev, p, where):
    # row slabs: S waves per workgroup own one or two passes each of every
    # row (S = P, or P / 2 for rows of 17-32 units), slabs of 4 or 8 rows,
    # 4 in flight (8 with two passes per wave); the grid's slabs cover M
    cus = dev["cus"]
    S = p["block"] // 64
    P = -(-(N // ELEMS_PER_CHUNK[kind]) // 64)
    assert kind in ("q8", "q4", "f16x32") and N % ELEMS_PER_CHUNK[kind] == 0, where
    two = P > 16 or (kind == "q8" and P >= 10 and P % 2 == 0)   # two passes per wave
    assert S == (P // 2 if two else P) and P % S == 0 and P <= 32, where
    assert p["units_in_flight"] == (8 if two else 4), where
    assert p["rows_per_wave"] % 4 == 0 and p["grid"] * p["rows_per_wave"] >= M, where
    assert p["lds_bytes"] == 0 and p["stage_order"] == -1, where
    if kind == "f16x32":
        assert M >= cus and (P >= 2 or M >= 14 * cus), where
    elif kind == "q4":
        nchunks = N // ELEMS_PER_CHUNK[kind]
        assert ((M >= cus and 3 <= P <= 16 and P != 6 and (P <= 7 or M <= 12 * cus))
                or (P == 1 and nchunks > 32 and M >= 4 * cus)), where
        assert p["grid"] <= max(1, 32 // S) * cus, where        # at most 32 waves per CU
    else:
        assert P >= 9 and 2 * cus <= M <= 12 * cus, where


def test_random_shapes_keep_the_invariants():
    # seeded random row counts and lengths (log-uniform) on random devices
    import numpy as np

    rng = np.random.default_rng(2026)
    for _ in range(3000):
        kind = KINDS[rng.integers(len(KINDS))]
        M = int(np.exp(rng.uniform(0, np.log(1 << 30))))
        N = int(np.exp(rng.uniform(0, np.log(1 << 20))))
        if kind == "q4":
            N = max(128, N // 128 * 128)
        dev = dict(cus=int(rng.choice([80, 104, 228, 256, 304])), lds_max=int(rng.choice([64, 160]) * 1024))
        p = plan(kind, M, N, **dev)
        where = (kind, M, N, dev, p)
        assert 1 <= p["grid"] and p["grid"] * p["block"] <= 1 << 30, where
        assert p["lds_bytes"] <= dev["lds_max"], where
        if p["variant"] == 7:
            _check_slab(kind, M, N, dev, p, where)
        elif p["variant"] != 4:
            assert p["grid"] * (p["block"] // 64) * p["rows_per_wave"] >= M, where
        if (p["variant"] in (1, 2) and M >= 8 * dev["cus"] and not _fewer_stagings(kind, M, p, dev["cus"])
                and not _four_rows(kind, M, N, dev["cus"])):
            assert p["grid"] >= dev["cus"], where


def test_fp_rows_pick_the_least_padding():
    # FP16 rows of 4-23 units with rows enough to fill every CU at two rows
    # per wave: each wave's unit sequence (rows x P) is padded to a multiple
    # of the loads in flight by no more than the best of the rules' four
    # choices (the cost model may take 2 in flight where that pads nothing)
    for P in range(4, 24):
        p = plan("f16", 16384, P * 512)
        assert p["variant"] == 2, (P, p)
        D, r = p["units_in_flight"], p["rows_per_wave"]
        pad = lambda d, rr: (-(rr * P) % d) / (rr * P)
        assert pad(D, r) <= min(pad(d, rr) for d in (4, 8) for rr in (1, 2)), (P, p)
    # too few rows to fill the CUs at two rows per wave: one row per wave
    assert plan("f16", 1000, 6144)["rows_per_wave"] == 1


def test_unaligned_operands_take_the_elementwise_kernel():
    for kind in KINDS:
        assert plan(kind, 4096, 4096, aligned=False)["variant"] == 3


def test_huge_shapes_take_the_elementwise_kernel():
    for kind in ("f16", "q8", "q4"):
        assert plan(kind, (1 << 30) + 1, 128)["variant"] == 3
        assert plan(kind, 1 << 30, 128)["variant"] != 3
    # rows of 2 GiB or more: 64-bit offsets
    assert plan("f16", 2, 1 << 30)["variant"] == 3
    assert plan("f16", 2, (1 << 30) - 8)["variant"] != 3
    assert plan("f32", 2, 1 << 29)["variant"] == 3


def test_headline_shapes_on_mi355x():
    # FP16 and FP32 read x with each unit; INT8 and INT4 14336x4096 stage it;
    # INT4 4096x14336 and FP16 with FP32 x take row slabs (x slices in
    # registers); all fill every CU
    for kind, M, N, variant in (("f16", 8192, 8192, 2), ("f16", 4096, 14336, 2), ("f16", 14336, 4096, 2),
                                ("f32", 8192, 8192, 2), ("q8", 8192, 8192, 1), ("q8", 14336, 4096, 1),
                                ("q4", 4096, 14336, 7), ("q4", 14336, 4096, 1), ("f16x32", 8192, 8192, 7),
                                ("f16x32", 4096, 14336, 7), ("f16x32", 14336, 4096, 7)):
        p = plan(kind, M, N)
        assert p["variant"] == variant and p["grid"] >= 256, (kind, M, N, p)


def test_slab_plans_of_the_named_shapes():
    # (variant, block = 64 S, loads in flight, rows per slab, grid)
    def geo(p):
        return (p["variant"], p["block"], p["units_in_flight"], p["rows_per_wave"], p["grid"])

    # INT4 4096x14336: 7 passes, 7 waves, one pass each, slabs of 4 rows
    assert geo(plan("q4", 4096, 14336)) == (7, 448, 4, 4, 1024)
    # FP16 with FP32 x: 16 passes, 16 waves; 28 passes: 14 waves of two
    # passes, 8 in flight, slabs of 8 rows (slabs of 4 would give the
    # busiest CU as many rows in twice the workgroups)
    assert geo(plan("f16x32", 8192, 8192)) == (7, 1024, 4, 4, 2048)
    assert geo(plan("f16x32", 4096, 14336)) == (7, 896, 8, 8, 512)
    # rows of 17-32 units with slabs of 4 rows where those load the busiest
    # CU less (INT8 2295x24576: 3 slabs of 4 rows against 2 of 8)
    assert geo(plan("q8", 2295, 24576)) == (7, 768, 8, 4, 574)
    # INT4: at most 32 waves per CU, workgroups walk the slabs beyond
    p = plan("q4", 300000, 8192)
    assert (p["variant"], p["block"], p["grid"]) == (7, 256, 8 * 256) and p["rows_per_wave"] >= 300000 / (8 * 256)
    # INT8 rows of an even count from 10 units: two passes per wave
    assert geo(plan("q8", 2567, 15616)) == (7, 512, 8, 4, 642)
    assert geo(plan("q8", 1913, 10240)) == (7, 320, 8, 4, 479)
    # INT4 one-unit rows past the packed kernel (more than 32 chunks), from
    # 4 rows per CU: one wave per slab, at most 32 per CU
    assert geo(plan("q4", 51636, 1408)) == (7, 64, 4, 4 * 2, 32 * 256) and plan("q4", 1023, 1408)["variant"] != 7
    assert plan("q4", 51636, 1024)["variant"] == 4
    # where the streaming kernel stays: INT4 rows of 2 or 6 units, INT8 rows
    # under 9 units, long INT4 rows beyond 12 rows per CU, INT8 beyond 100,
    # fewer rows than CUs
    for kind, M, N in (("q4", 14336, 4096), ("q4", 5113, 10880), ("q8", 14336, 4096), ("q8", 8192, 8192),
                       ("q8", 4039, 15616), ("q8", 5559, 13312),
                       ("q4", 9681, 21504), ("q8", 33708, 13184), ("q4", 255, 8192), ("f16x32", 255, 8192),
                       ("q8", 511, 24576)):
        assert plan(kind, M, N)["variant"] != 7, (kind, M, N)


def test_long_rows_stage_x_up_to_the_device_limit():
    # INT8/INT4 and FP16-with-FP32-x rows whose staged x passes 64 KiB stage
    # it while it fits a workgroup; a 64-KiB device reads x with each unit
    for kind, M, N in (("q8", 4096, 34816), ("q4", 4096, 34816), ("q4", 2048, 81920), ("f16x32", 4096, 24576)):
        assert staged_bytes(kind, N) > 64 * 1024
        p = plan(kind, M, N)
        spare = 64 * 16 if p["stage_order"] == 2 else 0
        assert p["variant"] == 1 and p["lds_bytes"] == staged_bytes(kind, N) + spare, (kind, M, N, p)
        assert plan(kind, M, N, lds_max=64 * 1024)["variant"] == 2, (kind, M, N)
    # one unit past what a workgroup may hold
    assert plan("q8", 4096, 81920)["variant"] == 1 and plan("q8", 4096, 81920 + 1024)["variant"] == 2
    assert plan("q4", 4096, 83968)["variant"] == 2
    assert plan("f16x32", 4096, 40960 + 512)["variant"] == 2
    assert plan("f16x32", 64, 40960 + 512)["variant"] == 6     # few rows: split, x read with each unit


def test_few_rows_rules():
    cus = 256
    # few INT4 rows of four units or more (rows of 6 units: the others take
    # row slabs): x per unit; one more row: staged
    assert plan("q4", 4 * cus, 12288)["variant"] == 2
    assert plan("q4", 4 * cus + 1, 12288)["variant"] == 1
    # INT8 rows of four units or more, up to 6 rows per CU: split rows, S for
    # 4 waves per CU, 2 in flight; a few more rows (up to 8 per CU, up to 16
    # units): x read with each unit
    p = plan("q8", 4 * cus, 8192)
    assert (p["variant"], p["block"], p["units_in_flight"], p["grid"]) == (6, 128, 2, 4 * cus)
    p = plan("q8", 300, 38592)
    assert (p["variant"], p["block"], p["units_in_flight"]) == (6, 256, 2)
    assert plan("q8", 6 * cus, 8192)["variant"] == 6
    assert plan("q8", 6 * cus + 1, 8192)["variant"] == 2
    # INT8 rows of 64 units with at most 8 rows per CU: x per unit, two rows a wave
    p = plan("q8", 2048, 65536)
    assert (p["variant"], p["units_in_flight"]) == (2, 8)


def test_short_rows_rules():
    # INT8/INT4 rows of at most 32 chunks: the packed kernel
    assert plan("q8", 14336, 512)["variant"] == 4
    assert plan("q4", 14336, 1024)["variant"] == 4
    # one unit just past: x in registers (INT4 from 4 rows per CU: row slabs)
    assert plan("q8", 14336, 528)["variant"] == 5
    assert plan("q4", 1000, 1152)["variant"] == 5
    assert plan("q4", 14336, 1152)["variant"] == 7
    # FP16 rows of one and two units: x in registers
    assert plan("f16", 4096, 512)["variant"] == 5
    assert plan("f16", 14336, 1024)["variant"] == 5


def test_grid_cap_makes_waves_walk():
    # more rows than 2^30 work-items allow at one row (or four) per wave
    p = plan("f16", (1 << 24) + (1 << 20) + 3, 3)
    assert p["variant"] == 3 and p["grid"] * p["block"] == 1 << 30 and p["rows_per_wave"] == 2
    p = plan("f16", (1 << 26) + 1000, 8)
    assert p["grid"] * p["block"] <= 1 << 30 and p["rows_per_wave"] >= 5


def test_describe_launch_for_rejects_bad_arguments():
    with pytest.raises(GemvError):
        plan("q4", 16, 200)              # N % 128 != 0
    with pytest.raises(GemvError):
        plan("f16", -1, 16)
    with pytest.raises(GemvError):
        plan("f16", 16, 16, cus=0)
    with pytest.raises(GemvError):
        plan("f16", 16, 16, lds_max=0)
    lib = binding.load()
    assert lib.gemv_describe_launch_for(6, 16, 16, 1, 256, 163840, None) == 1


def _acc16_terms(variant, N):
    # binary16 running-sum terms per lane and row, by kernel: the element-wise
    # kernel (3) adds one column per pass of 64 lanes; the streaming (2) and
    # x-in-registers (5) kernels keep an (even, odd) pair per lane and add four
    # column pairs of each 16-byte chunk, one chunk per 512-column pass
    if variant == 3:
        return -(-N // 64)
    assert variant in (2, 5), variant      # any other kernel needs its own count here
    return 4 * -(-N // 512)


@pytest.mark.parametrize("dev", _DEVICES, ids=lambda d: f"{d['cus']}cu_{d['lds_max'] // 1024}k")
def test_fp16_accumulation_plans_keep_the_gate_term_count(dev):
    # the FP16-accumulation gate (oracle.metrics.acc16_bound) assumes at most
    # k = max(ceil(N/64), 4) terms per binary16 sum; every plan the library can
    # choose must keep within it, unaligned operands included
    from oracle.metrics import acc16_bound  # noqa: F401  (the gate this pins)

    for N in _NS + [1, 7, 9, 4100, 65536, 131072]:
        k = max(-(-N // 64), 4)
        for M in _MS:
            for aligned in (True, False):
                p = plan("f16_acc16", M, N, dev["cus"], dev["lds_max"], aligned)
                assert _acc16_terms(p["variant"], N) <= k, (M, N, aligned, dev, p)


# (variant, grid, block, units in flight, rows per wave) of the named
# workloads on MI355X: the measured rules' plans, which the FP32/FP16 cost
# model leaves in place (it predicts less than its margin of a gain there)
_NAMED_PLANS = {
    ("f16", 8192, 8192): (2, 1024, 512, 8, 1),
    ("f16", 4096, 14336): (2, 256, 256, 8, 4),
    ("f16", 14336, 4096): (2, 3584, 256, 8, 1),
    ("f16", 4096, 4096): (2, 1024, 256, 8, 1),
    ("f32", 1024, 1024): (2, 256, 256, 4, 1),
    ("f32", 2048, 2048): (2, 512, 256, 8, 1),
    ("f32", 4096, 4096): (2, 512, 512, 8, 1),
    ("f32", 8192, 8192): (2, 2048, 256, 8, 1),
    ("f16", 1792, 4096): (2, 448, 256, 8, 1),
    ("f16", 14336, 512): (2, 448, 512, 4, 4),
}


def _geometry(p):
    return (p["variant"], p["grid"], p["block"], p["units_in_flight"], p["rows_per_wave"])


def test_named_workloads_keep_their_measured_plans():
    for (kind, M, N), want in _NAMED_PLANS.items():
        assert _geometry(plan(kind, M, N)) == want, (kind, M, N)


def test_cost_model_replaces_plans_the_measurements_beat():
    # Graph-timed times of every candidate plan on MI355X (us): the rules'
    # plan, the cost model's, and the fastest candidate.
    #   FP16 2552x9088: 8 waves, 4 in flight, 319 workgroups (63 CUs with two)
    #     12.42; split rows, 2 waves per row, 2 in flight 9.88; best 9.62
    #   FP16 4351x9856: 8 waves, 8 in flight, two rows per wave 21.33; split
    #     rows, 2 waves, 2 in flight 16.24; best 15.94
    #   FP16 278x16896: 16 waves per row, 4 in flight (each wave's 2-3 units
    #     padded to 4) 5.54; 4 waves per row, 4 in flight 4.74; best 4.50
    #   FP32 902x5248 and FP16 774x24704: 8 waves per row 6.22 and 10.43;
    #     the split rules' two waves per row (from two rows per CU), which
    #     the model keeps, 5.27 and 8.88; one wave per row, 4-wave
    #     workgroups, 8 in flight 4.97 and 8.43 (the fastest of all
    #     candidates, within the model's margin of the split here)
    assert _geometry(plan("f16", 2552, 9088)) == (6, 2552, 128, 2, 1)
    assert _geometry(plan("f16", 4351, 9856)) == (6, 4351, 128, 2, 1)
    assert _geometry(plan("f16", 278, 16896)) == (6, 278, 256, 4, 1)
    assert _geometry(plan("f32", 902, 5248)) == (6, 902, 128, 4, 1)
    assert _geometry(plan("f16", 774, 24704)) == (6, 774, 128, 4, 1)
    # From two rows per CU the model keeps split rows at two waves: its
    # 4-16 waves per row lost there in 9 of 11 measured shapes (FP32
    # 1399x28288 29.53 -> 26.76, 581x23168 12.95 -> 11.58, FP16 1071x29440
    # 13.84 -> 12.65); below that many waves per row still pay.
    assert _geometry(plan("f32", 1399, 28288)) == (6, 1399, 128, 4, 1)
    assert _geometry(plan("f32", 581, 23168)) == (6, 581, 128, 4, 1)
    assert _geometry(plan("f16", 1071, 29440)) == (6, 1071, 128, 4, 1)
    assert plan("f16", 400, 29440)["block"] > 128
    # the other formats keep the measured rules alone (FP16 with FP32 x:
    # row slabs)
    assert plan("f16_acc16", 2552, 9088)["variant"] == 2
    assert plan("f16x32", 2562, 14336)["variant"] == 7


def test_rules_remeasured_by_brute_force():
    # Rules the same brute-force search changed (graph-timed us, before ->
    # after): FP16 with FP32 x, rows of 4-11 units, many rows: staged, 4
    # waves, split staging, at most 2 workgroups per CU (5484x4608 13.25 ->
    # 9.67); INT4 rows of 2-3 units: at most 4 workgroups per CU (14336x4096
    # 7.52 -> 7.30); packed short rows beyond 16 groups per CU: two groups
    # per wave (INT4 40979x512 5.73 -> 4.79); INT8 rows of 8-10 units: 4
    # waves, two rows per wave, split staging (8192x8192 12.11 -> 11.65)
    # (FP16 with FP32 x 5484x4608 has since taken row slabs)
    p = plan("f16x32", 5484, 4608)
    assert (p["variant"], p["block"], p["units_in_flight"], p["grid"]) == (7, 576, 4, 1371)
    p = plan("q4", 14336, 4096)
    assert (p["variant"], p["block"], p["stage_order"], p["grid"]) == (1, 512, 2, 4 * 256)
    p = plan("q4", 40979, 512)
    assert (p["variant"], p["units_in_flight"], p["rows_per_wave"]) == (4, 2, 2 * 4)
    p = plan("q8", 8192, 8192)
    assert (p["variant"], p["block"], p["stage_order"], p["units_in_flight"], p["grid"]) == (1, 256, 2, 4, 1024)


def test_rules_from_the_random_shape_search():
    # Rules the brute-force search over seeded random shapes changed
    # (graph-timed us, before -> after):
    #   FP32/FP16 rows of 24 units and more, 11-16 rows per CU: 4 waves of
    #     four rows, 8 in flight, one workgroup per CU, kept from split rows
    #     and the cost model (FP32 3912x6784 19.27 -> 16.83, FP16
    #     3656x26752 33.58 -> 29.89)
    #   FP32/FP16 split rows from two rows per CU: two waves per row, 4 in
    #     flight (FP16 10463x3200 13.25 -> 11.43)
    #   INT4 rows of 10 units and more: 8 waves, split staging, one
    #     workgroup per CU; many rows of 4 units: two (5832x25088 17.59 ->
    #     16.10, 4096x8192 5.70 -> 5.45)
    #   FP16 with FP32 x: split rows of two waves up to 5-7 rows per CU
    #     (977x27392 15.08 -> 11.83); staged, 4 waves, 8 in flight, one
    #     workgroup per CU for rows of 16 units and more (12815x14720 63.45
    #     -> 57.50)
    for kind, M, N in (("f32", 3912, 6784), ("f16", 3656, 26752)):
        p = plan(kind, M, N)
        assert (p["variant"], p["block"], p["units_in_flight"], p["rows_per_wave"]) == (2, 256, 8, 4), (kind, M, N, p)
        assert p["grid"] == -(-M // 16) <= 256, (kind, M, N, p)
    p = plan("f16", 10463, 3200)
    assert (p["variant"], p["block"], p["units_in_flight"], p["grid"]) == (6, 128, 4, 10463)
    p = plan("q4", 5832, 25088)
    assert (p["variant"], p["block"], p["stage_order"], p["units_in_flight"], p["grid"]) == (1, 512, 2, 4, 256)
    # (INT4 4096x8192, rows of 4 units, has since taken row slabs)
    p = plan("q4", 4096, 8192)
    assert (p["variant"], p["block"], p["units_in_flight"], p["grid"]) == (7, 256, 4, 1024)
    p = plan("f16x32", 977, 27392)
    assert (p["variant"], p["block"], p["units_in_flight"], p["grid"]) == (6, 128, 2, 977)
    p = plan("f16x32", 12815, 14720)
    assert (p["variant"], p["block"], p["stage_order"], p["units_in_flight"], p["grid"]) == (1, 256, 2, 8, 256)


def test_plan_cache_gives_the_same_plans():
    # each host thread keeps its last 16 plans: more shapes than that,
    # interleaved across devices and in two orders, give the same plans
    import numpy as np

    rng = np.random.default_rng(7)
    shapes = [(KINDS[rng.integers(len(KINDS))], int(rng.integers(1, 70000)), int(rng.integers(1, 300)) * 128)
              for _ in range(60)]
    devs = [MI355X, dict(cus=80, lds_max=64 * 1024)]
    first = {(s, i): plan(*s, **d) for s in shapes for i, d in enumerate(devs)}
    for s in reversed(shapes):
        for i, d in reversed(list(enumerate(devs))):
            assert plan(*s, **d) == first[(s, i)], (s, d)


def _kernel_vgprs():
    """VGPR counts of the built library's gfx950 kernels, read from the
    code object's metadata: {demangled name: vgprs}."""
    import os
    import re
    import shutil
    import subprocess
    import tempfile

    from memory_bound_gemv_row_amd import build as hip_build

    lib = hip_build.LIB
    llvm = "/opt/rocm/llvm/bin"
    tools = [shutil.which("objcopy"), shutil.which("c++filt"), os.path.join(llvm, "clang-offload-bundler"),
             os.path.join(llvm, "llvm-readelf")]
    if not os.path.exists(lib) or not all(t and os.path.exists(t) for t in tools):
        pytest.skip("built library or code-object tools not available")
    with tempfile.TemporaryDirectory() as d:
        fat, dev, copy = os.path.join(d, "fat.bin"), os.path.join(d, "dev.o"), os.path.join(d, "copy.so")
        # (objcopy rewrites its input unless given an output file)
        subprocess.run([tools[0], "--dump-section", f".hip_fatbin={fat}", lib, copy], check=True)
        subprocess.run([tools[2], "--unbundle", "--type=o", f"--input={fat}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"], check=True)
        notes = subprocess.run([tools[3], "--notes", dev], check=True, capture_output=True, text=True).stdout
    out, name = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            name = m.group(1)
        m = re.match(r"\s+\.vgpr_count:\s+(\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    names = list(out)
    plain = subprocess.run([tools[1]], input="\n".join(names), check=True, capture_output=True,
                           text=True).stdout.splitlines()
    return {p.split("(")[0]: out[n] for n, p in zip(names, plain)}


def test_fp_kernel_occupancy_matches_the_cost_model():
    # The FP32/FP16 cost model assumes 7 waves per SIMD for the streaming
    # kernels with 8 units in flight and 8 for every other FP32/FP16 kernel
    # it chooses from (512 VGPRs per SIMD lane, allocated in blocks of 8).
    import re

    vg = _kernel_vgprs()
    seen = 0
    for name, v in vg.items():
        m = re.match(r"void gemv::gemv_(stream|xreg|split)<([01]), (\d+), (\d+)(.*)>$", name)
        if not m:
            continue
        kernel, D = m.group(1), int(m.group(4))
        if kernel == "stream" and not m.group(5).endswith("true, true, 0"):
            continue
        waves = min(8, 512 // (-(-v // 8) * 8))
        want = 7 if kernel == "stream" and D == 8 else 8
        assert waves == want, (name, v)
        seen += 1
    assert seen >= 40, seen


# ---------------------------------------------------------------- explicit plans (gemv_check_plan_for)
def check(kind, M, N, plan, cus=256, lds_max=160 * 1024):
    return binding.check_plan_for(kind, M, N, cus, lds_max, plan)


def test_planner_plans_as_explicit_plans():
    # the planner's choices, written as explicit plans, make the same launch
    for kind, M, N, p in (("f16", 8192, 8192, (2, 8, 8, 1, -1, 0)), ("q8", 8192, 8192, (1, 4, 4, 2, 2, 0)),
                             ("q4", 14336, 4096, (1, 8, 2, 1, 2, 4)), ("f16", 2552, 9088, (6, 2, 2, 1, -1, 0)),
                             ("q4", 14336, 512, (4, 8, 1, 1, -1, 0)), ("f16", 14336, 512, (2, 8, 4, 4, -1, 0)),
                             ("f16x32", 5484, 4608, (7, 9, 4, 4, -1, 0)), ("q8", 1000, 16400, (6, 2, 2, 1, -1, 0)),
                             ("q4", 4096, 14336, (7, 7, 4, 4, -1, 0)), ("f16x32", 4096, 14336, (7, 14, 8, 8, -1, 0)),
                             ("q4", 300000, 8192, (7, 4, 4, 4, -1, 8))):
        assert check(kind, M, N, p) == plan(kind, M, N), (kind, M, N, p)


def test_explicit_plans_the_library_has_no_kernel_for():
    for kind, M, N, p in (
            ("f16", 4096, 4096, (1, 8, 8, 1, 0, 0)),     # FP16 reads x with each unit: no staged kernel
            ("f16", 4096, 4096, (2, 12, 4, 1, -1, 0)),   # no 12-wave streaming kernel
            ("f16", 4096, 4096, (2, 4, 3, 1, -1, 0)),    # 3 in flight: INT4 staged rows only
            ("f16", 4096, 4096, (2, 4, 4, 1, 1, 0)),     # a stage order without staging
            ("q8", 4096, 4096, (1, 4, 4, 1, 3, 0)),      # stage orders are 0-2
            ("q8", 4096, 4096, (1, 4, 5, 1, 0, 0)),      # 5 in flight: INT8 split staging only
            ("f16", 4096, 4096, (5, 4, 2, 1, -1, 0)),    # x in registers: rows of 1-3 units only
            ("f16", 4096, 1024, (5, 8, 2, 1, -1, 0)),    # two-unit rows: 4 waves only
            ("f16", 4096, 4096, (4, 8, 1, 1, -1, 0)),    # packed rows: INT8/INT4 only
            ("q8", 4096, 1024, (4, 8, 1, 1, -1, 0)),     # packed rows: at most 32 chunks
            ("f16", 4096, 4096, (6, 8, 2, 1, -1, 0)),    # split rows: at least two units per wave
            ("f16", 4096, 4096, (6, 3, 2, 1, -1, 0)),    # waves per row: 2, 4, 8 or 16
            ("f16", 4096, 8192, (6, 2, 8, 1, -1, 0)),    # split rows: 2 or 4 in flight
            ("f16_acc16", 4096, 8192, (6, 2, 2, 1, -1, 0)),   # FP16 accumulation: variants 2 and 5
            ("q8", 4096, 98304, (1, 4, 4, 1, 1, 0)),     # staged x beyond the LDS a workgroup may hold
            ("f16", 4096, 4100, (2, 4, 4, 1, -1, 0)),    # not a multiple of the chunk: element-wise only
            ("f16", 4096, 4096, (7, 4, 4, 4, -1, 0)),    # row slabs: INT8, INT4, FP16 with FP32 x only
            ("q8", 4096, 8192, (7, 3, 4, 4, -1, 0)),     # slabs: S waves own P / S passes (P = 8)
            ("q8", 4096, 8192, (7, 2, 4, 4, -1, 0)),     # ... one or two passes per wave
            ("q8", 4096, 8192, (7, 8, 2, 4, -1, 0)),     # ... 4 or 8 in flight
            ("q8", 4096, 8192, (7, 8, 8, 4, -1, 0)),     # ... that divide the slab's units
            ("q8", 4096, 8192, (7, 8, 4, 2, -1, 0)),     # ... slabs of 4 or 8 rows
            ("q8", 4096, 8192, (7, 8, 4, 4, 2, 0)),      # ... nothing staged
            ("q8", 4096, 17408, (7, 17, 4, 4, -1, 0)),   # ... at most 16 waves
            ("f16", 4096, 4096, (7, 4, 4, 1, -1, 0)), ("f16", 4096, 4096, (2, 4, 4, 0, -1, 0)),
            ("f16", 4096, 4096, (2, 4, 4, 1, -1, -1))):
        assert check(kind, M, N, p) is None, (kind, M, N, p)
    with pytest.raises(GemvError):
        check("f16", 0, 4096, (2, 4, 4, 1, -1, 0))
    with pytest.raises(GemvError):
        check("f16", 4096, 4096, (2, 4, 4, 1, -1, 0), cus=0)


def test_every_candidate_plan_keeps_the_invariants():
    # the plan search's candidates that the library accepts, over seeded
    # shapes and devices: within the dispatch limit and the device's LDS,
    # every row covered, split rows one workgroup per row
    import numpy as np

    import bench

    rng = np.random.default_rng(11)
    for _ in range(60):
        kind = KINDS[rng.integers(len(KINDS))]
        M = int(np.exp(rng.uniform(0, np.log(1 << 22))))
        N = max(128, int(np.exp(rng.uniform(np.log(64), np.log(1 << 17)))) // 128 * 128)
        dev = dict(cus=int(rng.choice([80, 256, 304])), lds_max=int(rng.choice([64, 160]) * 1024))
        for p in bench.plan_candidates(kind, N):
            info = check(kind, M, N, p, **dev)
            if info is None:
                continue
            where = (kind, M, N, dev, p, info)
            assert info["variant"] == p[0] and info["units_in_flight"] == p[2], where
            assert 1 <= info["grid"] and info["grid"] * info["block"] <= 1 << 30, where
            assert info["lds_bytes"] <= dev["lds_max"], where
            if p[0] == 6:
                assert info["grid"] == M and info["block"] == 64 * p[1], where
            elif p[0] == 7:
                assert info["block"] == 64 * p[1] and info["grid"] * info["rows_per_wave"] >= M, where
            elif p[0] != 4:
                assert info["grid"] * (info["block"] // 64) * info["rows_per_wave"] >= M, where
