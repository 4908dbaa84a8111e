"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Full-size workloads are compared element by element on every output (the
oracle computes them all in seconds), in the same launch configuration the
benchmark times.  Smaller shapes cover several tiles and ragged tails, both
kernel variants (16-byte chunks and the element-wise path), every
rows-per-wave setting, and the degenerate cases.  Integer-valued and
subnormal inputs make every summation order exact, so those cases must match
bit for bit.
"""
import numpy as np
import pytest
import torch

from memory_bound_gemv_row_amd import inputs, binding

from gpu_util import dev, run_gpu, run_oracle, say, within_gate
from qpack import pack_int4, f16

pytestmark = pytest.mark.gpu


def _check(oracle, kind, ops, label):
    say(f"[parity] {label}")
    y = run_gpu(kind, ops)
    ref = run_oracle(oracle, kind, ops)
    rep = within_gate(oracle, kind, ops, y, ref)
    assert rep["ok"], (label, rep)
    return rep


# ---------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("w", inputs.all_workloads(), ids=lambda w: w.name)
def test_full_size_workload(gpu, oracle_mod, w):
    ops = inputs.make(w.kind, w.M, w.N, seed=0)
    info = binding.describe_launch(w.kind, w.M, w.N, aligned=True)
    assert info["variant"] in (1, 2, 7), info    # the bandwidth path is what runs
    rep = _check(oracle_mod, w.kind, ops, f"{w.name} seed 0 {info}")
    print(w.name, rep)


# ---------------------------------------------------------------- shapes, tiles, tails
_MS = [1, 2, 3, 4, 5, 7, 9, 16, 17, 33, 65, 257]
_NS = {
    # multiples of the chunk width (bandwidth path) and ragged ones (element-wise)
    "f32": [1, 3, 4, 8, 60, 64, 252, 256, 260, 1020, 1024, 2052, 4100, 9000, 17000],
    "f16": [1, 7, 8, 16, 504, 512, 520, 1000, 1024, 1528, 1536, 2056, 3584, 4648, 8200, 14336, 20000],
    # 16..512 (1-32 chunks) take the packed short-row kernel, 528 is the
    # first streaming width
    # 33024 (33 units) stages 66 KiB of x, past 64 KiB: one workgroup per CU
    # with so few rows; INT4 33280 (17 units, 68 KiB): few rows, x per unit
    "q8": [1, 15, 16, 32, 48, 272, 512, 528, 1008, 1024, 1040, 5000, 8192, 9232, 20000, 33024],
    # 5632 | 6144 straddle the staged-x threshold; 16392 stages just over
    # 64 KiB of FP32 x (one workgroup per CU)
    "f16x32": [1, 7, 8, 16, 504, 512, 520, 1000, 1024, 4648, 5632, 6144, 8200, 14336, 16384, 16392, 20000],
    "f16_acc16": [1, 7, 8, 16, 504, 512, 520, 1000, 1024, 4648, 8200, 14336, 20000],
    # up to 1024 (32 chunks) packed; 640 and 896 fill 20 and 28 of 32 lanes
    "q4": [128, 256, 384, 640, 896, 1024, 1152, 2048, 2176, 4096, 7296, 14336, 33280],
}


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
def test_shapes_and_tails(gpu, oracle_mod, kind):
    for N in _NS[kind]:
        for M in _MS:
            ops = inputs.make(kind, M, N, seed=M * 7919 + N)
            _check(oracle_mod, kind, ops, f"{kind} M={M} N={N}")


@pytest.mark.parametrize("kind,N", [("f32", 64 * 4 * 8 * 2 + 4), ("f16", 64 * 8 * 17 + 8), ("q8", 64 * 16 * 9 + 16),
                                    ("q4", 64 * 32 * 3 + 128), ("f16x32", 64 * 8 * 17 + 8), ("f16x32", 64 * 8 * 3 + 8)])
def test_many_passes_and_row_groups(gpu, oracle_mod, kind, N):
    # enough rows for several workgroups, a partial last workgroup, and rows
    # whose chunk count leaves a partly filled final pass
    ops = inputs.make(kind, 4 * 50 + 3, N, seed=5)
    _check(oracle_mod, kind, ops, f"{kind} tiles N={N}")


@pytest.mark.parametrize("kind,N,walk", [("q8", 2048, 2), ("q8", 4096 + 16, 2), ("q4", 2048 + 128, 2), ("q4", 14336, 2),
                                         ("f16x32", 1024, 2), ("f16x32", 8192 + 8, 4)])
def test_waves_walk_several_rows(gpu, oracle_mod, kind, N, walk):
    # grids capped per CU: each wave walks `walk` rows and more, the last ones
    # ragged across waves
    # (the cap can depend on M, so settle M against the plan it gets)
    M = 1 << 20
    for _ in range(4):
        probe = binding.describe_launch(kind, M, N)
        M = probe["grid"] * probe["block"] // 64 * walk + 37
    info = binding.describe_launch(kind, M, N)
    assert info["rows_per_wave"] >= 3, info
    ops = inputs.make(kind, M, N, seed=11)
    _check(oracle_mod, kind, ops, f"{kind} multi-row M={M} N={N} {info}")


@pytest.mark.parametrize("kind,N,small,large", [("q8", 1024, 5, 5), ("q8", 1008, 5, 5), ("q8", 2048, 2, 1),
                                                ("q8", 4096, 2, 1), ("q8", 8192 - 16, 2, 1),
                                                ("q4", 2048, 7, 7), ("q4", 4096, 5, 1), ("q4", 2176, 5, 1)])
def test_quantised_x_paths_by_rows(gpu, oracle_mod, kind, N, small, large):
    # INT8/INT4 take x in registers (variant 5: rows of one unit, and few
    # INT4 rows of two), read with each unit (2) for few longer rows, and
    # staged in LDS (1) for many; INT4 one-unit rows of more than 32 chunks
    # from 4 rows per CU take row slabs (7): each plan at the same row length, with a
    # ragged last workgroup (and, for many one-unit rows, waves walking
    # several rows two loads deep)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M, variant in ((8 * cus - 5, small), (16 * cus + 5, large), (40 * cus + 7, large)):
        info = binding.describe_launch(kind, M, N)
        assert info["variant"] == variant, (M, info)
        ops = inputs.make(kind, M, N, seed=M + N)
        _check(oracle_mod, kind, ops, f"{kind} M={M} N={N} {info}")


# (kind, M, N, variant, stage order) on a device of 256 CUs whose workgroups
# may hold 160 KiB of LDS; rows end in a ragged last pass
_LONG_ROWS = [
    ("q8", 1024, 32848, 6, -1),   # 66 KiB of x, few rows: split rows, x read with each unit
    ("q8", 3000, 32848, 1, 2),    # two workgroups per CU, waves walk two rows
    ("q8", 3000, 49168, 1, 1),    # 98 KiB: one workgroup per CU, waves walk two rows
    ("q8", 2000, 49168, 2, -1),   # one workgroup per CU and few rows: x per unit
    ("q8", 2200, 81936, 2, -1),   # staged x would not fit a workgroup
    ("q4", 3000, 34944, 1, 1),    # 72 KiB: one workgroup per CU
    ("q4", 1000, 34944, 2, -1),   # few rows: x per unit
    ("q4", 300, 82048, 2, -1),    # staged x would not fit a workgroup
    ("q8", 1000, 16400, 6, -1),   # rows of 17 units, few of them: split rows
    ("q4", 1000, 12160, 2, -1),   # few INT4 rows of 6 units: x per unit
    ("f16x32", 4100, 24584, 1, 2),  # 96 KiB of FP32 x: staged, one workgroup per CU
    ("f16x32", 1100, 24584, 6, -1),  # few rows of 49 units: two waves per row
    ("f16x32", 2100, 40968, 2, -1),  # FP32 x would not fit a workgroup
    ("q4", 3000, 81920, 1, 1),    # staged x of exactly 160 KiB
    ("q8", 3000, 80848, 1, 1),    # 158 KiB, ragged last pass
    ("f16x32", 4100, 40960, 1, 1),  # 160 KiB of FP32 x: no room for split staging's spare granules
]


@pytest.mark.parametrize("kind,M,N,variant,stg", _LONG_ROWS)
def test_long_rows_staged_or_per_unit(gpu, oracle_mod, kind, M, N, variant, stg):
    # rows whose staged x passes 64 KiB (and few long INT rows): staged up
    # to what one workgroup may hold (one or two workgroups per CU), x read
    # with each unit for few rows or beyond that
    props = torch.cuda.get_device_properties(0)
    info = binding.describe_launch(kind, M, N)
    if props.multi_processor_count == 256 and props.shared_memory_per_block == 160 * 1024:
        assert (info["variant"], info["stage_order"]) == (variant, stg), info
    ops = inputs.make(kind, M, N, seed=M + 7 * N)
    _check(oracle_mod, kind, ops, f"{kind} long rows M={M} N={N} {info}")


@pytest.mark.parametrize("kind,M,N,D,rows", [("f16_acc16", 8192, 14336 + 8, 8, 2), ("f32", 6144 + 3, 12288, 8, 1),
                                             ("f16_acc16", 3000, 12288 + 8, 8, 4), ("f16_acc16", 4096 + 1, 14336, 4, 2),
                                             ("f16_acc16", 6400, 16384, 8, 1), ("f16_acc16", 4096 + 7, 16384, 8, 1)])
def test_long_fp_rows(gpu, oracle_mod, kind, M, N, D, rows):
    # The measured rules for rows of 24 units and more: 8 in flight and one
    # row per wave from 24 rows per CU or for multiples of 16 units (two
    # where the units are not a multiple of 8), two rows per wave up to 11
    # per CU, four from 11 to 16 (rows not a multiple of 16 units), 4 in
    # flight between; ragged last passes.  FP16 accumulation
    # keeps these rules; FP32/FP16 take the cost model's plan where it
    # predicts a clear gain (its plans are checked in test_gpu_split.py)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    info = binding.describe_launch(kind, M, N)
    if cus == 256:
        assert (info["variant"], info["units_in_flight"]) == (2, D), info
        assert info["grid"] * info["block"] // 64 * rows >= M, info
    ops = inputs.make(kind, M, N, seed=M + N)
    _check(oracle_mod, kind, ops, f"{kind} long rows M={M} N={N} {info}")


@pytest.mark.parametrize("kind,M,N", [("q8", 26000, 9216 + 16), ("q8", 30000, 8192 + 16), ("f16x32", 3000, 12800 - 8),
                                      ("f16x32", 2048 + 3, 8704 - 8), ("f16_acc16", 4096 + 5, 4608 + 8)])
def test_two_rows_per_wave_where_that_pads_less(gpu, oracle_mod, kind, M, N):
    # rows whose unit count does not divide by the loads in flight: two rows
    # per wave (with enough rows to give every CU a workgroup), one padded
    # sequence per wave (ragged last passes too).  INT8 rows of 9-10 units
    # beyond 100 rows per CU and FP16-with-FP32-x rows of an odd number of
    # units past 16 (the others take row slabs)
    info = binding.describe_launch(kind, M, N)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert info["rows_per_wave"] == 2, info
    ops = inputs.make(kind, M, N, seed=M * 3 + N)
    _check(oracle_mod, kind, ops, f"{kind} two rows per wave M={M} N={N} {info}")


@pytest.mark.parametrize("M,N,block,stg", [(16384 + 3, 6144, 256, 2), (9000, 7168 - 16, 256, 2),
                                           (12000, 3072 - 16, 256, 2)])
def test_int8_rows_of_3_6_7_units(gpu, oracle_mod, M, N, block, stg):
    # many INT8 rows of 3, 6 or 7 units: 4 waves, split staging, at most 3
    # (rows of 3 units) or 4 workgroups per CU; waves walk several rows
    # (ragged passes too)
    info = binding.describe_launch("q8", M, N)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert (info["variant"], info["block"], info["stage_order"]) == (1, block, stg), info
        assert info["rows_per_wave"] >= 2, info
    ops = inputs.make("q8", M, N, seed=M - N)
    _check(oracle_mod, "q8", ops, f"q8 short staged rows M={M} N={N} {info}")


@pytest.mark.parametrize("kind,M,N,D", [("q4", 4096 + 5, 12288, 3), ("q8", 14336 + 1, 5120 - 16, 5),
                                        ("q8", 3000, 5120, 5)])
def test_depths_that_divide_the_row(gpu, oracle_mod, kind, M, N, D):
    # INT4 rows of 6 units and INT8 rows of 5: 3 or 5 units in flight
    # (waves walking one or several rows, a ragged last pass for INT8); INT4
    # rows of 5 units take row slabs, their 5-deep streaming kernel runs as
    # an explicit plan in test_gpu_plans
    info = binding.describe_launch(kind, M, N)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert (info["variant"], info["units_in_flight"]) == (1, D), info
    ops = inputs.make(kind, M, N, seed=M + 13 * N)
    _check(oracle_mod, kind, ops, f"{kind} depth {D} M={M} N={N} {info}")


@pytest.mark.parametrize("M,N,rows", [(20 * 256 + 5, 8192 - 16, 2), (32 * 256, 17408, 1), (24 * 256 + 3, 17408 - 16, 1)])
def test_int8_long_rows_split_staging(gpu, oracle_mod, M, N, rows):
    # INT8 rows of 8-31 units, many rows: 4-wave workgroups with split
    # staging; rows of 8-10 units two per wave, longer ones at most 2
    # workgroups per CU so that waves walk several rows (ragged last pass).
    # Rows of 8 and 17 units: rows of 9-16 units and of an even count up to
    # 32 take row slabs up to 100 rows per CU
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    info = binding.describe_launch("q8", M, N)
    if cus == 256:
        assert (info["variant"], info["block"], info["stage_order"]) == (1, 256, 2), info
        want = -(-M // 8) if rows == 2 else min(-(-M // 4), 2 * cus)
        assert info["grid"] == want, info
    ops = inputs.make("q8", M, N, seed=M ^ N)
    _check(oracle_mod, "q8", ops, f"q8 split staging M={M} N={N} {info}")


@pytest.mark.parametrize("kind,M,N", [("f32", 8000, 252), ("f32", 9000, 260), ("f16", 14336, 1000),
                                      ("f16x32", 3000, 512), ("f16x32", 3000, 504), ("f16_acc16", 6000, 1024),
                                      ("q8", 14336, 1008), ("q4", 900, 2048), ("f16", 14336, 1528),
                                      ("f32", 4096, 768), ("q4", 200, 6144)])
def test_x_in_registers_many_rows(gpu, oracle_mod, kind, M, N):
    # rows of one or two wave loads with x held in registers, enough rows
    # for capped grids (waves walking several rows) and ragged last passes
    # (FP16 with FP32 x from 14 rows per CU, and rows of 2-3 units from one
    # row per CU, take row slabs: their x-in-registers kernels run as
    # explicit plans in test_gpu_plans; few INT4 rows of 3 units)
    info = binding.describe_launch(kind, M, N)
    assert info["variant"] == 5, info
    ops = inputs.make(kind, M, N, seed=M ^ N)
    _check(oracle_mod, kind, ops, f"{kind} x-in-registers M={M} N={N} {info}")


@pytest.mark.parametrize("kind,N", [("q8", 16), ("q8", 48), ("q8", 272), ("q8", 512),
                                    ("q4", 128), ("q4", 384), ("q4", 640), ("q4", 1024)])
def test_packed_short_rows_many_groups(gpu, oracle_mod, kind, N):
    # rows of at most 32 chunks share wave loads (with more than 3 row
    # groups per CU): enough rows for every wave of a full grid, and a last
    # group only partly filled
    M = 14336 + 3 if N > 16 else 65536 + 3
    info = binding.describe_launch(kind, M, N)
    assert info["variant"] == 4, info
    ops = inputs.make(kind, M, N, seed=N)
    _check(oracle_mod, kind, ops, f"{kind} packed M={M} N={N} {info}")


@pytest.mark.parametrize("kind,N,M", [("q8", 512, 40000 + 1), ("q4", 1024, 40000 + 1), ("q4", 128, 140000 + 5),
                                      ("q8", 16, 600000 + 7)])
def test_packed_waves_take_two_groups(gpu, oracle_mod, kind, N, M):
    # more than 16 row groups per CU: each wave takes two groups, both in
    # flight, the last groups ragged
    nchunks = N // (16 if kind == "q8" else 32)
    R = 64 // (1 << (nchunks - 1).bit_length())
    info = binding.describe_launch(kind, M, N)
    assert info["variant"] == 4 and info["units_in_flight"] == 2 and info["rows_per_wave"] == 2 * R, info
    ops = inputs.make(kind, M, N, seed=M)
    _check(oracle_mod, kind, ops, f"{kind} packed multi-group M={M} N={N} {info}")


# ---------------------------------------------------------------- exactness
def _int_ops(kind, M, N, rng):
    x = rng.integers(-3, 4, N)
    if kind == "f32":
        return {"A": rng.integers(-3, 4, (M, N)).astype(np.float32), "x": x.astype(np.float32)}
    if kind == "f16":
        return {"A": rng.integers(-3, 4, (M, N)).astype(np.float16), "x": x.astype(np.float16)}
    if kind == "f16x32":
        return {"A": rng.integers(-3, 4, (M, N)).astype(np.float16), "x": x.astype(np.float32)}
    if kind == "f16_acc16":
        # integer sums stay below 2048 in every binary16 running sum
        # (at most 9 * ceil(N/64) <= 9 * 72), so they are exact
        return {"A": rng.integers(-3, 4, (M, N)).astype(np.float16), "x": x.astype(np.float16)}
    if kind == "q8":
        return {"A": rng.integers(-128, 128, (M, N), dtype=np.int8),
                "scale": np.full(M, 2.0 ** -7, np.float16), "x": x.astype(np.float16)}
    q = rng.integers(-8, 8, (M, N))
    g = np.arange(N // 128)
    s = np.tile((2.0 ** (g % 8 - 4)).astype(np.float16), (M, 1))
    return {"A": pack_int4(q), "scale": s, "x": x.astype(np.float16)}


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
@pytest.mark.parametrize("M,N", [(37, 1024), (8, 4096), (300, 256), (5, 1152)])
def test_integer_inputs_bit_exact(gpu, oracle_mod, kind, M, N):
    ops = _int_ops(kind, M, N, np.random.default_rng(M + N))
    say(f"[exact] {kind} M={M} N={N}")
    y = run_gpu(kind, ops)
    ref = run_oracle(oracle_mod, kind, ops)
    assert np.array_equal(y.astype(np.float64), ref), (kind, np.max(np.abs(y - ref)))


@pytest.mark.parametrize("N", [512, 4096, 1000])
def test_f16_subnormal_operands_bit_exact(gpu, oracle_mod, N):
    # A made only of binary16 subnormals k * 2^-24 (k in [-1023, 1023]) and
    # integer x: every partial sum is k' * 2^-24 with |k'| < 2^24, exact in FP32.
    rng = np.random.default_rng(N)
    M = 40
    k = rng.integers(-1023, 1024, (M, N))
    A = (np.where(k < 0, 0x8000, 0) | np.abs(k)).astype(np.uint16).view(np.float16)
    x = rng.integers(-3, 4, N).astype(np.float16)
    ops = {"A": A, "x": x}
    say(f"[subnormal A] N={N}")
    y = run_gpu("f16", ops)
    ref = run_oracle(oracle_mod, "f16", ops)
    assert np.array_equal(y.astype(np.float64), ref)
    # the same with the roles swapped: subnormal x, integer A
    ops = {"A": rng.integers(-3, 4, (M, N)).astype(np.float16), "x": A[0].copy()}
    say(f"[subnormal x] N={N}")
    assert np.array_equal(run_gpu("f16", ops).astype(np.float64), run_oracle(oracle_mod, "f16", ops))


@pytest.mark.parametrize("M,N", [(40, 1024), (9000, 1024), (24, 8192)])
def test_f16x32_full_precision_x_bit_exact(gpu, oracle_mod, M, N):
    # x = k * 2^-8 with |k| < 2^12 (up to 12 significant bits, so many values
    # are not binary16) and integer A: every product and partial sum is a
    # multiple of 2^-8 whose magnitude stays below sum_j |A_ij k_j| < 2^24
    # units, exact in FP32 in any order.  Covers x read per unit (N = 1024),
    # staged for many rows (M = 9000) and staged for long rows (N = 8192,
    # where A is drawn from {-1, 0, 1} to keep the bound).
    rng = np.random.default_rng(M + N)
    k = rng.integers(-4095, 4096, N)
    x = (k * 2.0 ** -8).astype(np.float32)
    assert np.any(x.astype(np.float16).astype(np.float32) != x)
    amax = 3 if N <= 1024 else 1
    A = rng.integers(-amax, amax + 1, (M, N))
    assert np.max(np.abs(A) @ np.abs(k)) < 2 ** 24
    ops = {"A": A.astype(np.float16), "x": x}
    say(f"[exact f16x32] M={M} N={N} {binding.describe_launch('f16x32', M, N)}")
    y = run_gpu("f16x32", ops)
    assert np.array_equal(y.astype(np.float64), run_oracle(oracle_mod, "f16x32", ops))


def test_f16x32_subnormal_weights_bit_exact(gpu, oracle_mod):
    # binary16 subnormal A (k * 2^-24) must be widened, not flushed
    rng = np.random.default_rng(17)
    M, N = 40, 4096
    k = rng.integers(-1023, 1024, (M, N))
    A = (np.where(k < 0, 0x8000, 0) | np.abs(k)).astype(np.uint16).view(np.float16)
    ops = {"A": A, "x": rng.integers(-3, 4, N).astype(np.float32)}
    say("[subnormal A] f16x32")
    assert np.array_equal(run_gpu("f16x32", ops).astype(np.float64), run_oracle(oracle_mod, "f16x32", ops))


def test_f16_acc16_is_lossy_and_within_its_bound(gpu, oracle_mod):
    # The FP16-accumulation entry point must really keep binary16 sums (its
    # error is well above the FP32-accumulating path's) and stay within the
    # derived componentwise bound.
    from gpu_util import within_gate

    ops = inputs.make("f16", 1024, 8192, seed=21)
    ref = run_oracle(oracle_mod, "f16", ops)
    say("[acc16 lossy] 1024x8192")
    y16 = run_gpu("f16_acc16", ops)
    y32 = run_gpu("f16", ops)
    rep = within_gate(oracle_mod, "f16_acc16", ops, y16, ref)
    assert rep["ok"], rep
    e16 = rep["floored_rel"]
    e32 = within_gate(oracle_mod, "f16", ops, y32, ref)["floored_rel"]
    assert e16 > 10 * e32, (e16, e32)


@pytest.mark.parametrize("kind", ["q8", "q4"])
def test_quantised_subnormal_x_bit_exact(gpu, oracle_mod, kind):
    rng = np.random.default_rng(3)
    M, N = 24, 2048
    ops = _int_ops(kind, M, N, rng)
    # |k| <= 15 keeps every partial sum below 2^24 units of its finest term
    k = rng.integers(-15, 16, N)
    ops["x"] = (np.where(k < 0, 0x8000, 0) | np.abs(k)).astype(np.uint16).view(np.float16)
    say(f"[subnormal x] {kind}")
    y = run_gpu(kind, ops)
    assert np.array_equal(y.astype(np.float64), run_oracle(oracle_mod, kind, ops))


# ---------------------------------------------------------------- layout probes
def test_q4_one_hot_columns(gpu, oracle_mod):
    # x = e_j recovers column j: pins nibble order, sign and group index
    rng = np.random.default_rng(11)
    M, N = 9, 512
    q = rng.integers(-8, 8, (M, N))
    s = np.array([[2.0 ** (g - 2 + (i % 3)) for g in range(N // 128)] for i in range(M)], np.float16)
    A, S = dev(pack_int4(q)), dev(s)
    for j in range(N):
        e = np.zeros(N, np.float16)
        e[j] = 1
        y = binding.gemv_q4(A, S, dev(e)).cpu().numpy()
        assert np.array_equal(y.astype(np.float64), q[:, j] * s[:, j // 128].astype(np.float64)), j


def test_rowmajor_one_hot_f32(gpu, oracle_mod):
    M, N = 3, 4 * 64
    A = np.arange(M * N, dtype=np.float32).reshape(M, N)
    Ad = dev(A)
    for j in (0, 1, 2, 3, 4, 255):
        e = np.zeros(N, np.float32)
        e[j] = 1
        y = binding.gemv_f32(Ad, dev(e)).cpu().numpy()
        assert list(y) == [i * N + j for i in range(M)]


# ---------------------------------------------------------------- degenerate cases
@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
def test_extreme_int_values_and_identity(gpu, oracle_mod, kind):
    n = 256
    rng = np.random.default_rng(0)
    xv = f16(rng.standard_normal(n))
    if kind == "f32":
        ops = {"A": np.eye(n, dtype=np.float32), "x": rng.uniform(-1, 1, n).astype(np.float32)}
        want = ops["x"].astype(np.float64)
    elif kind in ("f16", "f16_acc16"):
        ops = {"A": np.eye(n, dtype=np.float16), "x": xv}
        want = xv.astype(np.float64)
    elif kind == "f16x32":
        # x with 24 significant bits and outside the binary16 range: y = x
        # exactly only if x reaches the products unrounded
        x32 = (rng.uniform(-1, 1, n) * np.float32(2.0) ** rng.integers(-30, 30, n)).astype(np.float32)
        ops = {"A": np.eye(n, dtype=np.float16), "x": x32}
        want = x32.astype(np.float64)
    elif kind == "q8":
        A = np.full((n, n), -128, np.int8)        # the most negative code everywhere
        ops = {"A": A, "scale": np.full(n, 2.0 ** -7, np.float16), "x": np.ones(n, np.float16)}
        want = np.full(n, -128.0 * n * 2 ** -7)
    else:
        q = np.full((n, n), -8)
        ops = {"A": pack_int4(q), "scale": np.full((n, n // 128), 0.5, np.float16), "x": np.ones(n, np.float16)}
        want = np.full(n, -8.0 * 0.5 * n)
    say(f"[degenerate] {kind}")
    y = run_gpu(kind, ops)
    assert np.array_equal(y.astype(np.float64), want)
    assert np.array_equal(y.astype(np.float64), run_oracle(oracle_mod, kind, ops))


def _finite_rows_close(ops, kind, y, ref, rows):
    from gpu_util import abs_products

    bound = 1e-5 * abs_products(ops, kind)[rows] + 1e-30
    return np.all(np.abs(y[rows].astype(np.float64) - ref[rows]) <= bound)


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32"])
def test_special_values_follow_ieee(gpu, oracle_mod, kind):
    # NaN and infinities in A or x give exactly the definition's NaN / +-inf
    # per row (IEEE products and sums, in any order); other rows unaffected
    rng = np.random.default_rng(9)
    M, N = 8, 1024
    A = rng.uniform(-1, 1, (M, N))
    A[A == 0] = 0.5
    x = rng.uniform(0.25, 1, N)
    x[300] = 0.0
    A[1, 100] = np.nan                        # NaN
    A[2, 100] = np.inf                        # +inf
    A[3, 100], A[3, 200] = np.inf, -np.inf    # +inf - inf = NaN
    A[4, 100] = -np.inf                       # -inf
    A[5, 300] = np.inf                        # inf * 0 = NaN
    adt = np.float32 if kind == "f32" else np.float16
    xdt = np.float16 if kind == "f16" else np.float32
    cases = [("A special", {"A": A.astype(adt), "x": x.astype(xdt)}, [0, 6, 7])]
    x2 = x.copy()
    x2[400] = np.inf
    A2 = rng.uniform(-1, 1, (M, N))
    A2[A2 == 0] = 0.5
    A2[6, 400] = 0.0                          # 0 * inf = NaN; other rows +-inf
    cases.append(("x special", {"A": A2.astype(adt), "x": x2.astype(xdt)}, []))
    # a ragged last pass (N = 1000): the lanes past the row end must add
    # nothing, not 0 * x[0] = NaN when x[0] is infinite
    Nr = 1000
    A3 = rng.uniform(0.25, 1, (M, Nr))
    A3[1::2, 0] *= -1
    x3 = rng.uniform(-1, 1, Nr)
    x3[0] = np.inf
    cases.append(("ragged, x[0] = inf", {"A": A3.astype(adt), "x": x3.astype(xdt)}, []))
    for label, ops, finite in cases:
        say(f"[special values] {kind} {label}")
        y = run_gpu(kind, ops)
        ref = run_oracle(oracle_mod, kind, ops)
        assert np.array_equal(np.isnan(y), np.isnan(ref)), (label, y, ref)
        inf = np.isinf(ref)
        assert np.array_equal(y[inf].astype(np.float64), ref[inf]), (label, y, ref)
        assert np.array_equal(np.isfinite(y), np.isfinite(ref)), (label, y, ref)
        assert _finite_rows_close(ops, kind, y, ref, finite), (label, y, ref)


@pytest.mark.parametrize("kind,N", [("q8", 256), ("q8", 1024), ("q4", 512), ("q4", 2048)])
def test_quantised_special_values_are_not_finite(gpu, oracle_mod, kind, N):
    # The INT kernels factor scales out of FP32 partials, and INT8 removes a
    # 128 * sum(x) offset, so a non-finite scale or x gives a non-finite row,
    # though not always the definition's own choice between NaN and inf
    # (an infinite x entry meets the offset as inf - inf); a NaN always
    # stays NaN, and rows without special values are unaffected.
    M = 8
    ops = inputs.make(kind, M, N, seed=N)
    if kind == "q8":
        ops["scale"][2] = np.inf
        ops["scale"][3] = np.nan
    else:
        ops["scale"][2, 1] = np.inf
        ops["scale"][3, 0] = np.nan
    say(f"[special scales] {kind} N={N}")
    y = run_gpu(kind, ops)
    ref = run_oracle(oracle_mod, kind, ops)
    assert not np.isfinite(y[2]) and not np.isfinite(ref[2])
    assert np.isnan(y[3]) and np.isnan(ref[3])
    rows = [0, 1, 4, 5, 6, 7]
    assert np.all(np.isfinite(y[rows])) and _finite_rows_close(ops, kind, y, ref, rows)
    for v, want_nan in ((np.inf, False), (np.nan, True)):
        ops = inputs.make(kind, M, N, seed=N + 1)
        ops["x"][10] = v
        say(f"[special x] {kind} N={N} x={v}")
        y = run_gpu(kind, ops)
        assert not np.any(np.isfinite(y)), y
        if want_nan:
            assert np.all(np.isnan(y)) and np.all(np.isnan(run_oracle(oracle_mod, kind, ops)))


def test_nan_propagates(gpu, oracle_mod):
    A = np.ones((8, 1024), np.float32)
    A[3, 100] = np.nan
    y = run_gpu("f32", {"A": A, "x": np.ones(1024, np.float32)})
    assert np.isnan(y[3]) and np.all(y[[0, 1, 2, 4, 5, 6, 7]] == 1024)


# ---------------------------------------------------------------- brute force over small shapes
@pytest.mark.parametrize("M,N,variant", [((1 << 24) + (1 << 20) + 3, 3, 3), ((1 << 26) + 1000, 8, 2)])
def test_grids_past_the_dispatch_limit(gpu, oracle_mod, M, N, variant):
    # so many rows that one wave per row (element-wise path), or four rows
    # per wave, would pass 2^30 work-items: the grid is capped and the waves
    # walk the rest.  Integer-valued operands make every order exact, so the
    # sampled rows (both ends, the first rows past the grid, random others)
    # must match bit for bit.
    info = binding.describe_launch("f16", M, N)
    assert info["variant"] == variant, info
    assert info["grid"] * info["block"] <= 1 << 30, info
    assert info["rows_per_wave"] >= 2, info
    rng = np.random.default_rng(M)
    A = rng.integers(-3, 4, size=(M, N), dtype=np.int8).astype(np.float16)
    x = rng.integers(-3, 4, size=N, dtype=np.int8).astype(np.float16)
    say(f"[parity] f16 M={M} N={N} past the dispatch limit {info}")
    y = binding.gemv_f16(dev(A), dev(x))
    torch.cuda.synchronize()
    first_walk = info["grid"] * info["block"] // 64   # waves take rows w, w + waves, ...
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M),
                                     np.arange(first_walk - 32, min(first_walk + 32, M)),
                                     rng.integers(0, M, 4096)]))
    got = y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    want = oracle_mod.gemv_f16(np.ascontiguousarray(A[rows]), x)
    assert np.array_equal(got, want)


def test_rows_of_two_gibibytes(gpu, oracle_mod):
    # FP16 rows of 2^30 + 8 columns (2 GiB + 16 bytes): past a 32-bit byte
    # count, so the element-wise kernel with 64-bit offsets runs.  Sparse
    # integer entries near both ends of each row and past the 2^31-byte mark
    # of the second row make the sums exact and any offset slip visible.
    M, N = 2, (1 << 30) + 8
    info = binding.describe_launch("f16", M, N)
    assert info["variant"] == 3, info
    A = np.zeros((M, N), np.float16)
    cols = [0, 1, (1 << 29) + 3, (1 << 30) - 1, (1 << 30) + 7]
    for i in range(M):
        for k, j in enumerate(cols):
            A[i, j] = (i + 1) * (k + 1) * (-1) ** k
    x = np.ones(N, np.float16)
    x[cols[2]] = 2.0
    say(f"[parity] f16 M={M} N={N} rows of 2 GiB {info}")
    y = binding.gemv_f16(dev(A), dev(x))
    torch.cuda.synchronize()
    want = np.array([sum(float(A[i, j]) * float(x[j]) for j in cols) for i in range(M)])
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want)
    # the oracle agrees on a column slice holding every nonzero term's
    # neighbourhood (the full rows would take it minutes)
    sl = np.r_[0:64, (1 << 29):(1 << 29) + 64, (1 << 30) - 64:N]
    assert np.array_equal(oracle_mod.gemv_f16(np.ascontiguousarray(A[:, sl]), np.ascontiguousarray(x[sl])), want)


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "q8", "q4"])
def test_brute_force_small_shapes(gpu, oracle_mod, kind):
    # every N in 1..300 (odd, below one wave's width, not a multiple of the
    # chunk width) for several M up to 17; INT4 takes its whole-group N only
    # With M this small the floored relative error cannot absorb cancellation
    # in a single output, so the gate here is the componentwise FP32 bound;
    # a dropped or misplaced term exceeds it.
    from gpu_util import within_fp32_bound

    Ns = [128, 256] if kind == "q4" else list(range(1, 301))
    say(f"[brute force] {kind} N=1..300")
    for N in Ns:
        for M in (1, 2, 3, 5, 8, 13, 17):
            ops = inputs.make(kind, M, N, seed=M * 1000 + N)
            y = run_gpu(kind, ops)
            ref = run_oracle(oracle_mod, kind, ops)
            r = within_fp32_bound(kind, ops, y, ref)
            assert r <= 1.0, (kind, M, N, r)
