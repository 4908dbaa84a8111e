"""GPU checks of the row-slab kernel (gemv_slab, plan variant 7): a
workgroup of S waves takes 4 or 8 rows at a time, each wave one or two
passes of every row with its x slice in registers, the wave sums of a row
added in LDS.  Against the CPU oracle at the format's gate and within the
FP32 summation bound, through the planner and through explicit plans: both
pass counts per wave, both slab sizes, both depths, grids that make
workgroups walk several slabs, slabs cut short by the last row, and rows
ending in a ragged pass.  Integer-valued operands make every summation
order exact, so those cases must match the oracle bit for bit."""
import numpy as np
import pytest
import torch

from memory_bound_gemv_row_amd import binding, inputs

from gpu_util import dev, run_gpu, run_oracle, say, within_fp32_bound, within_gate

pytestmark = pytest.mark.gpu

_ELEMS = {"q8": 16, "q4": 32, "f16x32": 8}


def _launch(kind, ops, plan):
    M = ops["A"].shape[0]
    N = ops["x"].shape[0]
    A, x = dev(ops["A"]), dev(ops["x"])
    scale = dev(ops["scale"]) if "scale" in ops else None
    y = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    rc = binding.launch_plan_ptr(kind, A.data_ptr(), scale.data_ptr() if scale is not None else 0, x.data_ptr(),
                                 y.data_ptr(), M, N, plan, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, (kind, M, N, plan, rc)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _plans(kind, M, N, caps=(0, 1)):
    props = torch.cuda.get_device_properties(0)
    P = -(-(N // _ELEMS[kind]) // 64)
    out = []
    for S in sorted({P, P // 2}):
        for D in (4, 8):
            for R in (4, 8):
                for cap in caps:
                    plan = (7, S, D, R, -1, cap)
                    if binding.check_plan_for(kind, M, N, props.multi_processor_count,
                                              props.shared_memory_per_block, plan) is not None:
                        out.append(plan)
    return out


# (kind, M, N): rows of 8, 4, 16 and 9 units (one and two passes per wave),
# ragged last passes, a last slab cut short, and fewer rows than one slab
_SHAPES = [("q8", 3001, 8176), ("q8", 5, 8208), ("q4", 3003, 8064), ("q4", 3, 16512), ("f16x32", 2002, 8000),
           ("f16x32", 7, 4104)]


@pytest.mark.parametrize("case", _SHAPES, ids=lambda c: f"{c[0]}_{c[1]}x{c[2]}")
def test_every_slab_plan_matches_the_oracle(gpu, oracle_mod, case):
    kind, M, N = case
    ops = inputs.make(kind, M, N, seed=M + 5 * N)
    ref = run_oracle(oracle_mod, kind, ops)
    plans = _plans(kind, M, N)
    assert len(plans) >= 4, plans
    same = {}
    for plan in plans:
        label = f"{kind} {M}x{N} plan {plan}"
        say(f"[slab] {label}")
        y = _launch(kind, ops, plan)
        rep = within_gate(oracle_mod, kind, ops, y, ref)
        assert rep["ok"], (label, rep)
        assert within_fp32_bound(kind, ops, y, ref) <= 1.0, label
        # depth and grid cap leave each lane's order and the reduction as they are
        key = (plan[1], plan[3])
        if key in same:
            assert np.array_equal(y, same[key]), label
        same.setdefault(key, y)


@pytest.mark.parametrize("kind,M,N", [("q4", 40000 + 3, 8192), ("q4", 4096, 14336), ("f16x32", 8192, 8192),
                                      ("f16x32", 4096, 14336), ("q8", 2295, 24576), ("q8", 1913, 10240 - 16)])
def test_planner_slabs(gpu, oracle_mod, kind, M, N):
    # the planner's row slabs at the named shapes and beyond: INT4 with the
    # grid capped at 32 waves per CU (workgroups walk several slabs), two
    # passes per wave in slabs of 8 rows (FP16 with FP32 x 4096x14336) and of
    # 4 (INT8 rows of 24 units), a ragged last pass (INT8 rows of 10 units)
    info = binding.describe_launch(kind, M, N)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert info["variant"] == 7, info
    ops = inputs.make(kind, M, N, seed=M ^ N)
    label = f"{kind} {M}x{N} {info}"
    say(f"[slab planner] {label}")
    y = run_gpu(kind, ops)
    ref = run_oracle(oracle_mod, kind, ops)
    rep = within_gate(oracle_mod, kind, ops, y, ref)
    assert rep["ok"], (label, rep)
    assert within_fp32_bound(kind, ops, y, ref) <= 1.0, label


@pytest.mark.parametrize("kind,M,N", [("q8", 1003, 8176), ("q4", 1001, 8064), ("f16x32", 1002, 8000),
                                      ("q8", 601, 8208)])
def test_integer_inputs_bit_exact(gpu, oracle_mod, kind, M, N):
    # integer codes and x, power-of-two scales: every partial sum is exact,
    # so every slab plan must give the oracle's y bit for bit
    rng = np.random.default_rng(M + N)
    x = rng.integers(-3, 4, N).astype(np.float16)
    if kind == "q8":
        ops = {"A": rng.integers(-128, 128, (M, N), dtype=np.int8), "scale": np.full(M, 2.0 ** -7, np.float16), "x": x}
    elif kind == "q4":
        ops = {"A": rng.integers(0, 256, (M, N // 2), dtype=np.uint8),
               "scale": (2.0 ** (np.arange(N // 128) % 8 - 4)).astype(np.float16)[None, :].repeat(M, 0), "x": x}
    else:
        ops = {"A": rng.integers(-8, 9, (M, N)).astype(np.float16), "x": x.astype(np.float32)}
    ref = run_oracle(oracle_mod, kind, ops)
    for plan in _plans(kind, M, N):
        say(f"[slab exact] {kind} {M}x{N} plan {plan}")
        y = _launch(kind, ops, plan)
        assert np.array_equal(y.astype(np.float64), ref), (kind, M, N, plan, float(np.max(np.abs(y - ref))))
