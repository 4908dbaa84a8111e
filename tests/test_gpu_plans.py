"""GPU checks of gemv_launch_plan (explicit launch plans): every plan the
plan search tries that the library accepts for a shape -- each kernel
variant, waves per workgroup, loads in flight, rows per wave, staging order
and grid cap -- against the CPU oracle at the format's gate, and bit for bit
against the planner's own launch wherever the plan keeps each lane's
summation order (all but split rows and row slabs, whose waves add partial
sums of a row; row slabs of one waves-per-workgroup and rows-per-slab
choice match each other bit for bit).  The shapes end in a ragged last
pass, and the row-slab shapes in a ragged last slab."""
import numpy as np
import pytest
import torch

import bench
from memory_bound_gemv_row_amd import binding, inputs

from gpu_util import dev, run_gpu, run_oracle, say, within_gate

pytestmark = pytest.mark.gpu

# (FP16 with FP32 x at 300 x 16872: rows of 33 units, long enough for split
# rows of up to 16 waves, which its own planner no longer picks)
_SHAPES = [("f32", 1100, 2052), ("f16", 1100, 4104), ("f16x32", 900, 4104), ("f16x32", 300, 16872),
           ("f16_acc16", 600, 4104),
           ("q8", 1100, 8208), ("q4", 1100, 16512), ("q8", 3000, 512), ("q4", 3000, 1024),
           ("f16", 3000, 1024), ("f16", 2000, 1536), ("f16x32", 3000, 1016), ("f16x32", 3000, 1536),
           ("q8", 1003, 8176), ("q4", 1001, 8064), ("f16x32", 1002, 8000)]


@pytest.mark.parametrize("case", _SHAPES, ids=lambda c: f"{c[0]}_{c[1]}x{c[2]}")
def test_every_accepted_plan_matches(gpu, oracle_mod, case):
    kind, M, N = case
    props = torch.cuda.get_device_properties(0)
    ops = inputs.make(kind, M, N, seed=M + N)
    ref = run_oracle(oracle_mod, kind, ops)
    info = binding.describe_launch(kind, M, N)
    own = run_gpu(kind, ops) if info["variant"] not in (6, 7) else None   # the planner's launch, if it keeps lane order
    A, x = dev(ops["A"]), dev(ops["x"])
    scale = dev(ops["scale"]) if "scale" in ops else None
    y = torch.empty(M, dtype=torch.float32, device="cuda")
    tried = 0
    slabs = {}
    for plan in bench.plan_candidates(kind, N):
        if binding.check_plan_for(kind, M, N, props.multi_processor_count, props.shared_memory_per_block,
                                  plan) is None:
            continue
        say(f"[plans] {kind} {M}x{N} plan {plan}")
        y.fill_(float("nan"))
        rc = binding.launch_plan_ptr(kind, A.data_ptr(), scale.data_ptr() if scale is not None else 0,
                                     x.data_ptr(), y.data_ptr(), M, N, plan, torch.cuda.current_stream().cuda_stream)
        assert rc == 0, (plan, rc)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        rep = within_gate(oracle_mod, kind, ops, got, ref)
        assert rep["ok"], (kind, M, N, plan, rep)
        if plan[0] == 7:
            # row slabs: the same lane order for every depth and grid cap of
            # one (waves, rows per slab)
            key = (plan[1], plan[3])
            if key in slabs:
                assert np.array_equal(got, slabs[key]), (kind, M, N, plan)
            slabs.setdefault(key, got.copy())
        elif plan[0] != 6:
            if own is None:
                own = got.copy()
            assert np.array_equal(got, own), (kind, M, N, plan, float(np.max(np.abs(got - own))))
        tried += 1
    assert tried >= 10, tried


def test_launch_plan_rejects_what_it_cannot_run(gpu):
    A = torch.zeros((64, 4096), dtype=torch.float16, device="cuda")
    x = torch.zeros(4096, dtype=torch.float16, device="cuda")
    y = torch.zeros(64, dtype=torch.float32, device="cuda")
    h = torch.cuda.current_stream().cuda_stream
    ok = (2, 4, 4, 1, -1, 0)
    assert binding.launch_plan_ptr("f16", A.data_ptr(), 0, x.data_ptr(), y.data_ptr(), 64, 4096, ok, h) == 0
    # no kernel for this plan; a misaligned A; a null y
    assert binding.launch_plan_ptr("f16", A.data_ptr(), 0, x.data_ptr(), y.data_ptr(), 64, 4096,
                                   (1, 4, 4, 1, 0, 0), h) == 2
    assert binding.launch_plan_ptr("f16", A.data_ptr() + 2, 0, x.data_ptr(), y.data_ptr(), 64, 4088, ok, h) == 1
    assert binding.launch_plan_ptr("f16", A.data_ptr(), 0, x.data_ptr(), 0, 64, 4096, ok, h) == 1
    torch.cuda.synchronize()
