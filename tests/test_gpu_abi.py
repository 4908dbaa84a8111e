"""GPU checks of the C-ABI contract: status codes, degenerate sizes, output
bounds, streams, determinism, unaligned operands and the probes."""
import numpy as np
import pytest
import torch

from memory_bound_gemv_row_amd import binding, inputs

from gpu_util import dev, run_gpu, run_oracle, say, within_gate
from oracle.metrics import GATES, parity_error

pytestmark = pytest.mark.gpu


def _ptrs(kind, ops):
    A = dev(ops["A"])
    x = dev(ops["x"])
    s = dev(ops["scale"]) if "scale" in ops else None
    return A, s, x


def _call(kind, A, s, x, y, M, N, stream=0):
    if kind == "f32":
        return binding.gemv_f32_ptr(A, x, y, M, N, stream)
    if kind == "f16":
        return binding.gemv_f16_ptr(A, x, y, M, N, stream)
    if kind == "f16x32":
        return binding.gemv_f16x32_ptr(A, x, y, M, N, stream)
    if kind == "f16_acc16":
        return binding.gemv_f16_acc16_ptr(A, x, y, M, N, stream)
    if kind == "q8":
        return binding.gemv_q8_ptr(A, s, x, y, M, N, stream)
    return binding.gemv_q4_ptr(A, s, x, y, M, N, stream)


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
def test_status_codes(gpu, kind):
    M, N = 8, 256
    A, s, x = _ptrs(kind, inputs.make(kind, M, N))
    y = torch.zeros(M, device="cuda")
    sp = s.data_ptr() if s is not None else 0
    a, xp, yp = A.data_ptr(), x.data_ptr(), y.data_ptr()
    say(f"[status] {kind}")
    assert _call(kind, a, sp, xp, yp, -1, N) == 1
    assert _call(kind, a, sp, xp, yp, M, -5) == 1
    assert _call(kind, a, sp, xp, 0, M, N) == 1
    assert _call(kind, 0, sp, xp, yp, M, N) == 1
    assert _call(kind, a, sp, 0, yp, M, N) == 1
    if kind in ("q8", "q4"):
        assert _call(kind, a, 0, xp, yp, M, N) == 1
    assert _call(kind, 0, 0, 0, 0, 0, N) == 0          # M == 0: nothing to do
    if kind == "q4":
        assert _call(kind, a, sp, xp, yp, M, 200) == 2   # partial 128-column group
    torch.cuda.synchronize()
    assert torch.all(y == 0)                            # rejected calls wrote nothing
    with pytest.raises(ValueError):     # the binding checks shapes before the call
        binding.gemv_f32(torch.zeros(4, 4, device="cuda"), torch.zeros(5, device="cuda"))


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
def test_n_zero_writes_zeros(gpu, kind):
    M = 70
    y = torch.full((M,), 7.0, device="cuda")
    A = torch.zeros(16, dtype=torch.uint8, device="cuda")
    scale = torch.full((M,), float("inf"), dtype=torch.float16, device="cuda")   # must not matter
    say(f"[N=0] {kind}")
    assert _call(kind, A.data_ptr(), scale.data_ptr(), A.data_ptr(), y.data_ptr(), M, 0) == 0
    assert _call(kind, 0, 0, 0, y.data_ptr(), M, 0) == 0      # nothing is read when N == 0
    torch.cuda.synchronize()
    assert torch.all(y == 0)


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
def test_writes_only_y_0_to_M(gpu, oracle_mod, kind):
    M, N = 37, 1024
    ops = inputs.make(kind, M, N, seed=2)
    A, s, x = _ptrs(kind, ops)
    guard = torch.full((M + 128,), 12345.0, device="cuda")
    y = guard[64:64 + M]
    say(f"[canary] {kind}")
    assert _call(kind, A.data_ptr(), s.data_ptr() if s is not None else 0, x.data_ptr(), y.data_ptr(), M, N) == 0
    torch.cuda.synchronize()
    g = guard.cpu().numpy()
    assert np.all(g[:64] == 12345.0) and np.all(g[64 + M:] == 12345.0)
    assert within_gate(oracle_mod, kind, ops, g[64:64 + M], run_oracle(oracle_mod, kind, ops))["ok"]


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
def test_repeat_runs_bitwise_identical(gpu, kind):
    ops = inputs.make(kind, 1000, 4096, seed=4)
    say(f"[determinism] {kind}")
    ys = [run_gpu(kind, ops) for _ in range(3)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def test_non_default_stream(gpu, oracle_mod):
    ops = inputs.make("f16", 2048, 4096, seed=6)
    A, _, x = _ptrs("f16", ops)
    s = torch.cuda.Stream()
    y = torch.empty(2048, device="cuda")
    torch.cuda.synchronize()
    say("[stream]")
    with torch.cuda.stream(s):
        binding.gemv_f16(A, x, out=y)          # binding passes the current stream
    s.synchronize()
    assert parity_error(y.cpu().numpy(), run_oracle(oracle_mod, "f16", ops)) <= GATES["f16"]


@pytest.mark.parametrize("kind", ["f32", "f16", "f16x32", "f16_acc16", "q8", "q4"])
@pytest.mark.parametrize("offset", [2, 4, 8])
def test_unaligned_operands(gpu, oracle_mod, kind, offset):
    """A and x at byte offsets that break 16-byte alignment take the
    element-wise path and still agree with the oracle."""
    M, N = 33, 1024
    ops = inputs.make(kind, M, N, seed=offset)
    elt = {"f32": 4, "f16": 2, "f16x32": 4, "f16_acc16": 2, "q8": 1, "q4": 1}[kind]   # natural alignment of x
    if offset % elt:
        pytest.skip("offset not a multiple of the element size")
    Ab = ops["A"].view(np.uint8).ravel()
    xb = ops["x"].view(np.uint8).ravel()
    bufA = torch.zeros(Ab.size + 64, dtype=torch.uint8, device="cuda")
    bufx = torch.zeros(xb.size + 64, dtype=torch.uint8, device="cuda")
    bufA[offset:offset + Ab.size] = dev(Ab)
    bufx[offset:offset + xb.size] = dev(xb)
    s = dev(ops["scale"]) if "scale" in ops else None
    y = torch.empty(M, device="cuda")
    say(f"[unaligned] {kind} +{offset}")
    rc = _call(kind, bufA.data_ptr() + offset, s.data_ptr() if s is not None else 0,
               bufx.data_ptr() + offset, y.data_ptr(), M, N)
    assert rc == 0
    torch.cuda.synchronize()
    assert within_gate(oracle_mod, kind, ops, y.cpu().numpy(), run_oracle(oracle_mod, kind, ops))["ok"]


def test_describe_launch_fills_all_cus(gpu):
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    for kind, M, N in (("f32", 1024, 1024), ("f16", 8192, 8192), ("q4", 4096, 14336), ("q4", 14336, 4096),
                       ("f16x32", 8192, 8192), ("f16x32", 4096, 14336), ("f16x32", 14336, 4096),
                       ("f16x32", 4096, 4096)):
        info = binding.describe_launch(kind, M, N)
        assert info["grid"] >= cus, (kind, M, N, info, cus)
    assert binding.describe_launch("f16", 8, 1001)["variant"] == 3
    # INT8/INT4 rows whose staged x passes 64 KiB: staged while it fits a
    # workgroup's LDS and the rows are many, else x read with each unit
    lds_max = props.shared_memory_per_block
    assert binding.describe_launch("q8", 4096, 31744)["variant"] == 1
    assert binding.describe_launch("q8", 4096, 34816)["variant"] == 1   # (rows of 32 units: row slabs)
    assert binding.describe_launch("q4", 4096, 34816)["variant"] == 1
    assert binding.describe_launch("q4", 1024, 33280)["variant"] == 2
    q8_beyond = lds_max // 2048 * 1024 + 1024            # one unit past what fits
    q4_beyond = lds_max // 4096 * 2048 + 2048
    assert binding.describe_launch("q8", 4096, q8_beyond)["variant"] == 2
    assert binding.describe_launch("q4", 4096, q4_beyond)["variant"] == 2
    for kind, M, N in (("q8", 4096, 34816), ("q4", 4096, 34816), ("q8", 1024, 32768)):
        info = binding.describe_launch(kind, M, N)
        assert info["variant"] == 2 or info["lds_bytes"] <= lds_max, (kind, M, N, info)
    # INT8/INT4 rows of at most 32 chunks: the packed short-row kernel
    assert binding.describe_launch("q8", 14336, 512)["variant"] == 4
    assert binding.describe_launch("q4", 14336, 1024)["variant"] == 4
    # one-unit rows just past that: x in registers; two-unit rows: staged
    assert binding.describe_launch("q8", 14336, 528)["variant"] == 5
    assert binding.describe_launch("q4", 1000, 1152)["variant"] == 5
    assert binding.describe_launch("q4", 14336, 1152)["variant"] == 7   # from 4 rows per CU: row slabs
    assert binding.describe_launch("q8", 14336, 1040)["variant"] == 1
    assert binding.describe_launch("q4", 14336, 2176)["variant"] == 1
    # FP rows of one unit (up to 32 rows per CU) and of two units: x in registers
    assert binding.describe_launch("f16", 4096, 512)["variant"] == 5
    assert binding.describe_launch("f16", 14336, 1024)["variant"] == 5
    assert binding.describe_launch("f32", 14336, 256)["variant"] == 2
    assert binding.describe_launch("f16x32", 3000, 512)["variant"] == 5
    assert binding.describe_launch("f16x32", 200, 1024)["variant"] == 2
    # FP16 with FP32 x from one row per CU (one-unit rows from 14 per CU):
    # row slabs, x slices in registers
    assert binding.describe_launch("f16x32", 14336, 512)["variant"] == 7
    assert binding.describe_launch("f16x32", 4096, 1024)["variant"] == 7
    assert binding.describe_launch("f16", 14336, 1536)["variant"] == 5
    assert binding.describe_launch("q8", 4096, 3072)["variant"] == 1   # INT8 three-unit rows stay staged
    # more than 2^30 rows: the row-walking kernels' int cursors could wrap,
    # so the element-wise kernel (64-bit row indices) takes the call
    for kind in ("f16", "q8", "q4"):
        assert binding.describe_launch(kind, (1 << 30) + 1, 128)["variant"] == 3
        assert binding.describe_launch(kind, 1 << 30, 128)["variant"] != 3
    # FP16 A with FP32 x: row slabs for rows of up to 16 units (and an even
    # count up to 32); longer rows staged in LDS for many rows, read with
    # each unit otherwise, and never staged beyond what a workgroup may hold
    assert binding.describe_launch("f16x32", 8192, 8192)["variant"] == 7
    assert binding.describe_launch("f16x32", 14336, 4096)["variant"] == 7
    assert binding.describe_launch("f16x32", 4096, 4096)["variant"] == 7
    assert binding.describe_launch("f16x32", 8 * cus, 4096)["variant"] == 7
    info = binding.describe_launch("f16x32", 16 * cus, 32768)
    assert info["variant"] == 1 and info["lds_bytes"] == 4 * 32768 + 1024 <= lds_max, info   # x and spare granules
    assert binding.describe_launch("f16x32", 16 * cus, lds_max // 4 + 512)["variant"] == 2
    # few long rows (up to 5 per CU for rows of 16 units and more; shorter
    # ones from one row per CU take row slabs): split rows, x read with each
    # unit; two waves per row from one row per CU, below that enough waves
    # to fill the chip
    for M, N in ((cus, 32768), (4 * cus, 32768), (5 * cus, 32768), (cus, 4096 * 9)):
        info = binding.describe_launch("f16x32", M, N)
        assert info["variant"] == 6 and info["block"] == 128 and info["lds_bytes"] == 0 and info["grid"] == M, info
    info = binding.describe_launch("f16x32", 64, 32768)
    assert info["variant"] == 6 and info["grid"] * info["block"] // 64 >= 4 * cus, info
    assert binding.describe_launch("f16x32", 6 * cus, 32768)["variant"] == 1
    # few INT8 rows of four units or more (up to 6 per CU): split rows; a few
    # more: x read with each unit; few INT4 rows of six units (others take
    # row slabs) read x with each unit
    assert binding.describe_launch("q8", 6 * cus, 8192)["variant"] == 6
    assert binding.describe_launch("q8", 6 * cus + 1, 8192)["variant"] == 2
    assert binding.describe_launch("q4", 4 * cus, 12288)["variant"] == 2
    assert binding.describe_launch("q4", 4 * cus + 1, 12288)["variant"] == 1


def test_launches_stay_within_the_dispatch_limit(gpu):
    # a dispatch counts work-items in 32 bits: every plan keeps grid x block
    # at or below 2^30, the waves walking any rows beyond
    for kind in ("f32", "f16", "f16x32", "f16_acc16", "q8", "q4"):
        for M in (1 << 22, 1 << 24, (1 << 26) + 7, 1 << 28, 1 << 30):
            for N in (3, 8, 16, 128, 512, 1024, 4096, 65536):
                if kind == "q4" and N % 128:
                    continue
                info = binding.describe_launch(kind, M, N)
                assert 1 <= info["grid"] and info["grid"] * info["block"] <= 1 << 30, (kind, M, N, info)


def test_describe_launch_for_matches_the_device(gpu):
    # the device-free planner, given this device's CU count and LDS per
    # workgroup, reports exactly the plan the library launches
    props = torch.cuda.get_device_properties(0)
    cus, lds_max = props.multi_processor_count, props.shared_memory_per_block
    for kind in ("f32", "f16", "f16x32", "f16_acc16", "q8", "q4"):
        for M in (1, 1000, 1792, 4096, 8192, 14336, 100000):
            for N in (128, 512, 1024, 4096, 8192, 14336, 34816, 81920):
                assert binding.describe_launch(kind, M, N) == binding.describe_launch_for(kind, M, N, cus, lds_max)


def test_probe_copy_and_read(gpu):
    n = 64 << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    say("[probe]")
    binding.probe_copy(src, dst)
    binding.probe_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert binding.probe_read_ptr(src.data_ptr() + 4, 1024, sink.data_ptr()) == 1   # misaligned
    assert binding.probe_read_ptr(src.data_ptr(), 1000, sink.data_ptr()) == 1       # not a multiple of 16
