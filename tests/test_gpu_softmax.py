"""GPU parity of the row softmax against the CPU oracle, through the C ABI.

The output is binary16, compared with the oracle's double result relative to
max(|reference|, 1e-4), gate 2e-3 ("membound", section "Bonus kernel:
online softmax", scores the same way)."""
import numpy as np
import pytest
import torch

from memory_bound_gemv_row_amd import binding, inputs
from oracle.metrics import SOFTMAX_GATE, softmax_error

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _run(x):
    y = binding.softmax_f16(dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _check(oracle, x, label):
    say(f"[softmax] {label}")
    y = _run(x)
    err = softmax_error(y, oracle.softmax_f16(x))
    assert err <= SOFTMAX_GATE, (label, err)
    return y, err


@pytest.mark.parametrize("M,N", inputs.SOFTMAX_WORKLOADS, ids=lambda v: str(v))
def test_full_size(gpu, oracle_mod, M, N):
    x = inputs.make_logits(M, N, seed=0)
    y, err = _check(oracle_mod, x, f"{M}x{N} seed 0")
    assert np.all(np.abs(y.sum(axis=1) - 1.0) < 2e-3)


# P = ceil(N / 512) units per row: 16 | 17, 32 | 33, 64 | 65, 128 | 129,
# 256 (all in registers) | 257 (read twice); N % 8 != 0 -> element-wise
_NS = [1, 7, 8, 16, 504, 512, 520, 8192, 8200, 16384, 16392, 32768, 32776, 65536, 65544, 131072, 131080, 140000]


def test_shapes_and_tails(gpu, oracle_mod):
    for N in _NS:
        for M in ([1, 3, 37] if N <= 32776 else [1, 5]):
            rng = np.random.default_rng(M * 7919 + N)
            x = (rng.standard_normal((M, N)) * rng.uniform(0.5, 6)).astype(np.float16)
            _check(oracle_mod, x, f"M={M} N={N}")


@pytest.mark.parametrize("N", [2056, 8200, 24584])
def test_workgroups_walk_several_rows(gpu, oracle_mod, N):
    # more rows than workgroups, so each workgroup loads its next row while
    # it stores the current one (ragged last units padded with -inf); some
    # rows hold special values, so a prefetched row may be all -inf or NaN
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = 16 * cus * 2 + 3 if N <= 16384 else 3 * cus * 3 + 5
    rng = np.random.default_rng(N)
    x = (rng.standard_normal((M, N)) * 3).astype(np.float16)
    x[5] = -np.inf
    x[6, 100] = np.nan
    x[7, :N // 2] = -np.inf
    y, _ = _check(oracle_mod, x, f"M={M} N={N} several rows per workgroup")
    assert np.all(np.isnan(y[5])) and np.all(np.isnan(y[6])) and np.all(y[7, :N // 2] == 0)


def test_special_values(gpu, oracle_mod):
    N = 1024
    x = np.zeros((6, N), np.float16)
    x[0] = -np.inf                                  # no finite entry: NaN row
    x[1, 7] = np.inf                                # +inf: NaN row
    x[2, 9] = np.nan                                # NaN: NaN row
    x[3, :500] = -np.inf                            # masked entries: exact zeros
    x[4] = np.linspace(60000, -60000, N)            # large logits, no overflow
    x[5, 0] = 20.0                                  # one dominant entry: subnormal outputs elsewhere
    y, _ = _check(oracle_mod, x, "special values")
    assert np.all(np.isnan(y[:3]))
    assert np.all(y[3, :500] == 0)


def test_unaligned_takes_elementwise_path(gpu, oracle_mod):
    M, N = 5, 1024
    x = inputs.make_logits(M, N, seed=3)
    buf = torch.zeros(M * N + 16, dtype=torch.float16, device="cuda")
    buf[1:1 + M * N] = dev(x.ravel())
    out = torch.zeros(M * N + 16, dtype=torch.float16, device="cuda")
    say("[softmax unaligned]")
    assert binding.softmax_f16_ptr(buf.data_ptr() + 2, out.data_ptr() + 2, M, N) == 0
    torch.cuda.synchronize()
    y = out[1:1 + M * N].cpu().numpy().astype(np.float64).reshape(M, N)
    assert softmax_error(y, oracle_mod.softmax_f16(x)) <= SOFTMAX_GATE
    assert out[0].item() == 0 and torch.all(out[1 + M * N:] == 0)   # nothing written outside y


def test_status_codes_and_determinism(gpu):
    x = dev(inputs.make_logits(64, 4096, seed=1))
    y = torch.empty_like(x)
    say("[softmax status]")
    assert binding.softmax_f16_ptr(x.data_ptr(), y.data_ptr(), -1, 4096) == 1
    assert binding.softmax_f16_ptr(0, y.data_ptr(), 64, 4096) == 1
    assert binding.softmax_f16_ptr(x.data_ptr(), 0, 64, 4096) == 1
    assert binding.softmax_f16_ptr(0, 0, 0, 4096) == 0
    assert binding.softmax_f16_ptr(0, 0, 64, 0) == 0
    a = binding.softmax_f16(x).clone()
    b = binding.softmax_f16(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_elementwise_grid_past_the_dispatch_limit(gpu, oracle_mod):
    # rows of 7 logits take the element-wise kernel, one wave per row:
    # 2^24 + 5 rows would pass 2^30 work-items, so the grid is capped and the
    # waves walk the rest; sampled rows (both ends, the first walked rows,
    # random others) are checked against the oracle
    M, N = (1 << 24) + 5, 7
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((M, N)) * 3).astype(np.float16)
    say(f"[softmax] M={M} N={N} past the dispatch limit")
    y = _run(x)
    nwaves = (1 << 30) // 64
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), np.arange(nwaves - 32, nwaves + 5),
                                     rng.integers(0, M, 4096)]))
    assert softmax_error(y[rows], oracle_mod.softmax_f16(np.ascontiguousarray(x[rows]))) <= SOFTMAX_GATE
