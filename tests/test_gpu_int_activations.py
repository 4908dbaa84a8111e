"""GPU parity of the INT8/INT4 paths on activations and codes beyond the
workloads' zero-mean N(0, 1) x and uniform codes.

Decode hidden states after an activation are non-negative or off-centre, and
absmax-quantised Gaussian weights put most codes near zero (more so when an
outlier sets the row's scale).  The kernels form each product q*x exactly
and accumulate in FP32 ("membound", section "The kernel decode actually
runs: dequant GEMV": the reference weight is exactly q*s, FP32 accumulate),
so the error must not depend on the mean of x or on where the codes sit.
Every case runs at the shapes that reach each INT8/INT4 plan: staged x
(8192^2, 14336x4096), x read per unit (1792x4096), x in registers (INT8
rows of one unit: 4096x1024), packed short rows (14336x512) and row slabs
(INT4 4096x14336 and one-unit rows of 64 chunks, 4096x2048; INT8 rows of 10
and of 24 units, two passes per wave).  Codes made from Gaussian weights come from the oracle's
quantiser, never from the GPU's.
"""
import numpy as np
import pytest

from memory_bound_gemv_row_amd import binding, inputs

from gpu_util import run_gpu, run_oracle, say, within_fp32_bound, within_gate

pytestmark = pytest.mark.gpu

_SHAPES = {
    "q8": [(8192, 8192), (14336, 4096), (1792, 4096), (4096, 1024), (14336, 512), (1913, 10240), (2295, 24576)],
    "q4": [(4096, 14336), (14336, 4096), (1792, 4096), (4096, 2048), (14336, 512)],
}
_WEIGHTS = ("codes", "gauss", "outlier")


def _operands(oracle, kind, M, N, weights, seed):
    if weights == "codes":
        ops = inputs.make(kind, M, N, seed=seed)
        return {"A": ops["A"], "scale": ops["scale"]}
    W = inputs.make_gauss_weights(M, N, seed=seed, outlier=25.0 if weights == "outlier" else 0.0)
    q, s, _ = oracle.quantize_q8(W) if kind == "q8" else oracle.quantize_q4(W)
    return {"A": q, "scale": s.view(np.float16)}   # the oracle returns binary16 bit patterns


@pytest.mark.parametrize("weights", _WEIGHTS)
@pytest.mark.parametrize("kind", ["q8", "q4"])
def test_nonzero_mean_activations(gpu, oracle_mod, kind, weights):
    for M, N in _SHAPES[kind]:
        wops = _operands(oracle_mod, kind, M, N, weights, seed=M + 3 * N)
        info = binding.describe_launch(kind, M, N)
        for dist in ("abs_normal", "shifted"):
            ops = dict(wops, x=inputs.make_x_f16(N, dist, seed=N + 17))
            label = f"{kind} {M}x{N} weights={weights} x={dist} plan={info}"
            say(f"[int-activations] {label}")
            y = run_gpu(kind, ops)
            ref = run_oracle(oracle_mod, kind, ops)
            rep = within_gate(oracle_mod, kind, ops, y, ref)
            bound = within_fp32_bound(kind, ops, y, ref)
            print(label, f"floored {rep['floored_rel']:.2e} fp32-bound ratio {bound:.3f}", flush=True)
            assert rep["ok"], (label, rep)
            assert bound <= 1.0, (label, bound)
