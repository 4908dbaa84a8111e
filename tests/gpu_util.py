"""Helpers shared by the GPU tests: upload numpy operands, call the C ABI
through the binding, and compute the matching oracle result."""
import numpy as np
import torch

from memory_bound_gemv_row_amd import binding


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def run_gpu(kind: str, ops: dict) -> np.ndarray:
    """Call the HIP path on the operands ``ops`` (numpy) and return y (float32)."""
    A = dev(ops["A"])
    x = dev(ops["x"])
    if kind == "f32":
        y = binding.gemv_f32(A, x)
    elif kind == "f16":
        y = binding.gemv_f16(A, x)
    elif kind == "f16x32":
        y = binding.gemv_f16x32(A, x)
    elif kind == "f16_acc16":
        y = binding.gemv_f16_acc16(A, x)
    elif kind == "q8":
        y = binding.gemv_q8(A, dev(ops["scale"]), x)
    else:
        y = binding.gemv_q4(A, dev(ops["scale"]), x)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def run_oracle(oracle, kind: str, ops: dict) -> np.ndarray:
    if kind == "f32":
        return oracle.gemv_f32(ops["A"], ops["x"])
    if kind in ("f16", "f16_acc16"):
        # FP16 accumulation has the same exact result; only its gate differs
        return oracle.gemv_f16(ops["A"], ops["x"])
    if kind == "f16x32":
        return oracle.gemv_f16x32(ops["A"], ops["x"])
    if kind == "q8":
        return oracle.gemv_q8(ops["A"], ops["scale"], ops["x"])
    return oracle.gemv_q4(ops["A"], ops["scale"], ops["x"])


def abs_products(ops: dict, kind: str = "f16") -> np.ndarray:
    """sum_j |w_ij x_j| in float64, w the weights as the oracle reads them
    (INT8/INT4 dequantised with their scales)."""
    x = np.abs(np.asarray(ops["x"]).astype(np.float64))
    if kind == "q8":
        W = np.abs(ops["A"].astype(np.float64)) * ops["scale"].astype(np.float64)[:, None]
    elif kind == "q4":
        from qpack import unpack_int4

        W = np.abs(unpack_int4(ops["A"]).astype(np.float64)) * np.repeat(
            ops["scale"].astype(np.float64), 128, axis=1)
    else:
        W = np.abs(np.asarray(ops["A"]).astype(np.float64))
    return W @ x


def within_fp32_bound(kind: str, ops: dict, y: np.ndarray, ref: np.ndarray) -> float:
    """max_i |y_i - r_i| / (g(2N + 8) sum_j |w_ij x_j|), g(n) = n u / (1 - n u),
    u = 2^-24: the recursive-summation bound of an FP32 dot product of N exact
    products in any order, with room for v_dot2_f32_f16's two roundings per
    step and the scale multiplications.  At most 1 for a correct FP32-
    accumulating kernel, whatever the cancellation (unlike a relative error
    when M is too small for the floor to act)."""
    N = np.asarray(ops["x"]).shape[0]
    n = 2 * N + 8
    g = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    bound = g * abs_products(ops, kind) + 1e-300
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    return float(np.max(np.abs(y - ref) / bound)) if y.size else 0.0


def within_gate(oracle, kind: str, ops: dict, y: np.ndarray, ref: np.ndarray) -> dict:
    """Parity report plus the gate verdict: floored relative error for the
    FP32-accumulating paths, the derived componentwise bound for FP16
    accumulation."""
    from oracle.metrics import GATES, acc16_ratio, parity_report

    rep = parity_report(y, ref)
    if kind == "f16_acc16":
        N = np.asarray(ops["A"]).shape[1]
        rep["acc16_ratio"] = acc16_ratio(y, ref, abs_products(ops, kind), N)
        rep["ok"] = rep["acc16_ratio"] <= 1.0
    else:
        rep["ok"] = rep["floored_rel"] <= GATES[kind]
    return rep


def say(msg: str):
    """Name the case before a GPU step, so that a fault leaves a trace."""
    print(msg, flush=True)
