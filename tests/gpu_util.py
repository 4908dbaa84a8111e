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


def abs_products(ops: dict) -> np.ndarray:
    """sum_j |A_ij x_j| in float64 (the scale of the FP16-accumulation bound)."""
    A = np.abs(np.asarray(ops["A"]).astype(np.float64))
    return A @ np.abs(np.asarray(ops["x"]).astype(np.float64))


def within_gate(oracle, kind: str, ops: dict, y: np.ndarray, ref: np.ndarray) -> dict:
    """Parity report plus the gate verdict: floored relative error for the
    FP32-accumulating paths, the derived componentwise bound for FP16
    accumulation."""
    from oracle.metrics import GATES, acc16_ratio, parity_report

    rep = parity_report(y, ref)
    if kind == "f16_acc16":
        N = np.asarray(ops["A"]).shape[1]
        rep["acc16_ratio"] = acc16_ratio(y, ref, abs_products(ops), N)
        rep["ok"] = rep["acc16_ratio"] <= 1.0
    else:
        rep["ok"] = rep["floored_rel"] <= GATES[kind]
    return rep


def say(msg: str):
    """Name the case before a GPU step, so that a fault leaves a trace."""
    print(msg, flush=True)
