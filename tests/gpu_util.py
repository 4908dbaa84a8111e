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
    elif kind == "q8":
        y = binding.gemv_q8(A, dev(ops["scale"]), x)
    else:
        y = binding.gemv_q4(A, dev(ops["scale"]), x)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def run_oracle(oracle, kind: str, ops: dict) -> np.ndarray:
    if kind == "f32":
        return oracle.gemv_f32(ops["A"], ops["x"])
    if kind == "f16":
        return oracle.gemv_f16(ops["A"], ops["x"])
    if kind == "f16x32":
        return oracle.gemv_f16x32(ops["A"], ops["x"])
    if kind == "q8":
        return oracle.gemv_q8(ops["A"], ops["scale"], ops["x"])
    return oracle.gemv_q4(ops["A"], ops["scale"], ops["x"])


def say(msg: str):
    """Name the case before a GPU step, so that a fault leaves a trace."""
    print(msg, flush=True)
