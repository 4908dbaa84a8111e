"""ctypes wrapper over the C oracle (``gemv_oracle.c``, ``quant_oracle.c``,
``softmax_oracle.c``).

Test infrastructure only: the product path never imports this module.

Every function takes numpy arrays, checks dtypes and shapes, and returns the
oracle's result.  The arithmetic lives entirely in the C files: the GEMV
follows the plain definition y_i = sum_j A_ij x_j ("Making GEMV Fast",
section "Algorithm") with the INT8/INT4 reference weights taken as exactly
q*s, and the quantiser makes those operands from FP32 weights ("membound",
section "The kernel decode actually runs: dequant GEMV").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, f) for f in ("gemv_oracle.c", "quant_oracle.c", "softmax_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if not force and not _stale():
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
        *_SRCS, "-o", tmp, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _stale() -> bool:
    return not os.path.exists(_LIB) or any(os.path.getmtime(p) > os.path.getmtime(_LIB) for p in _SRCS)


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _stale():
            build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_half_to_double_array.argtypes = [p, p, i64]
        lib.oracle_half_to_double_array.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        lib.oracle_gemv_f32.argtypes = [p, p, p, i64, i64]
        lib.oracle_gemv_f16.argtypes = [p, p, p, i64, i64]
        lib.oracle_gemv_f16x32.argtypes = [p, p, p, i64, i64]
        lib.oracle_gemv_q8.argtypes = [p, p, p, p, i64, i64]
        lib.oracle_gemv_q4.argtypes = [p, p, p, p, i64, i64]
        for f in (lib.oracle_gemv_f32, lib.oracle_gemv_f16, lib.oracle_gemv_f16x32, lib.oracle_gemv_q8,
                  lib.oracle_gemv_q4):
            f.restype = ctypes.c_int
        lib.oracle_double_to_half.argtypes = [ctypes.c_double]
        lib.oracle_double_to_half.restype = ctypes.c_uint16
        for f in (lib.oracle_quantize_q8, lib.oracle_quantize_q4):
            f.argtypes = [p, p, p, p, i64, i64]
            f.restype = ctypes.c_int
        lib.oracle_softmax_f16.argtypes = [p, p, i64, i64]
        lib.oracle_softmax_f16.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _as(a, dtype, name):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"{name}: expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for later oracle calls (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def half_to_double(bits: int) -> float:
    return float(_load().oracle_half_to_double(int(bits) & 0xFFFF))


def half_to_double_array(bits: np.ndarray) -> np.ndarray:
    h = _as(bits, np.uint16, "bits").ravel()
    out = np.empty(h.size, dtype=np.float64)
    _load().oracle_half_to_double_array(_ptr(h), _ptr(out), h.size)
    return out


def _f16_bits(a, name):
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return _as(a, np.uint16, name)


def gemv_f32(A: np.ndarray, x: np.ndarray) -> np.ndarray:
    A = _as(A, np.float32, "A")
    x = _as(x, np.float32, "x")
    M, N = A.shape
    if x.shape != (N,):
        raise ValueError("x must have shape (N,)")
    y = np.empty(M, dtype=np.float64)
    rc = _load().oracle_gemv_f32(_ptr(A), _ptr(x), _ptr(y), M, N)
    if rc != 0:
        raise ValueError("oracle_gemv_f32 rejected its arguments")
    return y


def gemv_f16(A: np.ndarray, x: np.ndarray) -> np.ndarray:
    A = _f16_bits(A, "A")
    x = _f16_bits(x, "x")
    M, N = A.shape
    if x.shape != (N,):
        raise ValueError("x must have shape (N,)")
    y = np.empty(M, dtype=np.float64)
    rc = _load().oracle_gemv_f16(_ptr(A), _ptr(x), _ptr(y), M, N)
    if rc != 0:
        raise ValueError("oracle_gemv_f16 rejected its arguments")
    return y


def gemv_f16x32(A: np.ndarray, x: np.ndarray) -> np.ndarray:
    """FP16 A (binary16) with FP32 x."""
    A = _f16_bits(A, "A")
    x = _as(x, np.float32, "x")
    M, N = A.shape
    if x.shape != (N,):
        raise ValueError("x must have shape (N,)")
    y = np.empty(M, dtype=np.float64)
    rc = _load().oracle_gemv_f16x32(_ptr(A), _ptr(x), _ptr(y), M, N)
    if rc != 0:
        raise ValueError("oracle_gemv_f16x32 rejected its arguments")
    return y


def gemv_q8(A: np.ndarray, scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    A = _as(A, np.int8, "A")
    s = _f16_bits(scale, "scale")
    x = _f16_bits(x, "x")
    M, N = A.shape
    if x.shape != (N,) or s.shape != (M,):
        raise ValueError("shapes: A (M,N), scale (M,), x (N,)")
    y = np.empty(M, dtype=np.float64)
    rc = _load().oracle_gemv_q8(_ptr(A), _ptr(s), _ptr(x), _ptr(y), M, N)
    if rc != 0:
        raise ValueError("oracle_gemv_q8 rejected its arguments")
    return y


def gemv_q4(A: np.ndarray, scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    """A: uint8 [M, N/2] packed nibbles; scale: binary16 [M, N/128]; x: binary16 [N]."""
    A = _as(A, np.uint8, "A")
    s = _f16_bits(scale, "scale")
    x = _f16_bits(x, "x")
    M, half_n = A.shape
    N = 2 * half_n
    if x.shape != (N,) or N % 128 != 0 or s.shape != (M, N // 128):
        raise ValueError("shapes: A (M,N/2), scale (M,N/128), x (N,), N % 128 == 0")
    y = np.empty(M, dtype=np.float64)
    rc = _load().oracle_gemv_q4(_ptr(A), _ptr(s), _ptr(x), _ptr(y), M, N)
    if rc != 0:
        raise ValueError("oracle_gemv_q4 rejected its arguments")
    return y


# ---------------------------------------------------------------- quantiser
def double_to_half(v: float) -> int:
    """binary16 bit pattern of v, round to nearest, ties to even."""
    return int(_load().oracle_double_to_half(float(v)))


def quantize_q8(W: np.ndarray):
    """FP32 W [M, N] -> (q int8 [M, N], scale binary16 bits uint16 [M],
    row_sse float64 [M])."""
    W = _as(W, np.float32, "W")
    M, N = W.shape
    q = np.empty((M, N), dtype=np.int8)
    s = np.empty(M, dtype=np.uint16)
    e = np.empty(M, dtype=np.float64)
    if _load().oracle_quantize_q8(_ptr(W), _ptr(q), _ptr(s), _ptr(e), M, N) != 0:
        raise ValueError("oracle_quantize_q8 rejected its arguments")
    return q, s, e


def quantize_q4(W: np.ndarray):
    """FP32 W [M, N], N % 128 == 0 -> (packed uint8 [M, N/2], scale binary16
    bits uint16 [M, N/128], row_sse float64 [M])."""
    W = _as(W, np.float32, "W")
    M, N = W.shape
    if N % 128:
        raise ValueError("INT4 quantisation needs N % 128 == 0")
    q = np.zeros((M, N // 2), dtype=np.uint8)
    s = np.empty((M, N // 128), dtype=np.uint16)
    e = np.empty(M, dtype=np.float64)
    if _load().oracle_quantize_q4(_ptr(W), _ptr(q), _ptr(s), _ptr(e), M, N) != 0:
        raise ValueError("oracle_quantize_q4 rejected its arguments")
    return q, s, e


def quant_rmse(row_sse: np.ndarray, M: int, N: int) -> float:
    """sqrt(sum of squared quantisation errors / number of weights)."""
    return float(np.sqrt(np.sum(np.asarray(row_sse, dtype=np.float64)) / (M * N))) if M * N else 0.0


# ---------------------------------------------------------------- softmax
def softmax_f16(x: np.ndarray) -> np.ndarray:
    """Row-wise softmax of binary16 x [M, N], in float64 (not rounded)."""
    x = _f16_bits(x, "x")
    M, N = x.shape
    y = np.empty((M, N), dtype=np.float64)
    if _load().oracle_softmax_f16(_ptr(x), _ptr(y), M, N) != 0:
        raise ValueError("oracle_softmax_f16 rejected its arguments")
    return y
