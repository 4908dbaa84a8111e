"""ctypes binding over the C ABI in ``include/gemv.h``,
``include/gemv_quant.h`` and ``include/gemv_softmax.h``.

Argument marshalling only: every step of the product runs in the HIP
library.  PyTorch supplies device memory and the current stream; no torch
operator is on the path.  If the library is missing the first call raises:
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemv_amd.so")

KIND = {"f32": 0, "f16": 1, "q8": 2, "q4": 3, "f16x32": 4, "f16_acc16": 5}
STATUS = {0: "GEMV_OK", 1: "GEMV_E_INVAL", 2: "GEMV_E_UNSUPPORTED", 3: "GEMV_E_LAUNCH", 4: "GEMV_E_DEVICE"}

_lock = threading.Lock()
_lib = None


class GemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class LaunchInfo(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("grid", ctypes.c_int), ("block", ctypes.c_int),
                ("rows_per_wave", ctypes.c_int), ("units_in_flight", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("stage_order", ctypes.c_int)]


class Plan(ctypes.Structure):
    """gemv_plan: an explicit launch plan (variant, waves, units_in_flight,
    rows_per_wave, stage_order, cap)."""
    _fields_ = [("variant", ctypes.c_int), ("waves", ctypes.c_int), ("units_in_flight", ctypes.c_int),
                ("rows_per_wave", ctypes.c_int), ("stage_order", ctypes.c_int), ("cap", ctypes.c_int)]


def load():
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m memory_bound_gemv_row_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        p, i = ctypes.c_void_p, ctypes.c_int
        for name in ("gemv_f32", "gemv_f16", "gemv_f16x32", "gemv_f16_acc16"):
            getattr(lib, name).argtypes = [p, p, p, i, i, p]
            getattr(lib, name).restype = i
        for name in ("gemv_q8", "gemv_q4"):
            getattr(lib, name).argtypes = [p, p, p, p, i, i, p]
            getattr(lib, name).restype = i
        for name in ("gemv_quantize_q8", "gemv_quantize_q4"):
            getattr(lib, name).argtypes = [p, p, p, p, i, i, p]
            getattr(lib, name).restype = i
        lib.gemv_softmax_f16.argtypes = [p, p, i, i, p]
        lib.gemv_softmax_f16.restype = i
        lib.gemv_status_string.argtypes = [i]
        lib.gemv_status_string.restype = ctypes.c_char_p
        lib.gemv_probe_read.argtypes = [p, ctypes.c_size_t, p, ctypes.c_uint32, p]
        lib.gemv_probe_read.restype = i
        lib.gemv_probe_copy.argtypes = [p, p, ctypes.c_size_t, p]
        lib.gemv_probe_copy.restype = i
        lib.gemv_describe_launch.argtypes = [i, i, i, i, ctypes.POINTER(LaunchInfo)]
        lib.gemv_describe_launch.restype = i
        lib.gemv_describe_launch_for.argtypes = [i, i, i, i, i, i, ctypes.POINTER(LaunchInfo)]
        lib.gemv_describe_launch_for.restype = i
        lib.gemv_check_plan_for.argtypes = [i, i, i, i, i, ctypes.POINTER(Plan), ctypes.POINTER(LaunchInfo)]
        lib.gemv_check_plan_for.restype = i
        lib.gemv_launch_plan.argtypes = [i, p, p, p, p, i, i, ctypes.POINTER(Plan), p]
        lib.gemv_launch_plan.restype = i
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().gemv_status_string(int(status)).decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise GemvError(rc, where)


# ---------------------------------------------------------------- raw pointers
# Device pointers as integers, stream as an integer handle (0 = null stream).
def gemv_f32_ptr(A: int, x: int, y: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_f32(A, x, y, M, N, stream)


def gemv_f16_ptr(A: int, x: int, y: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_f16(A, x, y, M, N, stream)


def gemv_f16x32_ptr(A: int, x: int, y: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_f16x32(A, x, y, M, N, stream)


def gemv_f16_acc16_ptr(A: int, x: int, y: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_f16_acc16(A, x, y, M, N, stream)


def gemv_q8_ptr(A: int, scale: int, x: int, y: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_q8(A, scale, x, y, M, N, stream)


def gemv_q4_ptr(A: int, scale: int, x: int, y: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_q4(A, scale, x, y, M, N, stream)


def quantize_q8_ptr(W: int, q: int, scale: int, row_sse: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_quantize_q8(W, q, scale, row_sse, M, N, stream)


def quantize_q4_ptr(W: int, q: int, scale: int, row_sse: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_quantize_q4(W, q, scale, row_sse, M, N, stream)


def softmax_f16_ptr(x: int, y: int, M: int, N: int, stream: int = 0) -> int:
    return load().gemv_softmax_f16(x, y, M, N, stream)


def probe_read_ptr(buf: int, nbytes: int, sink: int, guard: int = 0xA5A5A5A5, stream: int = 0) -> int:
    return load().gemv_probe_read(buf, nbytes, sink, guard, stream)


def probe_copy_ptr(src: int, dst: int, nbytes: int, stream: int = 0) -> int:
    return load().gemv_probe_copy(src, dst, nbytes, stream)


def describe_launch(kind: str, M: int, N: int, aligned: bool = True) -> dict:
    info = LaunchInfo()
    _check(load().gemv_describe_launch(KIND[kind], M, N, int(aligned), ctypes.byref(info)), "gemv_describe_launch")
    return {f: getattr(info, f) for f, _ in LaunchInfo._fields_}


def describe_launch_for(kind: str, M: int, N: int, cus: int, lds_max: int, aligned: bool = True) -> dict:
    """describe_launch for a device of `cus` CUs and `lds_max` bytes of LDS
    per workgroup; touches no device."""
    info = LaunchInfo()
    _check(load().gemv_describe_launch_for(KIND[kind], M, N, int(aligned), cus, lds_max, ctypes.byref(info)),
           "gemv_describe_launch_for")
    return {f: getattr(info, f) for f, _ in LaunchInfo._fields_}


# ---------------------------------------------------------------- torch tensors
def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name, dtypes, shape):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        # the C ABI launches on the current device's stream
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_INT_MAX = (1 << 31) - 1


def _dims(*dims):
    # the C ABI takes M and N as int: larger values would wrap in ctypes
    for d in dims:
        if not 0 <= d <= _INT_MAX:
            raise ValueError(f"dimension {d} outside the C ABI's int range [0, 2^31 - 1]")


def _out(out, M, device):
    import torch

    if out is None:
        return torch.empty(M, dtype=torch.float32, device=device)
    _need(out, "out", (torch.float32,), (M,))
    return out


def gemv_f32(A, x, out=None, stream=None):
    import torch

    M, N = A.shape
    _dims(M, N)
    a = _need(A, "A", (torch.float32,), (M, N))
    xp = _need(x, "x", (torch.float32,), (N,))
    y = _out(out, M, A.device)
    _check(gemv_f32_ptr(a, xp, y.data_ptr(), M, N, _stream(stream)), "gemv_f32")
    return y


def gemv_f16(A, x, out=None, stream=None):
    import torch

    h = (torch.float16, torch.int16, torch.uint16)
    M, N = A.shape
    _dims(M, N)
    a = _need(A, "A", h, (M, N))
    xp = _need(x, "x", h, (N,))
    y = _out(out, M, A.device)
    _check(gemv_f16_ptr(a, xp, y.data_ptr(), M, N, _stream(stream)), "gemv_f16")
    return y


def gemv_f16x32(A, x, out=None, stream=None):
    """A: binary16 [M, N], x: float32 [N]."""
    import torch

    h = (torch.float16, torch.int16, torch.uint16)
    M, N = A.shape
    _dims(M, N)
    a = _need(A, "A", h, (M, N))
    xp = _need(x, "x", (torch.float32,), (N,))
    y = _out(out, M, A.device)
    _check(gemv_f16x32_ptr(a, xp, y.data_ptr(), M, N, _stream(stream)), "gemv_f16x32")
    return y


def gemv_f16_acc16(A, x, out=None, stream=None):
    """LOSSY: binary16 running sums (see gemv_f16_acc16 in include/gemv.h).
    A: binary16 [M, N], x: binary16 [N]."""
    import torch

    h = (torch.float16, torch.int16, torch.uint16)
    M, N = A.shape
    _dims(M, N)
    a = _need(A, "A", h, (M, N))
    xp = _need(x, "x", h, (N,))
    y = _out(out, M, A.device)
    _check(gemv_f16_acc16_ptr(a, xp, y.data_ptr(), M, N, _stream(stream)), "gemv_f16_acc16")
    return y


def gemv_q8(A, scale, x, out=None, stream=None):
    import torch

    h = (torch.float16, torch.int16, torch.uint16)
    M, N = A.shape
    _dims(M, N)
    a = _need(A, "A", (torch.int8,), (M, N))
    s = _need(scale, "scale", h, (M,))
    xp = _need(x, "x", h, (N,))
    y = _out(out, M, A.device)
    _check(gemv_q8_ptr(a, s, xp, y.data_ptr(), M, N, _stream(stream)), "gemv_q8")
    return y


def gemv_q4(A, scale, x, out=None, stream=None):
    """A: uint8 [M, N/2] (two INT4 per byte, low nibble = even column),
    scale: binary16 [M, N/128], x: binary16 [N]."""
    import torch

    h = (torch.float16, torch.int16, torch.uint16)
    M, half = A.shape
    N = 2 * half
    _dims(M, N)
    a = _need(A, "A", (torch.uint8,), (M, half))
    if N % 128:
        raise ValueError("INT4 needs N % 128 == 0")
    s = _need(scale, "scale", h, (M, N // 128))
    xp = _need(x, "x", h, (N,))
    y = _out(out, M, A.device)
    _check(gemv_q4_ptr(a, s, xp, y.data_ptr(), M, N, _stream(stream)), "gemv_q4")
    return y


def quantize_q8(W, with_error=True, stream=None):
    """FP32 W [M, N] -> (q int8 [M, N], scale float16 [M], row_sse float32 [M]
    or None).  RMSE = sqrt(row_sse.sum() / (M * N))."""
    import torch

    M, N = W.shape
    _dims(M, N)
    w = _need(W, "W", (torch.float32,), (M, N))
    q = torch.empty((M, N), dtype=torch.int8, device=W.device)
    s = torch.empty(M, dtype=torch.float16, device=W.device)
    e = torch.empty(M, dtype=torch.float32, device=W.device) if with_error else None
    _check(quantize_q8_ptr(w, q.data_ptr(), s.data_ptr(), e.data_ptr() if e is not None else 0, M, N,
                           _stream(stream)), "gemv_quantize_q8")
    return q, s, e


def quantize_q4(W, with_error=True, stream=None):
    """FP32 W [M, N], N % 128 == 0 -> (q uint8 [M, N/2] two INT4 per byte,
    low nibble = even column; scale float16 [M, N/128]; row_sse float32 [M]
    or None)."""
    import torch

    M, N = W.shape
    _dims(M, N)
    if N % 128:
        raise ValueError("INT4 quantisation needs N % 128 == 0")
    w = _need(W, "W", (torch.float32,), (M, N))
    q = torch.empty((M, N // 2), dtype=torch.uint8, device=W.device)
    s = torch.empty((M, N // 128), dtype=torch.float16, device=W.device)
    e = torch.empty(M, dtype=torch.float32, device=W.device) if with_error else None
    _check(quantize_q4_ptr(w, q.data_ptr(), s.data_ptr(), e.data_ptr() if e is not None else 0, M, N,
                           _stream(stream)), "gemv_quantize_q4")
    return q, s, e


def softmax_f16(x, out=None, stream=None):
    """Row-wise softmax of binary16 x [M, N] -> binary16 [M, N]."""
    import torch

    h = (torch.float16, torch.int16, torch.uint16)
    M, N = x.shape
    _dims(M, N)
    xp = _need(x, "x", h, (M, N))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", h, (M, N))
    _check(softmax_f16_ptr(xp, out.data_ptr(), M, N, _stream(stream)), "gemv_softmax_f16")
    return out


def probe_read(buf, sink, guard: int = 0xA5A5A5A5, stream=None):
    _check(probe_read_ptr(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), guard,
                          _stream(stream)), "gemv_probe_read")


def probe_copy(src, dst, stream=None):
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _check(probe_copy_ptr(src.data_ptr(), dst.data_ptr(), n, _stream(stream)), "gemv_probe_copy")


def check_plan_for(kind: str, M: int, N: int, cus: int, lds_max: int, plan: tuple) -> dict | None:
    """The launch an explicit plan (variant, waves, units_in_flight,
    rows_per_wave, stage_order, cap) makes on a device of `cus` CUs and
    `lds_max` bytes of LDS per workgroup, or None where the library holds no
    kernel for it or it does not fit the shape; touches no device."""
    _dims(M, N)
    info = LaunchInfo()
    rc = load().gemv_check_plan_for(KIND[kind], M, N, cus, lds_max, ctypes.byref(Plan(*plan)), ctypes.byref(info))
    if rc == 2:
        return None
    _check(rc, "gemv_check_plan_for")
    return {f: getattr(info, f) for f, _ in LaunchInfo._fields_}


def launch_plan_ptr(kind: str, A: int, scale: int, x: int, y: int, M: int, N: int, plan: tuple,
                    stream: int = 0) -> int:
    """gemv_launch_plan on raw device pointers (scale 0 for FP formats)."""
    _dims(M, N)
    return load().gemv_launch_plan(KIND[kind], A, scale or None, x, y, M, N, ctypes.byref(Plan(*plan)), stream)
